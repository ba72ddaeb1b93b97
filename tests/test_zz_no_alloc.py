"""ssd_fwd_noalloc (the entry point for callers that cannot allocate) against
ssd_fwd, through the C ABI: two calls in a row on one GPU, the second with a
smaller input, each equal bit for bit to ssd_fwd with its own workspace (the
same kernels and plan) and within the fp16 path's bound of the fp64 oracle.
"""
import sys

import numpy as np
import pytest
import torch

from oracle import ssd_recurrence
from workloads import random_inputs

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


# (B, L, H, N, G, chunk, chunks_per_wg): both plans cut the sequences into
# several chunk groups, so the static scratch holds group states; the first
# folds them in the main pass, the second (more groups) chains them first
CALLS = [(2, 1500, 8, 128, 2, 128, 2), (1, 700, 4, 64, 1, 64, 1)]


def test_noalloc_matches_ssd_fwd_on_two_calls(gpu_lib):
    st = torch.cuda.current_stream().cuda_stream
    for k, (Bsz, L, H, N, G, Q, cpw) in enumerate(CALLS):
        _say(f"[case] noalloc call {k}: [{Bsz},{L},{H},64,{N},{Q},{G}] chunks_per_wg={cpw}")
        d = random_inputs(Bsz, L, H, 64, N, G, seed=1200 + k, has_D=True, has_z=True,
                          has_h0=True, dt_bias=True)
        g = {n: (None if v is None else v.cuda()) for n, v in d.items()}
        call, out, fin, ws = gpu_lib.prepare(g["x"], g["dt"], g["A"], g["B"], g["C"], Q, D=g["D"],
                                             z=g["z"], dt_bias=g["dt_bias"],
                                             initial_states=g["initial_states"], dt_softplus=True,
                                             return_final_state=True, chunks_per_wg=cpw)
        assert ws is not None and ws.numel() <= gpu_lib.NOALLOC_MAX_SCRATCH
        call.launch(st)
        torch.cuda.synchronize()
        ref_out, ref_fin = out.clone(), fin.clone()
        out.fill_(float("nan"))
        fin.fill_(float("nan"))
        ws.fill_(255)           # the caller's workspace is not what the variant reads
        call.launch_noalloc(st)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), f"call {k}: out differs from ssd_fwd"
        assert torch.equal(fin, ref_fin), f"call {k}: final_state differs from ssd_fwd"
        ro, rf = ssd_recurrence(d["x"], d["dt"], d["A"], d["B"], d["C"], D=d["D"], z=d["z"],
                                dt_bias=d["dt_bias"], initial_states=d["initial_states"],
                                dt_softplus=True)
        for got, ref, what in ((out, ro, "out"), (fin, rf, "final_state")):
            e = float(np.abs(got.double().cpu().numpy() - ref).max() / np.abs(ref).max())
            _say(f"    {what}: max_err/max_ref={e:.3e}")
            assert e <= 2e-3


def test_noalloc_refuses_a_plan_beyond_its_scratch(gpu_lib):
    d = random_inputs(1, 64, 2, 64, 64, 1, seed=1210)
    g = {n: (None if v is None else v.cuda()) for n, v in d.items()}
    call, out, fin, ws = gpu_lib.prepare(g["x"], g["dt"], g["A"], g["B"], g["C"], 64,
                                         dt_softplus=True, noalloc=True)
    assert ws is None
    call.launch(torch.cuda.current_stream().cuda_stream)       # one group: no scratch needed
    torch.cuda.synchronize()
    big = gpu_lib.make_desc(1, 100000, 8, 64, 128, 1)
    big.chunks_per_wg = 1
    assert gpu_lib.workspace_size(big, 64) > gpu_lib.NOALLOC_MAX_SCRATCH
    rc = gpu_lib.load_library().ssd_fwd_noalloc(16, 16, 16, 16, 16, None, 64, 1, 0, 16, None,
                                                None, __import__("ctypes").byref(big))
    assert rc == gpu_lib.SSD_ERR_WORKSPACE
