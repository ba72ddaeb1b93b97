"""GPU parity of packed variable-length sequences (ssd_fwd with cu_seqlens,
through the C ABI) against the fp64 per-sequence oracle.

Sequences packed on one token axis (page "Mamba-2 SSD for Ascend NPU",
"Limitations and roadmap": varlen / cu_seqlens; page "ops-transformer
MambaV2 算子套件" §1.4).  Same bar as the dense path: max|gpu - oracle| <=
tol * max|oracle| for out and for final_state, tol = 2e-3 on the fp16-operand
MFMA path and 1e-4 on the fp32 path.
"""
import sys

import numpy as np
import pytest
import torch

from oracle import ssd_varlen
from workloads import WORKLOADS, make_inputs, packed_inputs

pytestmark = pytest.mark.gpu

TOL = {"f16": 2e-3, "f32": 1e-4}


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def rel_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    assert got.shape == ref.shape and np.isfinite(got).all()
    scale = float(np.abs(ref).max())
    return float(np.abs(got - ref).max()) / (scale if scale > 0 else 1.0)


def run_both(ssd, d, chunk, mma="f16", cpw=0, out_dtype=None, max_seqlen=None):
    g = {k: (None if v is None else v.cuda()) for k, v in d.items()}
    out, fin = ssd.ssd_fwd(g["x"], g["dt"], g["A"], g["B"], g["C"], chunk, D=g["D"], z=g["z"],
                           dt_bias=g.get("dt_bias"), initial_states=g["initial_states"],
                           dt_softplus=True, return_final_state=True, mma=mma,
                           out_dtype=out_dtype, chunks_per_wg=cpw, cu_seqlens=g["cu_seqlens"],
                           max_seqlen=max_seqlen)
    torch.cuda.synchronize()
    ref_o, ref_f = ssd_varlen(d["x"], d["dt"], d["A"], d["B"], d["C"], d["cu_seqlens"], D=d["D"],
                              z=d["z"], dt_bias=d.get("dt_bias"),
                              initial_states=d["initial_states"], dt_softplus=True)
    return out[0].float().cpu().numpy(), fin.cpu().numpy(), ref_o, ref_f


# (lengths, chunk, N, G, chunks_per_wg): empty and one-token sequences, ragged
# tails, sequences with one chunk group and with several (folded into the main
# pass, or chained by the passing pass when more than nine)
CASES = [
    ((1, 64, 65, 200, 0, 129, 7), 64, 64, 2, 0),
    ((300, 1, 0, 513, 256), 128, 128, 1, 0),
    ((300, 1, 0, 513, 256), 128, 128, 1, 1),
    ((1000, 17, 640, 3), 64, 128, 4, 1),           # up to 16 groups: passing pass
    ((700, 0, 0, 255, 256, 257), 256, 128, 2, 1),
    ((64,) * 9 + (33,), 64, 64, 4, 0),
]


@pytest.mark.parametrize("mma", ["f16", "f32"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: f"L{len(c[0])}q{c[1]}n{c[2]}g{c[3]}c{c[4]}")
def test_packed_matches_oracle(gpu_lib, case, mma):
    lens, Q, N, G, cpw = case
    _say(f"  varlen lens={lens} Q={Q} N={N} G={G} cpw={cpw} mma={mma}")
    d = packed_inputs(lens, 4, 64, N, G, seed=sum(lens) + Q + N, has_D=True, has_z=True,
                      has_h0=True, dt_bias=True)
    o, f, ro, rf = run_both(gpu_lib, d, Q, mma=mma, cpw=cpw)
    eo, ef = rel_err(o, ro), rel_err(f, rf)
    _say(f"    out {eo:.3e} final {ef:.3e}")
    assert eo <= TOL[mma] and ef <= TOL[mma]


def test_packed_bf16_io_and_out(gpu_lib):
    d = packed_inputs((129, 0, 300, 5), 8, 64, 128, 2, seed=91, has_D=True, has_z=True,
                      has_h0=True, io_dtype="bf16")
    o, f, ro, rf = run_both(gpu_lib, d, 128, out_dtype=torch.bfloat16)
    # bf16 output adds its own rounding (2^-9 relative) to the fp16 path's bound
    assert rel_err(o, ro) <= TOL["f16"] + 2 ** -8 and rel_err(f, rf) <= TOL["f16"]


def test_empty_sequences_pass_the_initial_state(gpu_lib):
    d = packed_inputs((0, 40, 0, 0, 3), 4, 64, 64, 1, seed=92, has_h0=True)
    o, f, ro, rf = run_both(gpu_lib, d, 64)
    h0 = d["initial_states"].numpy()
    for s in (0, 2, 3):
        np.testing.assert_array_equal(f[s], h0[s])      # copied, not recomputed
    assert rel_err(o, ro) <= TOL["f16"] and rel_err(f, rf) <= TOL["f16"]


def test_packed_equals_dense_rows(gpu_lib):
    """Equal-length sequences packed give bit-identical results to the same
    data as dense batch rows (same plan, same kernels)."""
    lens = (256, 256, 256)
    d = packed_inputs(lens, 4, 64, 128, 2, seed=93, has_D=True, has_h0=True)
    g = {k: (None if v is None else v.cuda()) for k, v in d.items()}
    o_p, f_p = gpu_lib.ssd_fwd(g["x"], g["dt"], g["A"], g["B"], g["C"], 128, D=g["D"],
                               initial_states=g["initial_states"], dt_softplus=True,
                               return_final_state=True, cu_seqlens=g["cu_seqlens"])
    r = lambda t, *s: t.reshape(len(lens), lens[0], *s).contiguous()
    o_d, f_d = gpu_lib.ssd_fwd(r(g["x"], 4, 64), r(g["dt"], 4), g["A"], r(g["B"], 2, 128),
                               r(g["C"], 2, 128), 128, D=g["D"], initial_states=g["initial_states"],
                               dt_softplus=True, return_final_state=True)
    torch.cuda.synchronize()
    assert torch.equal(o_p.reshape(o_d.shape), o_d) and torch.equal(f_p, f_d)


def test_sequence_longer_than_max_seqlen_is_reported(gpu_lib):
    """A sequence longer than the max_seqlen the caller gave: the kernels set
    the call's device error flag and check() raises; the sequences that keep
    the contract are still right."""
    d = packed_inputs((50, 90), 4, 64, 64, 1, seed=94)
    g = {k: (None if v is None else v.cuda()) for k, v in d.items()}
    call, out, fin, _ = gpu_lib.prepare(g["x"], g["dt"], g["A"], g["B"], g["C"], 64,
                                        dt_softplus=True, return_final_state=True,
                                        cu_seqlens=g["cu_seqlens"], max_seqlen=60)
    call.launch(torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    with pytest.raises(ValueError, match="cu_seqlens"):
        call.check()
    call.check()                  # the flag was cleared with the report
    ro, rf = ssd_varlen(d["x"][:, :50], d["dt"][:, :50], d["A"], d["B"][:, :50], d["C"][:, :50],
                        [0, 50], dt_softplus=True)
    assert rel_err(out[0, :50].cpu().numpy(), ro) <= TOL["f16"]
    assert rel_err(fin[:1].cpu().numpy(), rf) <= TOL["f16"]
    # the convenience call checks by default when max_seqlen is given
    with pytest.raises(ValueError, match="cu_seqlens"):
        gpu_lib.ssd_fwd(g["x"], g["dt"], g["A"], g["B"], g["C"], 64, dt_softplus=True,
                        cu_seqlens=g["cu_seqlens"], max_seqlen=60)
    # and a max_seqlen that holds raises nothing
    gpu_lib.ssd_fwd(g["x"], g["dt"], g["A"], g["B"], g["C"], 64, dt_softplus=True,
                    cu_seqlens=g["cu_seqlens"], max_seqlen=90)


def test_malformed_offsets_are_clamped_and_reported(gpu_lib):
    """Offsets past the packed token count or decreasing: the kernels clamp
    every sequence to [0, T] (nothing outside x, B, C or out is addressed)
    and report the call; host-read offsets are refused before any launch."""
    d = packed_inputs((40, 30, 30), 4, 64, 64, 1, seed=95)
    g = {k: (None if v is None else v.cuda()) for k, v in d.items()}
    for bad in ([0, 40, 30, 100], [0, 40, 70, 130]):
        cu = torch.tensor(bad, dtype=torch.int32, device="cuda")
        call, out, fin, _ = gpu_lib.prepare(g["x"], g["dt"], g["A"], g["B"], g["C"], 64,
                                            dt_softplus=True, return_final_state=True,
                                            cu_seqlens=cu, max_seqlen=64)
        call.launch(torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        with pytest.raises(ValueError, match="cu_seqlens"):
            call.check()
        with pytest.raises(ValueError, match="cu_seqlens"):
            gpu_lib.prepare(g["x"], g["dt"], g["A"], g["B"], g["C"], 64, cu_seqlens=cu)


def test_varlen_workload_full_size(gpu_lib):
    """The packed workload at its full size, in the launch the benchmark times."""
    w = WORKLOADS["varlen"]
    d = make_inputs(w)
    _say(f"  varlen workload {w.shape_str()} {w.nseq} sequences")
    o, f, ro, rf = run_both(gpu_lib, d, w.chunk, max_seqlen=w.max_len)
    eo, ef = rel_err(o, ro), rel_err(f, rf)
    _say(f"    out {eo:.3e} final {ef:.3e}")
    assert eo <= TOL["f16"] and ef <= TOL["f16"]
