"""GPU parity of the SSD backward (ssd_bwd through the C ABI) against the fp64
autograd oracle.

Scope of the backward: P = N = chunk = 64, fp32, with the optional z gate
(page "Mamba-2 SSD for Ascend NPU", "AscendC training" and "Limitations and
roadmap").  Bar per
gradient tensor: max|gpu - oracle| <= 1e-4 * max|oracle|, the all-fp32 bound
of the forward check path; every product and the carried state gradient are
fp32 with fp32 accumulation, and the exponentials use the hardware exp2.
"""
import math
import sys

import numpy as np
import pytest
import torch

from oracle import ssd_grads
from workloads import WORKLOADS, make_inputs, random_inputs

pytestmark = pytest.mark.gpu

TOL = 1e-4
NAMES = ("dx", "ddt", "dA", "dB", "dC", "dD", "dz", "ddt_bias", "dinitial_states")


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def rel_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    assert got.shape == ref.shape and np.isfinite(got).all()
    scale = float(np.abs(ref).max())
    return float(np.abs(got - ref).max()) / (scale if scale > 0 else 1.0)


def grads_both(ssd, d, dout, dfin, softplus=True, limit=(0.0, math.inf)):
    g = {k: (None if v is None else v.cuda()) for k, v in d.items()}
    got = ssd.ssd_bwd(g["x"], g["dt"], g["A"], g["B"], g["C"], dout.cuda(), 64, D=g["D"],
                      z=g.get("z"), dt_bias=g.get("dt_bias"), initial_states=g["initial_states"],
                      dfinal_state=None if dfin is None else dfin.cuda(), dt_softplus=softplus,
                      dt_limit=limit)
    torch.cuda.synchronize()
    ref = ssd_grads(d["x"], d["dt"], d["A"], d["B"], d["C"], dout, D=d["D"], z=d.get("z"),
                    dt_bias=d.get("dt_bias"), initial_states=d["initial_states"],
                    dfinal_state=dfin, dt_softplus=softplus, dt_limit=limit)
    return got, ref


def compare(got, ref):
    for k in NAMES:
        if ref.get(k) is None:
            assert got.get(k) is None
            continue
        e = rel_err(got[k].cpu().numpy(), ref[k])
        _say(f"    {k}: max_err/max_ref={e:.3e}")
        assert e <= TOL, f"{k}: {e:.3e} > {TOL}"


def _dout(shape_x, shape_s, seed, fin=True):
    g = torch.Generator().manual_seed(seed)
    dout = torch.randn(*shape_x, generator=g)
    dfin = torch.randn(*shape_s, generator=g) if fin else None
    return dout, dfin


# (B, L, H, G): one chunk, ragged tails, several chunks, grouped heads
SHAPES = [(1, 64, 1, 1), (2, 100, 2, 1), (1, 257, 4, 2), (2, 130, 4, 4), (1, 33, 2, 2)]


@pytest.mark.parametrize("opts", [True, False], ids=["all_options", "bare"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_backward_matches_oracle(gpu_lib, shape, opts):
    Bsz, L, H, G = shape
    _say(f"  bwd B={Bsz} L={L} H={H} G={G} options={opts}")
    d = random_inputs(Bsz, L, H, 64, 64, G, seed=Bsz * 100 + L + H, has_D=opts, has_z=opts,
                      has_h0=opts, dt_bias=opts)
    dout, dfin = _dout((Bsz, L, H, 64), (Bsz, H, 64, 64), seed=L, fin=opts)
    got, ref = grads_both(gpu_lib, d, dout, dfin)
    compare(got, ref)


def test_backward_clamp_and_no_softplus(gpu_lib):
    d = random_inputs(1, 150, 2, 64, 64, 1, seed=77, has_D=True, has_h0=True, dt_bias=True)
    dout, dfin = _dout((1, 150, 2, 64), (1, 2, 64, 64), seed=78)
    got, ref = grads_both(gpu_lib, d, dout, dfin, softplus=False, limit=(0.2, 0.7))
    compare(got, ref)
    clamped = ~((d["dt"] + d["dt_bias"]) >= 0.2) | ~((d["dt"] + d["dt_bias"]) <= 0.7)
    assert bool(clamped.any())
    assert torch.all(got["ddt"].cpu()[clamped] == 0)


def test_backward_deterministic(gpu_lib):
    d = random_inputs(2, 200, 4, 64, 64, 2, seed=79, has_D=True, has_h0=True, dt_bias=True)
    dout, dfin = _dout((2, 200, 4, 64), (2, 4, 64, 64), seed=80)
    g = {k: (None if v is None else v.cuda()) for k, v in d.items()}
    call = gpu_lib.prepare_bwd(g["x"], g["dt"], g["A"], g["B"], g["C"], dout.cuda(), 64,
                               D=g["D"], dt_bias=g["dt_bias"], initial_states=g["initial_states"],
                               dfinal_state=dfin.cuda(), dt_softplus=True)
    st = torch.cuda.current_stream().cuda_stream
    call.launch(st)
    torch.cuda.synchronize()
    first = {k: v.clone() for k, v in call.grads.items() if v is not None}
    call.launch(st)
    torch.cuda.synchronize()
    for k, v in first.items():
        assert torch.equal(v, call.grads[k]), k


def test_backward_full_size_sampled(gpu_lib):
    """The training-shape workload [8,4096,256,64,64,64,64] (P = N = chunk =
    64) at full size, in the launch the benchmark times; the oracle checks one
    batch row and the four heads of one group (dA, dD and ddt_bias sum over
    the whole batch and are checked on the small shapes above)."""
    ssd = gpu_lib
    w = WORKLOADS["h256"]
    d = make_inputs(w)
    _say(f"  bwd full size {w.shape_str()}")
    g = torch.Generator().manual_seed(81)
    dout = torch.randn(w.batch, w.seqlen, w.nheads, 64, generator=g)
    dfin = torch.randn(w.batch, w.nheads, 64, 64, generator=g)
    gd = {k: (None if v is None else v.cuda()) for k, v in d.items()}
    got = ssd.ssd_bwd(gd["x"], gd["dt"], gd["A"], gd["B"], gd["C"], dout.cuda(), 64,
                      initial_states=gd["initial_states"], dfinal_state=dfin.cuda(),
                      dt_softplus=True)
    torch.cuda.synchronize()
    b, grp = 5, 17
    hs = slice(grp * 4, grp * 4 + 4)
    ref = ssd_grads(d["x"][b:b + 1, :, hs], d["dt"][b:b + 1, :, hs], d["A"][hs],
                    d["B"][b:b + 1, :, grp:grp + 1], d["C"][b:b + 1, :, grp:grp + 1],
                    dout[b:b + 1, :, hs], dfinal_state=dfin[b:b + 1, hs], dt_softplus=True)
    sel = {"dx": got["dx"][b:b + 1, :, hs], "ddt": got["ddt"][b:b + 1, :, hs],
           "dB": got["dB"][b:b + 1, :, grp:grp + 1], "dC": got["dC"][b:b + 1, :, grp:grp + 1]}
    for k, v in sel.items():
        e = rel_err(v.cpu().numpy(), ref[k])
        _say(f"    {k}: max_err/max_ref={e:.3e}")
        assert e <= TOL, f"{k}: {e:.3e} > {TOL}"
