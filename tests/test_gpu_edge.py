"""GPU parity of the forward's edge cases and degenerate decays, through the
C ABI, against the fp64 oracle (and, where the method reduces to one, a
closed form computed here from its definition).

Cases (page "Mamba-2 SSD for Ascend NPU", "Implementation": dt_softplus,
dt_bias and dt_limit are options of the forward):
  * strong decay: |delta*A| large enough that the main pass drops its
    factored intra-chunk decay and takes one exponential per element;
  * A = -1e4: exp(delta*A) underflows to zero, so
    y_t = delta_t (C_t . B_t) x_t + D x_t and final = delta_{L-1} x_{L-1} (outer) B_{L-1};
  * A = 0: no decay, the state is a running sum (causal linear attention);
  * dt_softplus off, with and without a dt_limit;
  * dt_bias in [-11, -5]: softplus of a very negative argument (steps of
    1e-5 .. 7e-3, the range a Mamba-2 dt_bias set up for small steps gives);
  * the headline workload [4,2048,16,64,128,128,4] on the all-fp32 check path.

Bar: max|gpu - ref| <= tol * max|ref| per output, tol = 2e-3 on the
fp16-operand MFMA path and 1e-4 on the all-fp32 check path.
"""
import math
import sys

import numpy as np
import pytest
import torch

from oracle import discretize, ssd_linear_attention_closed_form, ssd_recurrence
from workloads import WORKLOADS, make_inputs, random_inputs

pytestmark = pytest.mark.gpu

TOL = {"f16": 2e-3, "f32": 1e-4}
LOG2E = 1.4426950408889634


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def rel_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), "non-finite values"
    scale = float(np.abs(ref).max())
    return float(np.abs(got - ref).max()) / (scale if scale > 0 else 1.0)


def check(got, ref, tol, what):
    e = rel_err(got, ref)
    _say(f"    {what}: max_err/max_ref={e:.3e} (tol {tol:g})")
    assert e <= tol, f"{what}: {e:.3e} > {tol:g}"


def run_gpu(ssd, d, chunk, mma, softplus=True, limit=(0.0, math.inf), cpw=0):
    g = {k: (None if v is None else v.cuda()) for k, v in d.items()}
    out, fin = ssd.ssd_fwd(g["x"], g["dt"], g["A"], g["B"], g["C"], chunk, D=g.get("D"),
                           z=g.get("z"), dt_bias=g.get("dt_bias"),
                           initial_states=g.get("initial_states"), dt_softplus=softplus,
                           dt_limit=limit, return_final_state=True, mma=mma, chunks_per_wg=cpw)
    torch.cuda.synchronize()
    return out.double().cpu().numpy(), fin.double().cpu().numpy()


def run_oracle(d, softplus=True, limit=(0.0, math.inf)):
    return ssd_recurrence(d["x"], d["dt"], d["A"], d["B"], d["C"], D=d.get("D"), z=d.get("z"),
                          dt_bias=d.get("dt_bias"), initial_states=d.get("initial_states"),
                          dt_softplus=softplus, dt_limit=limit)


def decay_log2(d, chunk, softplus=True):
    """|delta*A| in log2 units per token, [B, L, H] (to confirm which branch
    of the main pass the inputs take), and the per-chunk maximum."""
    delta = discretize(d["dt"], d.get("dt_bias"), softplus)
    a = np.abs(delta * d["A"].double().numpy()[None, None, :]) * LOG2E
    B, L, H = a.shape
    nc = -(-L // chunk)
    pad = np.zeros((B, nc * chunk, H))
    pad[:, :L] = a
    return a, pad.reshape(B, nc, chunk, H).max(axis=2)


@pytest.mark.parametrize("mma", ["f16", "f32"])
@pytest.mark.parametrize("Q,A_range,cpw", [(64, (8.0, 12.0), 0), (128, (8.0, 12.0), 1),
                                          (256, (4.0, 8.0), 0), (128, (0.05, 8.0), 2)])
def test_strong_decay_takes_the_exact_branch(gpu_lib, mma, Q, A_range, cpw):
    """|delta*A| above 7 (log2 units) for some token of every chunk, or of
    some heads' chunks (mixed): the per-element exponential branch."""
    _say(f"[case] strong decay Q={Q} A=-U{A_range} cpw={cpw} mma={mma}")
    d = random_inputs(2, 3 * Q + 37, 4, 64, 128, 2, seed=910 + Q, has_D=True, has_h0=True,
                      A_range=A_range)
    _, cmax = decay_log2(d, Q)
    if A_range[0] >= 8.0:
        assert (cmax > 7.0).all(), "every chunk must take the exact branch"
    else:
        assert (cmax > 7.0).any(), "some chunks must take the exact branch"
    ref_o, ref_f = run_oracle(d)
    out, fin = run_gpu(gpu_lib, d, Q, mma, cpw=cpw)
    check(out, ref_o, TOL[mma], "out")
    check(fin, ref_f, TOL[mma], "final_state")


@pytest.mark.parametrize("mma", ["f16", "f32"])
@pytest.mark.parametrize("Q", [64, 128, 256])
def test_zero_decay_closed_form(gpu_lib, mma, Q):
    """A = -1e4: every exp(delta*A) underflows, so each token sees only its own
    term: y_t = delta_t (C_t . B_t) x_t + D x_t, final = delta_{L-1} x_{L-1} (outer) B_{L-1}."""
    _say(f"[case] zero decay Q={Q} mma={mma}")
    H, G = 4, 2
    d = random_inputs(2, 2 * Q + 19, H, 64, 64, G, seed=930 + Q, has_D=True, has_h0=True,
                      A_value=-1e4)
    ref_o, ref_f = run_oracle(d)
    # the closed form, from its definition
    delta = discretize(d["dt"], None, True)                       # [B, L, H]
    x = d["x"].double().numpy()
    Bh = np.repeat(d["B"].double().numpy(), H // G, axis=2)       # [B, L, H, N]
    Ch = np.repeat(d["C"].double().numpy(), H // G, axis=2)
    cb = np.sum(Ch * Bh, axis=-1)                                 # [B, L, H]
    closed_o = (delta * cb)[..., None] * x + d["D"].double().numpy()[None, None, :, None] * x
    closed_f = (delta[:, -1, :, None, None] * x[:, -1, :, :, None]) * Bh[:, -1, :, None, :]
    check(ref_o, closed_o, 1e-12, "oracle vs closed form (out)")
    check(ref_f, closed_f, 1e-12, "oracle vs closed form (final)")
    out, fin = run_gpu(gpu_lib, d, Q, mma)
    check(out, closed_o, TOL[mma], "out")
    check(fin, closed_f, TOL[mma], "final_state")


@pytest.mark.parametrize("mma", ["f16", "f32"])
@pytest.mark.parametrize("Q,cpw", [(64, 1), (128, 0), (256, 1)])
def test_no_decay_linear_attention(gpu_lib, mma, Q, cpw):
    """A = 0: the state is the running sum h0 + sum_s delta_s x_s (outer) B_s."""
    _say(f"[case] A = 0 Q={Q} cpw={cpw} mma={mma}")
    d = random_inputs(1, 3 * Q + 11, 4, 64, 128, 1, seed=950 + Q, has_D=True, has_h0=True,
                      A_value=0.0)
    closed_o, closed_f = ssd_linear_attention_closed_form(
        d["x"], d["dt"], d["B"], d["C"], D=d["D"], initial_states=d["initial_states"],
        dt_softplus=True)
    ref_o, ref_f = run_oracle(d)
    check(ref_o, closed_o, 1e-10, "oracle vs closed form (out)")
    out, fin = run_gpu(gpu_lib, d, Q, mma, cpw=cpw)
    check(out, ref_o, TOL[mma], "out")
    check(fin, ref_f, TOL[mma], "final_state")


@pytest.mark.parametrize("mma", ["f16", "f32"])
@pytest.mark.parametrize("limit", [(0.0, math.inf), (0.05, 0.9)])
def test_softplus_off(gpu_lib, mma, limit):
    """dt_softplus = 0: delta = clamp(dt + dt_bias) with the raw step."""
    _say(f"[case] softplus off limit={limit} mma={mma}")
    d = random_inputs(2, 333, 4, 64, 128, 2, seed=970, has_D=True, has_z=True, has_h0=True,
                      dt_bias=True)
    d["dt_bias"] = d["dt_bias"] * 0.1 + 0.05        # keep dt + bias mostly positive
    ref_o, ref_f = run_oracle(d, softplus=False, limit=limit)
    for Q, cpw in ((64, 1), (128, 0)):
        out, fin = run_gpu(gpu_lib, d, Q, mma, softplus=False, limit=limit, cpw=cpw)
        check(out, ref_o, TOL[mma], f"out Q={Q}")
        check(fin, ref_f, TOL[mma], f"final_state Q={Q}")


@pytest.mark.parametrize("mma", ["f16", "f32"])
@pytest.mark.parametrize("Q,N", [(64, 64), (128, 128), (256, 128)])
def test_very_negative_dt_bias(gpu_lib, mma, Q, N):
    """dt_bias ~ U(-11, -5): softplus of arguments in [-11, -4] gives steps of
    about 1.7e-5 .. 2e-2; a softplus that cancels loses their digits."""
    _say(f"[case] dt_bias in [-11,-5] Q={Q} N={N} mma={mma}")
    d = random_inputs(2, 2 * Q + 45, 4, 64, N, 2, seed=990 + Q, has_D=True, has_h0=True,
                      bias_range=(-11.0, -5.0))
    ref_o, ref_f = run_oracle(d)
    for cpw in (0, 1):
        out, fin = run_gpu(gpu_lib, d, Q, mma, cpw=cpw)
        check(out, ref_o, TOL[mma], f"out cpw={cpw}")
        check(fin, ref_f, TOL[mma], f"final_state cpw={cpw}")


def test_headline_workload_fp32_check_path(gpu_lib):
    """The headline workload on the all-fp32 check path, in the plan the
    benchmark uses, with sampled (b, h) sequences against the oracle."""
    w = WORKLOADS["same_device"]
    _say(f"[case] headline {w.shape_str()} mma=f32")
    d = make_inputs(w)
    out, fin = run_gpu(gpu_lib, d, w.chunk, "f32")
    H, G = w.nheads, w.ngroups
    pairs = sorted({(0, 0), (w.batch - 1, H - 1), (1, 5), (2, 10), (3, 3)})
    ref_o, ref_f = ssd_recurrence(d["x"], d["dt"], d["A"], d["B"], d["C"], dt_softplus=True,
                                  pairs=pairs)
    for b, h in pairs:
        check(out[b, :, h], ref_o[b, :, h], TOL["f32"], f"out (b={b}, h={h})")
        check(fin[b, h], ref_f[b, h], TOL["f32"], f"final (b={b}, h={h})")
