"""Pins of the backward oracle (CPU only).

ssd_grads takes the gradients of the token recurrence by autograd in PyTorch
fp64.  It is pinned against central finite differences of the forward
computed by the separate fp64 C recurrence (ssd_recurrence), element by
element for every input, and against the A = 0 closed form of dx and dB.
A dropped decay term, a wrong group map, a missing softplus derivative or
clamp mask, a gate derivative taken as sigmoid, or a final-state gradient
not reaching the inputs each fails.
"""
import math

import numpy as np
import pytest

from oracle import ssd_grads, ssd_recurrence


def _case(seed, Bsz=1, L=7, H=2, P=3, N=2, G=1, opts=True):
    r = np.random.default_rng(seed)
    d = {"x": r.standard_normal((Bsz, L, H, P)), "dt": r.random((Bsz, L, H)) - 0.5,
         "A": -r.random(H) - 0.2, "B": r.standard_normal((Bsz, L, G, N)),
         "C": r.standard_normal((Bsz, L, G, N)),
         "D": r.standard_normal(H) if opts else None,
         "z": r.standard_normal((Bsz, L, H, P)) if opts else None,
         "dt_bias": r.random(H) - 0.5 if opts else None,
         "initial_states": 0.3 * r.standard_normal((Bsz, H, P, N)) if opts else None}
    dout = r.standard_normal((Bsz, L, H, P))
    dfin = r.standard_normal((Bsz, H, P, N)) if opts else None
    return d, dout, dfin


def _loss(d, dout, dfin, softplus, limit):
    out, fin = ssd_recurrence(d["x"], d["dt"], d["A"], d["B"], d["C"], D=d["D"], z=d["z"],
                              dt_bias=d["dt_bias"], initial_states=d["initial_states"],
                              dt_softplus=softplus, dt_limit=limit)
    val = float(np.sum(out * dout))
    if dfin is not None:
        val += float(np.sum(fin * dfin))
    return val


NAMES = {"x": "dx", "dt": "ddt", "A": "dA", "B": "dB", "C": "dC", "D": "dD", "z": "dz",
         "dt_bias": "ddt_bias", "initial_states": "dinitial_states"}


@pytest.mark.parametrize("cfg", [dict(seed=1, softplus=True, limit=(0.0, math.inf)),
                                 dict(seed=2, softplus=False, limit=(0.0, math.inf), H=4, G=2),
                                 dict(seed=3, softplus=True, limit=(0.3, 0.9), Bsz=2, N=3),
                                 dict(seed=4, softplus=True, limit=(0.0, math.inf), opts=False)],
                         ids=["softplus", "groups", "clamp_batch", "bare"])
def test_matches_finite_differences(cfg):
    cfg = dict(cfg)
    softplus, limit = cfg.pop("softplus"), cfg.pop("limit")
    d, dout, dfin = _case(**cfg)
    g = ssd_grads(d["x"], d["dt"], d["A"], d["B"], d["C"], dout, D=d["D"], z=d["z"],
                  dt_bias=d["dt_bias"], initial_states=d["initial_states"], dfinal_state=dfin,
                  dt_softplus=softplus, dt_limit=limit)
    eps = 1e-6
    for k, arr in d.items():
        if arr is None:
            continue
        fd = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            keep = arr[idx]
            arr[idx] = keep + eps
            up = _loss(d, dout, dfin, softplus, limit)
            arr[idx] = keep - eps
            dn = _loss(d, dout, dfin, softplus, limit)
            arr[idx] = keep
            fd[idx] = (up - dn) / (2 * eps)
        got = g[NAMES[k]]
        scale = max(1.0, float(np.abs(fd).max()))
        np.testing.assert_allclose(got, fd, rtol=0, atol=2e-7 * scale, err_msg=k)


def test_clamped_steps_have_no_dt_gradient():
    d, dout, dfin = _case(5, L=9)
    limit = (0.45, 0.75)
    g = ssd_grads(d["x"], d["dt"], d["A"], d["B"], d["C"], dout, D=d["D"], z=d["z"],
                  dt_bias=d["dt_bias"], initial_states=d["initial_states"], dfinal_state=dfin,
                  dt_softplus=True, dt_limit=limit)
    u = d["dt"] + d["dt_bias"][None, None, :]
    sp = np.log1p(np.exp(u))
    clamped = (sp < limit[0]) | (sp > limit[1])
    assert clamped.any() and (~clamped).any()
    assert np.all(g["ddt"][clamped] == 0) and np.all(g["ddt"][~clamped] != 0)


def test_zero_decay_closed_form():
    # A = 0, no softplus: h_t = h0 + sum_{s<=t} delta_s x_s B_s^T, so
    # dx_s = delta_s sum_{t>=s} (C_t . B_s) dout_t + D dout_s and
    # dB_s = delta_s sum_{t>=s} (dout_t . x_s) C_t  (one head, one group)
    r = np.random.default_rng(6)
    L, P, N = 8, 3, 4
    x, dt = r.standard_normal((1, L, 1, P)), r.random((1, L, 1)) + 0.1
    B, C = r.standard_normal((1, L, 1, N)), r.standard_normal((1, L, 1, N))
    dout, D = r.standard_normal((1, L, 1, P)), np.array([0.7])
    g = ssd_grads(x, dt, np.zeros(1), B, C, dout, D=D)
    xs, bs, cs, dy, dl = x[0, :, 0], B[0, :, 0], C[0, :, 0], dout[0, :, 0], dt[0, :, 0]
    dx = np.array([dl[s] * sum((cs[t] @ bs[s]) * dy[t] for t in range(s, L)) + D[0] * dy[s]
                   for s in range(L)])
    dB = np.array([dl[s] * sum((dy[t] @ xs[s]) * cs[t] for t in range(s, L)) for s in range(L)])
    np.testing.assert_allclose(g["dx"][0, :, 0], dx, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(g["dB"][0, :, 0], dB, rtol=1e-12, atol=1e-12)
