"""Pins for the CPU oracle (runs without a GPU).

The fp64 recurrence in oracle/ssd_oracle.c is the reference every GPU result
is compared against, so it is pinned here to things other than itself:
  * hand-derived golden values (tests/golden/*.json, derivations inside);
  * the quadratic semiseparable-matrix form (an independent NumPy
    restatement of the SSD "attention view");
  * the four-stage chunked form at several chunk sizes (chunk-size
    invariance; Q = 1 is the recurrence, Q = L the quadratic form);
  * the A = 0 closed form (causal linear attention) and the zero-decay
    closed form (each token sees only itself);
  * invariants: split-sequence (initial/final state chaining), group
    replication (head h -> group h // (H/G)), causality, linearity in x,
    and the D / z identities.
A plausible slip in the recurrence (wrong update order, a dropped term, a
wrong sign, index or group map) breaks at least one of these.
"""
import glob
import json
import math
import os

import numpy as np
import pytest

from oracle import (discretize, ssd_chunked, ssd_linear_attention_closed_form, ssd_quadratic,
                    ssd_recurrence)
from workloads import WORKLOADS, make_inputs, random_inputs

GOLDEN = sorted(glob.glob(os.path.join(os.path.dirname(__file__), "golden", "*.json")))


def _np(d, k):
    v = d.get(k)
    return None if v is None else np.asarray(v, dtype=np.float64)


@pytest.mark.parametrize("path", GOLDEN, ids=[os.path.basename(p)[:-5] for p in GOLDEN])
def test_golden_hand_derived(path):
    with open(path) as f:
        c = json.load(f)
    lim = c["dt_limit"]
    dt_limit = (lim[0], math.inf if lim[1] is None else lim[1])
    kw = dict(D=_np(c, "D"), z=_np(c, "z"), dt_bias=_np(c, "dt_bias"),
              initial_states=_np(c, "initial_states"), dt_softplus=c["dt_softplus"],
              dt_limit=dt_limit)
    args = [_np(c, k) for k in ("x", "dt", "A", "B", "C")]
    out, fin = ssd_recurrence(*args, **kw)
    np.testing.assert_allclose(out, np.asarray(c["out"]), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(fin, np.asarray(c["final_state"]), rtol=1e-12, atol=1e-12)
    # the independent forms reproduce the same hand values
    q_out, q_fin = ssd_quadratic(*args, **kw)
    np.testing.assert_allclose(q_out, np.asarray(c["out"]), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(q_fin, np.asarray(c["final_state"]), rtol=1e-12, atol=1e-12)
    L = c["shape"]["L"]
    for Q in sorted({1, 2, L}):
        k_out, k_fin, _ = ssd_chunked(*args, Q, **kw)
        np.testing.assert_allclose(k_out, np.asarray(c["out"]), rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(k_fin, np.asarray(c["final_state"]), rtol=1e-12, atol=1e-12)


def test_softplus_values():
    # softplus(0) = ln 2; softplus(u) -> u for large u; softplus(-u) = softplus(u) - u
    d = discretize(np.array([0.0, 40.0, -3.0, 3.0]), dt_softplus=True)
    assert abs(d[0] - math.log(2.0)) < 1e-15
    assert abs(d[1] - 40.0) < 1e-12
    assert abs(d[3] - d[2] - 3.0) < 1e-12
    # bias added before softplus, clamp after
    d2 = discretize(np.array([[0.5]]), dt_bias=np.array([-0.5]), dt_softplus=True,
                    dt_limit=(0.0, 0.5))
    assert abs(d2[0, 0] - 0.5) < 1e-15
    d3 = discretize(np.array([[0.5]]), dt_bias=np.array([-0.5]), dt_softplus=True)
    assert abs(d3[0, 0] - math.log(2.0)) < 1e-15


SMALL_CASES = [
    # (B, L, H, P, N, G, has_D, has_z, has_h0, dt_bias, seed)
    (1, 37, 2, 4, 3, 1, False, False, False, False, 1),
    (2, 64, 4, 8, 16, 2, True, False, False, False, 2),
    (2, 50, 4, 3, 5, 4, True, True, True, True, 3),
    (1, 29, 6, 2, 7, 3, False, True, True, False, 4),
]


def _case_kwargs(d, softplus=True, limit=(0.0, math.inf)):
    return dict(D=d["D"], z=d["z"], dt_bias=d["dt_bias"], initial_states=d["initial_states"],
                dt_softplus=softplus, dt_limit=limit)


def _args(d):
    return d["x"], d["dt"], d["A"], d["B"], d["C"]


@pytest.mark.parametrize("case", SMALL_CASES)
def test_recurrence_equals_quadratic_form(case):
    Bsz, L, H, P, N, G, hD, hz, hh, hb, seed = case
    d = random_inputs(Bsz, L, H, P, N, G, seed, has_D=hD, has_z=hz, has_h0=hh, dt_bias=hb)
    for softplus, limit in ((True, (0.0, math.inf)), (False, (0.05, 0.8))):
        kw = _case_kwargs(d, softplus, limit)
        out, fin = ssd_recurrence(*_args(d), **kw)
        q_out, q_fin = ssd_quadratic(*_args(d), **kw)
        np.testing.assert_allclose(out, q_out, rtol=1e-10, atol=1e-10)
        np.testing.assert_allclose(fin, q_fin, rtol=1e-10, atol=1e-10)


@pytest.mark.parametrize("case", SMALL_CASES)
def test_chunk_size_invariance(case):
    Bsz, L, H, P, N, G, hD, hz, hh, hb, seed = case
    d = random_inputs(Bsz, L, H, P, N, G, seed, has_D=hD, has_z=hz, has_h0=hh, dt_bias=hb)
    kw = _case_kwargs(d)
    out, fin = ssd_recurrence(*_args(d), **kw)
    for Q in (1, 3, 8, 16, L):
        c_out, c_fin, inter = ssd_chunked(*_args(d), Q, **kw)
        np.testing.assert_allclose(c_out, out, rtol=1e-10, atol=1e-10, err_msg=f"Q={Q}")
        np.testing.assert_allclose(c_fin, fin, rtol=1e-10, atol=1e-10, err_msg=f"Q={Q}")
        # the state entering chunk c is the final state of the prefix [0, cQ)
        nc = -(-L // Q)
        for c in {1, nc // 2, nc - 1}:
            if c < 1 or c * Q >= L:
                continue
            sub = {k: (None if v is None else (v[:, :c * Q] if k in ("x", "dt", "B", "C", "z")
                                               else v)) for k, v in d.items()}
            _, pre_fin = ssd_recurrence(*_args(sub), **_case_kwargs(sub))
            np.testing.assert_allclose(inter["S_in"][:, :, c], pre_fin, rtol=1e-10, atol=1e-10)


def test_tiny_workload_forms_agree():
    w = WORKLOADS["tiny"]
    d = make_inputs(w)
    out, fin = ssd_recurrence(*_args(d), dt_softplus=True)
    q_out, q_fin = ssd_quadratic(*_args(d), dt_softplus=True)
    c_out, c_fin, _ = ssd_chunked(*_args(d), w.chunk, dt_softplus=True)
    scale = np.abs(out).max()
    assert np.abs(out - q_out).max() <= 1e-12 * scale
    assert np.abs(out - c_out).max() <= 1e-12 * scale
    np.testing.assert_allclose(fin, q_fin, rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(fin, c_fin, rtol=1e-10, atol=1e-10)


def test_A_zero_linear_attention_closed_form():
    d = random_inputs(2, 41, 4, 5, 6, 2, 11, has_D=True, has_h0=True, dt_bias=True)
    A0 = np.zeros(4)
    out, fin = ssd_recurrence(d["x"], d["dt"], A0, d["B"], d["C"], D=d["D"],
                              dt_bias=d["dt_bias"], initial_states=d["initial_states"],
                              dt_softplus=True)
    ref, ref_fin = ssd_linear_attention_closed_form(d["x"], d["dt"], d["B"], d["C"], D=d["D"],
                                                    dt_bias=d["dt_bias"],
                                                    initial_states=d["initial_states"],
                                                    dt_softplus=True)
    np.testing.assert_allclose(out, ref, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(fin, ref_fin, rtol=1e-11, atol=1e-11)


def test_zero_decay_closed_form():
    # A = -1e4 with delta >= ln 2: exp(delta*A) underflows to exactly 0, so each
    # token sees only itself: y_t = delta_t (C_t . B_t) x_t + D x_t.
    d = random_inputs(2, 23, 4, 3, 5, 2, 12, has_D=True)
    H = 4
    A = np.full(H, -1e4)
    out, fin = ssd_recurrence(d["x"], d["dt"], A, d["B"], d["C"], D=d["D"], dt_softplus=True)
    delta = discretize(d["dt"], dt_softplus=True)
    x = d["x"].double().numpy()
    Bh = np.repeat(d["B"].double().numpy(), 2, axis=2)
    Ch = np.repeat(d["C"].double().numpy(), 2, axis=2)
    cb = np.sum(Ch * Bh, axis=-1)                                   # [B,L,H]
    ref = (delta * cb)[..., None] * x + d["D"].double().numpy()[None, None, :, None] * x
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)
    ref_fin = delta[:, -1, :, None, None] * x[:, -1, :, :, None] * Bh[:, -1, :, None, :]
    np.testing.assert_allclose(fin, ref_fin, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("k", [1, 16, 33, 63])
def test_split_sequence_invariance(k):
    d = random_inputs(2, 64, 4, 6, 8, 2, 13, has_D=True, has_z=True, has_h0=True, dt_bias=True)
    kw = _case_kwargs(d)
    out, fin = ssd_recurrence(*_args(d), **kw)
    first = {key: (None if v is None else (v[:, :k] if key in ("x", "dt", "B", "C", "z") else v))
             for key, v in d.items()}
    out1, fin1 = ssd_recurrence(*_args(first), **_case_kwargs(first))
    second = {key: (None if v is None else (v[:, k:] if key in ("x", "dt", "B", "C", "z") else v))
              for key, v in d.items()}
    second["initial_states"] = fin1
    out2, fin2 = ssd_recurrence(*_args(second), **_case_kwargs(second))
    np.testing.assert_allclose(np.concatenate([out1, out2], axis=1), out, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(fin2, fin, rtol=1e-11, atol=1e-11)


def test_group_replication():
    # G < H must equal G = H with B/C repeated so that head h reads group h // (H/G)
    import torch
    d = random_inputs(2, 31, 6, 4, 5, 3, 14, has_D=True)
    out, fin = ssd_recurrence(*_args(d), D=d["D"], dt_softplus=True)
    Bf = torch.repeat_interleave(d["B"], 2, dim=2)
    Cf = torch.repeat_interleave(d["C"], 2, dim=2)
    out_f, fin_f = ssd_recurrence(d["x"], d["dt"], d["A"], Bf, Cf, D=d["D"], dt_softplus=True)
    np.testing.assert_array_equal(out, out_f)
    np.testing.assert_array_equal(fin, fin_f)
    # the other plausible map (h % G) gives a different answer on this input
    Bm = d["B"][:, :, [h % 3 for h in range(6)]]
    Cm = d["C"][:, :, [h % 3 for h in range(6)]]
    out_m, _ = ssd_recurrence(d["x"], d["dt"], d["A"], Bm, Cm, D=d["D"], dt_softplus=True)
    assert np.abs(out_m - out).max() > 1e-3


def test_causality():
    d = random_inputs(1, 40, 2, 4, 6, 1, 15, has_D=True, has_z=True, has_h0=True)
    kw = _case_kwargs(d)
    out, _ = ssd_recurrence(*_args(d), **kw)
    t = 17
    x2 = d["x"].clone()
    x2[:, t] += 1.0
    out2, _ = ssd_recurrence(x2, d["dt"], d["A"], d["B"], d["C"], **kw)
    np.testing.assert_array_equal(out2[:, :t], out[:, :t])
    assert np.abs(out2[:, t:] - out[:, t:]).max() > 0


def test_linearity_in_x():
    d = random_inputs(1, 33, 2, 3, 4, 1, 16, has_D=True)
    x1 = d["x"]
    x2 = random_inputs(1, 33, 2, 3, 4, 1, 17)["x"]
    a, b = 0.75, -1.25
    o1, f1 = ssd_recurrence(x1, d["dt"], d["A"], d["B"], d["C"], D=d["D"], dt_softplus=True)
    o2, f2 = ssd_recurrence(x2, d["dt"], d["A"], d["B"], d["C"], D=d["D"], dt_softplus=True)
    o3, f3 = ssd_recurrence(a * x1.double() + b * x2.double(), d["dt"], d["A"], d["B"], d["C"],
                            D=d["D"], dt_softplus=True)
    np.testing.assert_allclose(o3, a * o1 + b * o2, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(f3, a * f1 + b * f2, rtol=1e-11, atol=1e-11)


def test_D_and_z_identities():
    d = random_inputs(2, 27, 4, 5, 3, 2, 18, has_D=True, has_z=True, has_h0=True)
    base_kw = dict(initial_states=d["initial_states"], dt_softplus=True)
    y0, f0 = ssd_recurrence(*_args(d), **base_kw)
    yD, fD = ssd_recurrence(*_args(d), D=d["D"], **base_kw)
    x = d["x"].double().numpy()
    np.testing.assert_allclose(yD - y0, d["D"].double().numpy()[None, None, :, None] * x,
                               rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(fD, f0)       # D never enters the state
    yDz, fDz = ssd_recurrence(*_args(d), D=d["D"], z=d["z"], **base_kw)
    z = d["z"].double().numpy()
    np.testing.assert_allclose(yDz, yD * z / (1.0 + np.exp(-z)), rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(fDz, f0)      # nor does the gate


def test_pairs_subset_matches_full():
    d = random_inputs(3, 20, 4, 3, 4, 2, 19, has_D=True, has_h0=True)
    kw = _case_kwargs(d)
    out, fin = ssd_recurrence(*_args(d), **kw)
    pairs = [(0, 3), (2, 1)]
    o2, f2 = ssd_recurrence(*_args(d), pairs=pairs, **kw)
    for b, h in pairs:
        np.testing.assert_array_equal(o2[b, :, h], out[b, :, h])
        np.testing.assert_array_equal(f2[b, h], fin[b, h])
    assert np.isnan(o2[1]).all()


def test_tail_padding_is_inert():
    # a ragged last chunk gives the unpadded recurrence (padded tokens change nothing)
    d = random_inputs(1, 45, 2, 3, 4, 1, 20, has_h0=True)
    kw = _case_kwargs(d)
    out, fin = ssd_recurrence(*_args(d), **kw)
    for Q in (16, 32, 64):
        c_out, c_fin, inter = ssd_chunked(*_args(d), Q, **kw)
        np.testing.assert_allclose(c_out, out, rtol=1e-11, atol=1e-11)
        np.testing.assert_allclose(c_fin, fin, rtol=1e-11, atol=1e-11)
        assert np.all(inter["delta"].reshape(1, 2, -1)[:, :, 45:] == 0)


def test_float_instance_is_the_same_recurrence():
    """The fp32 instance the benchmark times as its CPU baseline follows the
    fp64 recurrence to single-precision rounding (every option on)."""
    from oracle import ssd_recurrence_f32
    d = random_inputs(2, 150, 4, 8, 16, 2, seed=77, has_D=True, has_z=True, has_h0=True,
                      dt_bias=True)
    kw = dict(D=d["D"], z=d["z"], dt_bias=d["dt_bias"], initial_states=d["initial_states"],
              dt_softplus=True, dt_limit=(0.7, 1.2))
    ref = ssd_recurrence(d["x"], d["dt"], d["A"], d["B"], d["C"], **kw)
    for threads in (1, 0):
        got = ssd_recurrence_f32(d["x"], d["dt"], d["A"], d["B"], d["C"], nthreads=threads, **kw)
        for g, r in zip(got, ref):
            assert g.dtype == np.float32
            assert np.abs(g - r).max() <= 1e-5 * np.abs(r).max()
