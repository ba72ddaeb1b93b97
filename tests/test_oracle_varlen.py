"""Pins of the packed variable-length oracle (CPU only).

Packed sequences: page "Mamba-2 SSD for Ascend NPU", "Limitations and
roadmap" (varlen / cu_seqlens), and page "ops-transformer MambaV2 算子套件"
§1.4 (sequences concatenated on one token axis, delimited by cumulative
offsets).  ssd_varlen (the recurrence per sequence) is pinned by
hand-derived fixtures (tests/golden/varlen, derivations inside), by the
independent masked-matrix form ssd_quadratic_seq_idx, and by invariants a
plausible slip breaks: a state carried across a boundary, the wrong
sequence's initial state, an off-by-one start offset, a dropped D or gate.
"""
import glob
import json
import os

import numpy as np
import pytest

from oracle import (ssd_linear_attention_closed_form, ssd_quadratic, ssd_quadratic_seq_idx,
                    ssd_varlen)

FIXTURES = sorted(glob.glob(os.path.join(os.path.dirname(__file__), "golden", "varlen", "*.json")))


def test_fixtures_present():
    assert len(FIXTURES) == 2


@pytest.mark.parametrize("path", FIXTURES, ids=[os.path.basename(p)[:-5] for p in FIXTURES])
@pytest.mark.parametrize("fn", [ssd_varlen, ssd_quadratic_seq_idx], ids=["varlen", "quadratic"])
def test_golden_hand_derived(path, fn):
    with open(path, encoding="utf-8") as f:
        c = json.load(f)
    T = len(c["x"])
    nseq = len(c["cu_seqlens"]) - 1
    x = np.array(c["x"]).reshape(T, 1, 1)
    dt = np.array(c["dt"]).reshape(T, 1)
    B = np.array(c["B"]).reshape(T, 1, 1)
    C = np.array(c["C"]).reshape(T, 1, 1)
    D = None if c["D"] is None else np.array([c["D"]])
    h0 = None if c["h0"] is None else np.array(c["h0"]).reshape(nseq, 1, 1, 1)
    out, fin = fn(x, dt, np.array([c["A"]]), B, C, c["cu_seqlens"], D=D, initial_states=h0,
                  dt_softplus=c["dt_softplus"])
    np.testing.assert_allclose(out.reshape(-1), c["out"], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(fin.reshape(-1), c["final"], rtol=1e-13, atol=1e-13)


def _packed(lens, H=4, P=8, N=6, G=2, seed=0, D=True, z=True, h0=True, bias=True):
    rng = np.random.default_rng(seed)
    T = int(sum(lens))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    d = {"x": rng.standard_normal((T, H, P)), "dt": rng.random((T, H)), "A": -rng.random(H),
         "B": rng.standard_normal((T, G, N)), "C": rng.standard_normal((T, G, N)),
         "D": rng.standard_normal(H) if D else None,
         "z": rng.standard_normal((T, H, P)) if z else None,
         "dt_bias": -rng.random(H) if bias else None,
         "initial_states": 0.1 * rng.standard_normal((len(lens), H, P, N)) if h0 else None}
    return d, cu


def _call(fn, d, cu, **kw):
    return fn(d["x"], d["dt"], d["A"], d["B"], d["C"], cu, D=d["D"], z=d["z"],
              dt_bias=d["dt_bias"], initial_states=d["initial_states"], dt_softplus=True, **kw)


@pytest.mark.parametrize("lens,G", [([5, 0, 1, 13, 7], 2), ([1, 1, 1], 1), ([30], 4), ([0, 9, 0], 4),
                                    ([2, 17, 3, 11, 1, 6], 1)])
@pytest.mark.parametrize("opts", [dict(), dict(D=False, z=False, h0=False, bias=False)],
                         ids=["all_options", "bare"])
def test_recurrence_matches_masked_matrix(lens, G, opts):
    d, cu = _packed(lens, G=G, seed=len(lens) * 31 + G, **opts)
    o1, f1 = _call(ssd_varlen, d, cu)
    o2, f2 = _call(ssd_quadratic_seq_idx, d, cu)
    np.testing.assert_allclose(o1, o2, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(f1, f2, rtol=1e-11, atol=1e-11)


def test_one_sequence_is_the_plain_forward():
    # against the unpacked quadratic form (a different construction again)
    d, cu = _packed([23], seed=3)
    o, f = _call(ssd_varlen, d, cu)
    q = {k: (None if v is None else v[None]) for k, v in d.items()
         if k in ("x", "dt", "B", "C", "z")}
    oq, fq = ssd_quadratic(q["x"], q["dt"], d["A"], q["B"], q["C"], D=d["D"], z=q["z"],
                           dt_bias=d["dt_bias"], initial_states=d["initial_states"],
                           dt_softplus=True)
    np.testing.assert_allclose(o, oq[0], rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(f, fq, rtol=1e-11, atol=1e-11)


@pytest.mark.parametrize("fn", [ssd_varlen, ssd_quadratic_seq_idx], ids=["varlen", "quadratic"])
def test_sequences_are_independent(fn):
    lens = [6, 9, 4]
    d, cu = _packed(lens, seed=4)
    o, f = _call(fn, d, cu)
    d2 = {k: (None if v is None else v.copy()) for k, v in d.items()}
    sl = slice(cu[1], cu[2])                    # perturb everything of sequence 1
    for k in ("x", "dt", "B", "C", "z"):
        d2[k][sl] = -3.0 * d2[k][sl] + 0.5
    d2["initial_states"][1] *= -7.0
    o2, f2 = _call(fn, d2, cu)
    # (the masked matrix takes decays as differences of one cumulative sum over
    # the whole packed axis, so other sequences move by rounding only)
    for s in (0, 2):
        np.testing.assert_allclose(o2[cu[s]:cu[s + 1]], o[cu[s]:cu[s + 1]], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(f2[s], f[s], rtol=1e-12, atol=1e-12)
    assert not np.allclose(o2[sl], o[sl]) and not np.allclose(f2[1], f[1])


@pytest.mark.parametrize("fn", [ssd_varlen, ssd_quadratic_seq_idx], ids=["varlen", "quadratic"])
def test_split_sequence_chains_through_initial_state(fn):
    # one sequence of 19 tokens == the same tokens packed as 8 + 11 with the
    # second part starting from the first part's final state
    d, cu = _packed([19], seed=5)
    o_whole, f_whole = _call(fn, d, cu)
    part = [0, 8, 19]
    h0 = d["initial_states"][0]
    d1 = dict(d, initial_states=np.stack([h0, np.zeros_like(h0)]))
    _, f_first = _call(fn, d1, part)            # sequence 0's final state = after 8 tokens
    d2 = dict(d, initial_states=np.stack([h0, f_first[0]]))
    o_split, f_split = _call(fn, d2, part)
    np.testing.assert_allclose(o_split, o_whole, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(f_split[1], f_whole[0], rtol=1e-11, atol=1e-11)


def test_zero_decay_closed_form_per_sequence():
    # A = 0: each sequence is causal linear attention from its own h0
    d, cu = _packed([7, 0, 12, 3], seed=6, z=False)
    d["A"] = np.zeros_like(d["A"])
    o, f = _call(ssd_varlen, d, cu)
    for s in range(len(cu) - 1):
        a, e = cu[s], cu[s + 1]
        if a == e:
            np.testing.assert_array_equal(f[s], d["initial_states"][s])
            continue
        oc, fc = ssd_linear_attention_closed_form(
            d["x"][None, a:e], d["dt"][None, a:e], d["B"][None, a:e], d["C"][None, a:e], D=d["D"],
            dt_bias=d["dt_bias"], initial_states=d["initial_states"][s:s + 1], dt_softplus=True)
        np.testing.assert_allclose(o[a:e], oc[0], rtol=1e-11, atol=1e-11)
        np.testing.assert_allclose(f[s], fc[0], rtol=1e-11, atol=1e-11)


def test_batch_of_one_layout_accepted():
    d, cu = _packed([4, 5], seed=7)
    o1, f1 = _call(ssd_varlen, d, cu)
    d1 = {k: (v[None] if k in ("x", "dt", "B", "C", "z") else v) for k, v in d.items()}
    o2, f2 = _call(ssd_varlen, d1, cu)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(f1, f2)


@pytest.mark.parametrize("cu", [[1, 5], [0, 4], [0, 3, 2, 5], [5]])
def test_bad_offsets_rejected(cu):
    d, _ = _packed([5], seed=8)
    with pytest.raises(ValueError):
        _call(ssd_varlen, d, cu)
