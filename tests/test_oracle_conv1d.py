"""Pins of the causal conv1d oracle (CPU only).

Page "ops-transformer MambaV2 算子套件", §1.4 and §4.1 (mamba2_causal_conv1d).
Pinned by hand-derived fixtures (tests/golden/conv1d, derivations inside),
by the page's own reference construction (a grouped torch conv1d padded by
W-1 and cut to S steps, in fp64) and by numpy's full convolution, and by
invariants that a plausible slip breaks: reversed taps, a missing bias, a
sigmoid instead of SiLU, an off-by-one window, a non-causal pad, a conv state
taken from the wrong end.
"""
import glob
import json
import os

import numpy as np
import pytest
import torch

from oracle import causal_conv1d

FIXTURES = sorted(glob.glob(os.path.join(os.path.dirname(__file__), "golden", "conv1d", "*.json")))


def test_fixtures_present():
    assert len(FIXTURES) == 3


@pytest.mark.parametrize("path", FIXTURES, ids=[os.path.basename(p)[:-5] for p in FIXTURES])
def test_golden_hand_derived(path):
    with open(path, encoding="utf-8") as f:
        c = json.load(f)
    arr = lambda v: None if v is None else np.array(v)
    out, fin = causal_conv1d(arr(c["x"]), arr(c["w"]), arr(c["bias"]), arr(c["x_prev"]),
                             activation=c["activation"])
    np.testing.assert_allclose(out, np.array(c["out"]), rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(fin, np.array(c["final"]), rtol=1e-14, atol=1e-14)


def _rand(B, D, S, W, seed):
    r = np.random.default_rng(seed)
    return r.standard_normal((B, D, S)), r.standard_normal((D, W)), r.standard_normal(D)


@pytest.mark.parametrize("W", [2, 3, 4])
def test_matches_the_pages_torch_reference(W):
    # F.conv1d(x, weight [D,1,W], bias, padding=W-1, groups=D)[..., :S], then SiLU
    x, w, b = _rand(2, 5, 37, W, seed=W)
    ref = torch.nn.functional.conv1d(torch.from_numpy(x), torch.from_numpy(w)[:, None, :],
                                     torch.from_numpy(b), stride=1, padding=W - 1, dilation=1,
                                     groups=5)[..., :37]
    ref = torch.nn.functional.silu(ref).numpy()
    out, _ = causal_conv1d(x, w, b)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)


def test_matches_numpy_full_convolution():
    # a causal FIR filter: np.convolve(x, w reversed) cut to S steps
    x, w, _ = _rand(1, 3, 50, 4, seed=11)
    out, _ = causal_conv1d(x, w, None, activation=False)
    for d in range(3):
        np.testing.assert_allclose(out[0, d], np.convolve(x[0, d], w[d, ::-1])[:50], rtol=1e-12,
                                   atol=1e-12)


def test_causal_and_impulse_response():
    x = np.zeros((1, 2, 20))
    x[0, :, 9] = 1.0
    w = np.array([[1.0, 2.0, 3.0, 4.0], [-1.0, 0.5, 0.25, 2.0]])
    out, _ = causal_conv1d(x, w, None, activation=False)
    assert np.all(out[..., :9] == 0) and np.all(out[..., 13:] == 0)
    np.testing.assert_array_equal(out[0, :, 9:13], w[:, ::-1])      # taps newest-first


def test_state_chaining_splits_a_sequence():
    x, w, b = _rand(2, 4, 30, 4, seed=12)
    whole, fin_whole = causal_conv1d(x, w, b)
    first, fin_first = causal_conv1d(x[..., :13], w, b)
    second, fin_second = causal_conv1d(x[..., 13:], w, b, x_prev=fin_first)
    np.testing.assert_allclose(np.concatenate([first, second], axis=2), whole, rtol=1e-13,
                               atol=1e-13)
    np.testing.assert_array_equal(fin_second, fin_whole)
    np.testing.assert_array_equal(fin_whole, x[..., -3:])


def test_channels_independent_and_linear_before_activation():
    x, w, _ = _rand(1, 3, 16, 4, seed=13)
    y, _ = causal_conv1d(x, w, None, activation=False)
    x2 = x.copy()
    x2[0, 1] *= -2.5
    y2, _ = causal_conv1d(x2, w, None, activation=False)
    np.testing.assert_array_equal(y2[0, [0, 2]], y[0, [0, 2]])
    np.testing.assert_allclose(y2[0, 1], -2.5 * y[0, 1], rtol=1e-13)
