"""Pins of the gated grouped RMSNorm oracle (CPU only).

The operator follows page "ops-transformer MambaV2 算子套件", section 4.6
(mamba2_rmsnormgated).  Pinned by hand-derived fixtures (tests/golden/rmsnorm,
derivations inside) and by closed forms and invariants that a plausible slip
breaks: interleaved instead of contiguous groups, a sum instead of a mean,
eps outside the root, a sigmoid instead of SiLU, a missing weight.
"""
import glob
import json
import os

import numpy as np
import pytest

from oracle import rmsnorm_gated

FIXTURES = sorted(glob.glob(os.path.join(os.path.dirname(__file__), "golden", "rmsnorm", "*.json")))


def test_fixtures_present():
    assert len(FIXTURES) == 4


@pytest.mark.parametrize("path", FIXTURES, ids=[os.path.basename(p)[:-5] for p in FIXTURES])
def test_golden_hand_derived(path):
    with open(path, encoding="utf-8") as f:
        c = json.load(f)
    got = rmsnorm_gated(np.array(c["x"]), None if c["z"] is None else np.array(c["z"]),
                        np.array(c["w"]), c["ngroups"], c["eps"])
    np.testing.assert_allclose(got, np.array(c["out"]), rtol=1e-14, atol=1e-14)


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_group_of_one_is_the_sign():
    # each group holds one element: g / |g| * w (eps = 0)
    x, z, w = _rand((3, 8), 1), _rand((3, 8), 2), _rand(8, 3)
    g = x * z / (1 + np.exp(-z))
    np.testing.assert_allclose(rmsnorm_gated(x, z, w, 8, 0.0), np.sign(g) * w, rtol=0, atol=1e-15)


def test_each_group_has_unit_rms():
    x, z = _rand((5, 24), 4), _rand((5, 24), 5)
    out = rmsnorm_gated(x, z, np.ones(24), 3, 0.0).reshape(5, 3, 8)
    np.testing.assert_allclose(np.mean(out * out, axis=-1), 1.0, rtol=1e-13)


def test_scale_invariance_and_odd_symmetry():
    x, w = _rand((4, 16), 6), _rand(16, 7)
    ref = rmsnorm_gated(x, None, w, 4, 0.0)
    np.testing.assert_allclose(rmsnorm_gated(3.7 * x, None, w, 4, 0.0), ref, rtol=1e-13)
    np.testing.assert_allclose(rmsnorm_gated(-x, None, w, 4, 0.0), -ref, rtol=1e-13)
    # a constant positive gate is a positive scale: no effect at eps = 0
    zc = np.full_like(x, 0.8)
    np.testing.assert_allclose(rmsnorm_gated(x, zc, w, 4, 0.0), ref, rtol=1e-13)


def test_groups_are_contiguous_and_independent():
    x, z, w = _rand((2, 12), 8), _rand((2, 12), 9), _rand(12, 10)
    ref = rmsnorm_gated(x, z, w, 3, 1e-3)
    x2 = x.copy()
    x2[:, 4:8] *= -2.5       # only group 1 changes
    got = rmsnorm_gated(x2, z, w, 3, 1e-3)
    np.testing.assert_array_equal(got[:, :4], ref[:, :4])
    np.testing.assert_array_equal(got[:, 8:], ref[:, 8:])
    assert not np.allclose(got[:, 4:8], ref[:, 4:8])


def test_large_eps_limit():
    # sqrt(mean g^2 + eps) -> sqrt(eps): out * sqrt(eps) -> g * w
    x, z, w = _rand((3, 10), 11), _rand((3, 10), 12), _rand(10, 13)
    g = x * z / (1 + np.exp(-z))
    eps = 1e12
    np.testing.assert_allclose(rmsnorm_gated(x, z, w, 2, eps) * np.sqrt(eps), g * w, rtol=1e-10)


def test_zero_input_gives_zero():
    assert np.all(rmsnorm_gated(np.zeros((2, 8)), None, np.ones(8), 2, 1e-5) == 0.0)


def test_group_count_must_divide():
    with pytest.raises(ValueError):
        rmsnorm_gated(np.zeros((1, 10)), None, np.ones(10), 3, 0.0)
