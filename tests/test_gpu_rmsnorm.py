"""GPU parity of the gated grouped RMSNorm (ssd_rmsnorm_gated through the C
ABI) against the fp64 oracle, page "ops-transformer MambaV2 算子套件",
section 4.6.

Bar: |gpu - oracle| <= 1e-5 * |oracle| + 1e-6 * max|oracle| element-wise.
Everything is fp32 and every error source is multiplicative: the gate
(hardware exp2 and reciprocal, a few ulp), the sum of at most 4096 squares
(at most 64 sequential terms per lane, then a 6-level lane tree: below
70 * 2^-24 = 4.2e-6 relative in the worst case) and the reciprocal root, so
each output is within a few 1e-6 of its own magnitude.
"""
import sys

import numpy as np
import pytest
import torch

from oracle import rmsnorm_gated as oracle_norm
from workloads import NORM_EPS, WORKLOADS, norm_inputs, norm_shape

pytestmark = pytest.mark.gpu

RTOL, ATOL_REL = 1e-5, 1e-6


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def check(got, ref, what):
    got = np.asarray(got, dtype=np.float64)
    assert got.shape == ref.shape
    scale = float(np.nanmax(np.abs(ref))) if np.isfinite(ref).any() else 0.0
    err = np.abs(got - ref)
    worst = float(np.nanmax(err / (RTOL * np.abs(ref) + ATOL_REL * scale + 1e-300)))
    _say(f"    {what}: max_err/max_ref={float(np.nanmax(err)) / (scale or 1):.3e} "
         f"worst/bound={worst:.3f}")
    np.testing.assert_allclose(got, ref, rtol=RTOL, atol=ATOL_REL * scale, equal_nan=True)


def run(ssd, d, ngroups, eps, out=None):
    g = {k: (None if v is None else v.cuda()) for k, v in d.items()}
    res = ssd.rmsnorm_gated(g["x"], g["z"], g["w"], ngroups, eps, out=out)
    torch.cuda.synchronize()
    return res


# (rows, dim, ngroups): group sizes 4 .. 4096, every per-lane slot count,
# groups that fill a wave exactly and ragged ones (a partial last slot row).
SHAPES = [(1, 4, 1), (3, 12, 3), (5, 64, 1), (7, 256, 4), (9, 260, 1), (4, 1000, 2),
          (6, 1024, 4), (3, 2048, 1), (2, 3076, 1), (2, 4096, 1), (2, 8192, 2), (33, 768, 3),
          (130, 512, 8)]


@pytest.mark.parametrize("gate", [True, False], ids=["z", "noz"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_random_shapes_match_oracle(gpu_lib, shape, gate):
    rows, dim, G = shape
    _say(f"  rmsnorm rows={rows} dim={dim} G={G} z={gate}")
    d = norm_inputs(rows, dim, seed=rows * 7919 + dim * 31 + G, has_z=gate)
    got = run(gpu_lib, d, G, NORM_EPS).cpu().numpy()
    ref = oracle_norm(d["x"].numpy(), None if d["z"] is None else d["z"].numpy(), d["w"].numpy(),
                      G, NORM_EPS)
    check(got, ref, "out")


@pytest.mark.parametrize("eps", [0.0, 1e-2, 10.0])
def test_eps_values(gpu_lib, eps):
    d = norm_inputs(16, 640, seed=404, has_z=True)
    got = run(gpu_lib, d, 5, eps).cpu().numpy()
    check(got, oracle_norm(d["x"].numpy(), d["z"].numpy(), d["w"].numpy(), 5, eps), f"eps={eps}")


def test_leading_dims_and_in_place(gpu_lib):
    d = norm_inputs(2 * 37, 512, seed=405, has_z=True)
    x = d["x"].view(2, 37, 512).cuda()
    z = d["z"].view(2, 37, 512).cuda()
    w = d["w"].cuda()
    ref = oracle_norm(d["x"].numpy(), d["z"].numpy(), d["w"].numpy(), 2, NORM_EPS)
    out = gpu_lib.rmsnorm_gated(x, z, w, 2, NORM_EPS)
    torch.cuda.synchronize()
    check(out.cpu().numpy().reshape(74, 512), ref, "[B,S,D]")
    same = gpu_lib.rmsnorm_gated(x, z, w, 2, NORM_EPS, out=x)       # in place over x
    torch.cuda.synchronize()
    assert same is x
    assert torch.equal(x, out)                                      # bit-identical


def test_zero_groups_and_eps_zero(gpu_lib):
    # eps > 0: an all-zero group gives exact zeros.  eps = 0: 0/0 is NaN, on
    # both sides, and only in that group.
    d = norm_inputs(4, 256, seed=406, has_z=False)
    d["x"][1, 64:128] = 0.0
    d["x"][3, :] = 0.0
    got = run(gpu_lib, d, 4, 1e-6).cpu().numpy()
    assert (got[1, 64:128] == 0).all() and (got[3] == 0).all()
    check(got, oracle_norm(d["x"].numpy(), None, d["w"].numpy(), 4, 1e-6), "eps>0")
    with np.errstate(invalid="ignore", divide="ignore"):
        ref = oracle_norm(d["x"].numpy(), None, d["w"].numpy(), 4, 0.0)
    got = run(gpu_lib, d, 4, 0.0).cpu().numpy()
    assert np.isnan(got[1, 64:128]).all() and np.isfinite(got[1, :64]).all()
    check(got, ref, "eps=0")


def test_extreme_gate_values(gpu_lib):
    # z far below zero switches the gate off (silu -> -0), far above it
    # passes x through; no overflow to NaN either way.
    d = norm_inputs(4, 256, seed=407, has_z=True)
    d["z"][0] = -200.0
    d["z"][1] = 200.0
    d["z"][2, ::2] = -95.0
    got = run(gpu_lib, d, 1, 1e-5).cpu().numpy()
    assert np.isfinite(got).all()
    with np.errstate(over="ignore"):
        ref = oracle_norm(d["x"].numpy(), d["z"].numpy(), d["w"].numpy(), 1, 1e-5)
    check(got, ref, "extreme z")


def test_deterministic(gpu_lib):
    d = norm_inputs(300, 2048, seed=408, has_z=True)
    a = run(gpu_lib, d, 2, NORM_EPS)
    b = run(gpu_lib, d, 2, NORM_EPS)
    assert torch.equal(a, b)


@pytest.mark.parametrize("name", ["same_device", "h256", "long", "gated"])
def test_full_size_sampled_rows(gpu_lib, name):
    """The norm after each SSD workload at its full size, in the launch the
    benchmark times; the oracle checks a spread of sampled rows."""
    rows, dim, G = norm_shape(WORKLOADS[name])
    _say(f"  rmsnorm full size {name}: rows={rows} dim={dim} G={G}")
    d = norm_inputs(rows, dim, seed=WORKLOADS[name].seed + 500, has_z=True, device="cuda")
    out = gpu_lib.rmsnorm_gated(d["x"], d["z"], d["w"], G, NORM_EPS)
    torch.cuda.synchronize()
    idx = torch.unique(torch.cat([torch.tensor([0, rows - 1]),
                                  torch.randint(0, rows, (254,), generator=torch.Generator().manual_seed(9))]))
    idx_d = idx.cuda()
    x, z = d["x"][idx_d].cpu().numpy(), d["z"][idx_d].cpu().numpy()
    ref = oracle_norm(x, z, d["w"].cpu().numpy(), G, NORM_EPS)
    check(out[idx_d].cpu().numpy(), ref, f"{name} {len(idx)} rows")
    del d, out
    torch.cuda.empty_cache()
