"""GPU parity over a seeded sweep of small random configurations.

Each case draws, from its own seed, a shape (batch, length with a ragged
tail, heads, B/C groups, state size), a chunk size, chunk groups per
workgroup, the storage dtypes of x and of B/C, the MFMA operand precision,
the output dtype, the optional inputs (D, z, initial state, dt_bias), the
discretisation (softplus or not, a dt limit) and the decay strength (the
benchmark's A = -U(0,1), or A = -U(5,10), whose steps leave the factored
intra-chunk decay for the exact per-element one), then compares out and
final_state with the fp64 oracle's token recurrence on the same stored
values.  The bar is the parity bar of test_gpu_parity.py (2e-3, 1.6e-2 and
1e-4 of max|oracle| for fp16, bf16 and fp32 operands), plus bf16's storage
rounding (2^-8) when out is bf16.

A second sweep draws configurations of the forward with the gated RMSNorm
fused into its epilogue (1 to 32 heads per norm group, every chunk size,
chunk groups split over workgroups, fp32 or bf16 storage, every operand
precision) and holds them to the propagated bound of test_gpu_norm_fused.py
against the oracle chain (the token recurrence, then the gated norm).
Two more draw packed variable-length sequences (empty, one-token and
chunk-edge lengths among them) against the per-sequence oracle, and the
backward's scope (P = N = chunk = 64, fp32) against the fp64 autograd
oracle at the backward's 1e-4 bound.
"""
import math
import sys

import numpy as np
import pytest
import torch

from oracle import ssd_recurrence
from workloads import random_inputs

pytestmark = pytest.mark.gpu

TOL = {"f16": 2e-3, "bf16": 8 * 2e-3, "f32": 1e-4}
NCASES = 120


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def draw(case: int):
    r = np.random.RandomState(70000 + case)
    pick = lambda xs: xs[r.randint(len(xs))]
    H = int(pick([1, 2, 3, 4, 6, 8]))
    G = int(pick([g for g in (1, 2, 3, 4, 8) if H % g == 0]))
    chunk = int(pick([64, 128, 256]))
    cfg = dict(
        B=int(r.randint(1, 4)), L=int(r.randint(1, 700)), H=H, G=G,
        N=int(pick([64, 128])), chunk=chunk,
        cpw=int(pick([0, 0, 1, 2, 3])),
        x_io=str(pick(["f32", "f32", "bf16"])), bc_io=str(pick(["f32", "f32", "bf16"])),
        mma=str(pick(["f16", "f16", "bf16", "f32"])),
        out_bf16=bool(r.rand() < 0.25), ret_final=bool(r.rand() < 0.8),
        D=bool(r.rand() < 0.5), z=bool(r.rand() < 0.4), h0=bool(r.rand() < 0.4),
        dt_bias=bool(r.rand() < 0.5), softplus=bool(r.rand() < 0.8),
        limit=bool(r.rand() < 0.3), strong=bool(r.rand() < 0.2),
    )
    return cfg


def inputs(case: int, c):
    d = random_inputs(c["B"], c["L"], c["H"], 64, c["N"], c["G"], seed=71000 + case,
                      has_D=c["D"], has_z=c["z"], has_h0=c["h0"], dt_bias=c["dt_bias"],
                      A_range=(5.0, 10.0) if c["strong"] else None)
    dt = {"f32": torch.float32, "bf16": torch.bfloat16}
    d["x"] = d["x"].to(dt[c["x_io"]])
    d["B"], d["C"] = d["B"].to(dt[c["bc_io"]]), d["C"].to(dt[c["bc_io"]])
    return d


def check(got, ref, tol, what):
    got = np.asarray(got, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite values"
    scale = float(np.abs(ref).max())
    err = float(np.abs(got - ref).max())
    rel = err / scale if scale > 0 else err
    _say(f"    {what}: max_err/max_ref={rel:.3e} (tol {tol:g})")
    assert rel <= tol, f"{what}: max_err/max_ref={rel:.3e} > {tol:g}"


@pytest.mark.parametrize("case", range(NCASES))
def test_random_configuration_matches_the_oracle(gpu_lib, case):
    c = draw(case)
    _say(f"[case] sweep {case}: {c}")
    d = inputs(case, c)
    limit = (0.5, 1.2) if c["limit"] else (0.0, math.inf)
    ref_out, ref_fin = ssd_recurrence(d["x"], d["dt"], d["A"], d["B"], d["C"], D=d.get("D"),
                                      z=d.get("z"), dt_bias=d.get("dt_bias"),
                                      initial_states=d.get("initial_states"),
                                      dt_softplus=c["softplus"], dt_limit=limit)
    g = {k: (None if v is None else v.cuda()) for k, v in d.items()}
    res = gpu_lib.ssd_fwd(g["x"], g["dt"], g["A"], g["B"], g["C"], c["chunk"], D=g.get("D"),
                          z=g.get("z"), dt_bias=g.get("dt_bias"),
                          initial_states=g.get("initial_states"), dt_softplus=c["softplus"],
                          dt_limit=limit, return_final_state=c["ret_final"], mma=c["mma"],
                          out_dtype=torch.bfloat16 if c["out_bf16"] else None,
                          chunks_per_wg=c["cpw"])
    torch.cuda.synchronize()
    out, fin = res if c["ret_final"] else (res, None)
    tol = TOL[c["mma"]]
    check(out.float().cpu().numpy(), ref_out, tol + (2 ** -8 if c["out_bf16"] else 0.0), "out")
    if c["ret_final"]:
        check(fin.cpu().numpy(), ref_fin, tol, "final_state")


# ------------------------------------------------------------------ fused gated RMSNorm

NNORM = 40


def draw_norm(case: int):
    """A configuration of the forward with the norm fused into its epilogue:
    k heads per norm group (at most 32, at most 16 with 256-token chunks)."""
    r = np.random.RandomState(72000 + case)
    pick = lambda xs: xs[r.randint(len(xs))]
    chunk = int(pick([64, 128, 256]))
    kmax = 16 if chunk == 256 else 32
    H = int(pick([2, 4, 6, 8, 12, 16, 32]))
    ks = [k for k in (1, 2, 3, 4, 6, 8, 16, 32) if H % k == 0 and k <= kmax]
    k = int(pick(ks))
    return dict(B=int(r.randint(1, 3)), L=int(r.randint(1, 600)), H=H, k=k,
                G=int(pick([g for g in (1, 2, 4) if H % g == 0])), N=int(pick([64, 128])),
                chunk=chunk, cpw=int(pick([0, 0, 1, 2])),
                io=str(pick(["f32", "f32", "bf16"])), mma=str(pick(["f16", "f16", "bf16", "f32"])),
                D=bool(r.rand() < 0.5), z=bool(r.rand() < 0.6), h0=bool(r.rand() < 0.4),
                dt_bias=bool(r.rand() < 0.5))


@pytest.mark.parametrize("case", range(NNORM))
def test_random_fused_norm_configuration_matches_the_oracle_chain(gpu_lib, case):
    from test_gpu_norm_fused import Chain, fused, norm_weight
    c = draw_norm(case)
    _say(f"[case] fused-norm sweep {case}: {c}")
    d = random_inputs(c["B"], c["L"], c["H"], 64, c["N"], c["G"], seed=73000 + case,
                      has_D=c["D"], has_z=c["z"], has_h0=c["h0"], io_dtype=c["io"],
                      dt_bias=c["dt_bias"])
    w = norm_weight(c["H"] * 64, 74000 + case)
    ngroups = c["H"] // c["k"]
    ref = Chain(d, w, ngroups)
    out, fin = fused(gpu_lib, d, w, ngroups, c["chunk"], mma=c["mma"], chunks_per_wg=c["cpw"])
    tol = TOL[c["mma"]]
    ref.check(out.cpu().numpy(), tol)
    check(fin.cpu().numpy(), ref.fin, tol, "final_state")


# ------------------------------------------------------------------ packed sequences

NPACK = 30


def draw_packed(case: int):
    """Packed variable-length sequences: 1 to 12 sequences of 0 to 700 tokens
    (empty and one-token ones included), every chunk size, chunk groups per
    workgroup from the plan or forced small (several groups per sequence)."""
    r = np.random.RandomState(75000 + case)
    pick = lambda xs: xs[r.randint(len(xs))]
    n = int(r.randint(1, 13))
    lens = tuple(int(pick([0, 1, 2, 63, 64, 65])) if r.rand() < 0.3 else int(r.randint(1, 700))
                 for _ in range(n))
    if sum(lens) == 0:
        lens = lens[:-1] + (5,)
    H = int(pick([2, 4, 6, 8]))
    return dict(lens=lens, H=H, G=int(pick([g for g in (1, 2, 3, 4) if H % g == 0])),
                N=int(pick([64, 128])), chunk=int(pick([64, 128, 256])),
                cpw=int(pick([0, 0, 1, 2])), mma=str(pick(["f16", "f16", "f32"])))


@pytest.mark.parametrize("case", range(NPACK))
def test_random_packed_sequences_match_the_oracle(gpu_lib, case):
    from oracle import ssd_varlen
    from workloads import packed_inputs
    c = draw_packed(case)
    _say(f"[case] packed sweep {case}: {c}")
    d = packed_inputs(c["lens"], c["H"], 64, c["N"], c["G"], seed=76000 + case, has_D=True,
                      has_z=True, has_h0=True, dt_bias=True)
    g = {k: (None if v is None else v.cuda()) for k, v in d.items()}
    out, fin = gpu_lib.ssd_fwd(g["x"], g["dt"], g["A"], g["B"], g["C"], c["chunk"], D=g["D"],
                               z=g["z"], dt_bias=g["dt_bias"], initial_states=g["initial_states"],
                               dt_softplus=True, return_final_state=True, mma=c["mma"],
                               chunks_per_wg=c["cpw"], cu_seqlens=g["cu_seqlens"])
    torch.cuda.synchronize()
    ref_o, ref_f = ssd_varlen(d["x"], d["dt"], d["A"], d["B"], d["C"], d["cu_seqlens"], D=d["D"],
                              z=d["z"], dt_bias=d["dt_bias"], initial_states=d["initial_states"],
                              dt_softplus=True)
    tol = TOL[c["mma"]]
    check(out[0].float().cpu().numpy(), ref_o, tol, "out")
    check(fin.cpu().numpy(), ref_f, tol, "final_state")


# ------------------------------------------------------------------ backward

NBWD = 12


def draw_bwd(case: int):
    """The backward's scope (P = N = chunk = 64, fp32): random batch, length,
    heads and groups, optional D, z, dt_bias, initial state and final-state
    gradient, softplus or a dt limit."""
    r = np.random.RandomState(77000 + case)
    pick = lambda xs: xs[r.randint(len(xs))]
    H = int(pick([1, 2, 4, 6]))
    return dict(B=int(r.randint(1, 3)), L=int(r.randint(1, 330)), H=H,
                G=int(pick([g for g in (1, 2, 3) if H % g == 0])),
                D=bool(r.rand() < 0.5), z=bool(r.rand() < 0.5), h0=bool(r.rand() < 0.5),
                dt_bias=bool(r.rand() < 0.5), dfin=bool(r.rand() < 0.6),
                softplus=bool(r.rand() < 0.7), limit=bool(r.rand() < 0.3))


@pytest.mark.parametrize("case", range(NBWD))
def test_random_backward_configuration_matches_the_oracle(gpu_lib, case):
    from test_gpu_bwd import NAMES, grads_both, rel_err
    c = draw_bwd(case)
    _say(f"[case] backward sweep {case}: {c}")
    d = random_inputs(c["B"], c["L"], c["H"], 64, 64, c["G"], seed=78000 + case, has_D=c["D"],
                      has_z=c["z"], has_h0=c["h0"], dt_bias=c["dt_bias"])
    gen = torch.Generator().manual_seed(79000 + case)
    dout = torch.randn(c["B"], c["L"], c["H"], 64, generator=gen)
    dfin = torch.randn(c["B"], c["H"], 64, 64, generator=gen) if c["dfin"] else None
    limit = (0.5, 1.2) if c["limit"] else (0.0, math.inf)
    got, ref = grads_both(gpu_lib, d, dout, dfin, softplus=c["softplus"], limit=limit)
    for k in NAMES:
        if ref.get(k) is None:
            assert got.get(k) is None, k
            continue
        e = rel_err(got[k].cpu().numpy(), ref[k])
        _say(f"    {k}: max_err/max_ref={e:.3e}")
        assert e <= 1e-4, f"{k}: {e:.3e} > 1e-4"
