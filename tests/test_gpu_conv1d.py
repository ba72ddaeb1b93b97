"""GPU parity of the depthwise causal conv1d (ssd_causal_conv1d through the C
ABI) against the fp64 oracle, page "ops-transformer MambaV2 算子套件", §1.4
and §4.1.

Bar: |gpu - oracle| <= 1e-5 * |oracle| + 1e-5 * max|oracle| element-wise.
Each output is at most four fp32 fused multiply-adds plus the bias (error
below 5 * 2^-24 of the sum of the terms' magnitudes), then SiLU from the
hardware exp2 and reciprocal (a few ulp); the conv state is a copy and must
match bit for bit.
"""
import sys

import numpy as np
import pytest
import torch

from oracle import causal_conv1d as oracle_conv
from workloads import CONV_WIDTH, conv_inputs, conv_shape

pytestmark = pytest.mark.gpu

RTOL = ATOL_REL = 1e-5


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def check(got, ref, what):
    got = np.asarray(got, dtype=np.float64)
    assert got.shape == ref.shape and np.isfinite(got).all()
    scale = float(np.abs(ref).max()) if ref.size else 0.0
    err = float(np.abs(got - ref).max()) if ref.size else 0.0
    _say(f"    {what}: max_err/max_ref={err / (scale or 1):.3e}")
    np.testing.assert_allclose(got, ref, rtol=RTOL, atol=ATOL_REL * scale)


def np_(t):
    return None if t is None else t.cpu().numpy()


def run(ssd, d, act=True, final=True, x=None):
    g = {k: (None if v is None else v.cuda()) for k, v in d.items()}
    xg = g["x"] if x is None else x
    res = ssd.causal_conv1d(xg, g["w"], g["bias"], g["conv_state"],
                            activation="silu" if act else None, return_final_state=final)
    torch.cuda.synchronize()
    return res


# (B, D, S, W): S from one step up, multiples of 4 (vector path) and not
# (one-step path), one and several 1024-step blocks, ragged last blocks
SHAPES = [(1, 1, 1, 4), (2, 3, 2, 4), (1, 5, 3, 3), (2, 7, 4, 2), (1, 3, 5, 4), (3, 16, 64, 4),
          (2, 9, 1000, 3), (1, 8, 1024, 4), (2, 5, 1028, 4), (1, 4, 2050, 2), (1, 6, 3001, 4),
          (2, 3, 4096, 4), (1, 33, 300, 3)]


@pytest.mark.parametrize("opts", [dict(act=True, bias=True, state=True),
                                  dict(act=False, bias=False, state=False)],
                         ids=["silu_bias_state", "plain"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_random_shapes_match_oracle(gpu_lib, shape, opts):
    B, D, S, W = shape
    _say(f"  conv1d B={B} D={D} S={S} W={W} {opts}")
    d = conv_inputs(B, D, S, W, seed=B * 1000 + D * 37 + S + W, has_bias=opts["bias"],
                    has_state=opts["state"])
    out, fin = run(gpu_lib, d, act=opts["act"])
    ref, ref_fin = oracle_conv(np_(d["x"]), np_(d["w"]), np_(d["bias"]), np_(d["conv_state"]),
                               activation=opts["act"])
    check(out.cpu().numpy(), ref, "out")
    np.testing.assert_array_equal(fin.cpu().numpy(), ref_fin.astype(np.float32))


def test_misaligned_rows_take_the_step_path(gpu_lib):
    # x and out start 4 bytes past a 16-byte boundary
    B, D, S, W = 2, 5, 256, 4
    d = conv_inputs(B, D, S, W, seed=7, has_state=True)
    n = B * D * S
    xb = torch.empty(n + 1, device="cuda")
    xb[1:] = d["x"].reshape(-1).cuda()
    ob = torch.empty(n + 1, device="cuda")
    x, out = xb[1:].view(B, D, S), ob[1:].view(B, D, S)
    gpu_lib.causal_conv1d(x, d["w"].cuda(), d["bias"].cuda(), d["conv_state"].cuda(), out=out)
    torch.cuda.synchronize()
    ref, _ = oracle_conv(np_(d["x"]), np_(d["w"]), np_(d["bias"]), np_(d["conv_state"]))
    check(out.cpu().numpy(), ref, "misaligned")


def test_chunked_calls_chain_the_state_bit_identically(gpu_lib):
    """A sequence processed in pieces, each starting from the previous piece's
    final state (updated in place), equals one call on the whole."""
    B, D, S, W = 2, 6, 2048, 4
    d = conv_inputs(B, D, S, W, seed=8, has_state=True)
    g = {k: v.cuda() for k, v in d.items()}
    whole, fin_whole = gpu_lib.causal_conv1d(g["x"], g["w"], g["bias"], g["conv_state"],
                                             return_final_state=True)
    state = g["conv_state"].clone()
    pieces = []
    for a, b in [(0, 4), (4, 516), (516, 517), (517, 1536), (1536, 2048)]:
        xp = g["x"][:, :, a:b].contiguous()
        o, _ = gpu_lib.causal_conv1d(xp, g["w"], g["bias"], state, return_final_state=True,
                                     final_state=state)               # in place
        pieces.append(o)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat(pieces, dim=2), whole)
    assert torch.equal(state, fin_whole)


def test_rejects_forbidden_overlap(gpu_lib):
    d = conv_inputs(1, 2, 2048, 4, seed=9, has_state=True)
    g = {k: v.cuda() for k, v in d.items()}
    with pytest.raises(ValueError):                  # out over x
        gpu_lib.causal_conv1d(g["x"], g["w"], out=g["x"])
    with pytest.raises(ValueError):                  # in-place state with two blocks per row
        gpu_lib.causal_conv1d(g["x"], g["w"], None, g["conv_state"], return_final_state=True,
                              final_state=g["conv_state"])


@pytest.mark.parametrize("name", ["page", "same_device", "gated"])
def test_full_size(gpu_lib, name):
    """The page's test shape and the conv before two SSD workloads, at full
    size, in the launch the benchmark times."""
    B, D, S = conv_shape(name)
    _say(f"  conv1d full size {name}: B={B} D={D} S={S}")
    d = conv_inputs(B, D, S, CONV_WIDTH, seed=11, device="cuda", has_state=True)
    out, fin = gpu_lib.causal_conv1d(d["x"], d["w"], d["bias"], d["conv_state"],
                                     return_final_state=True)
    torch.cuda.synchronize()
    rows = torch.unique(torch.randint(0, B * D, (64,), generator=torch.Generator().manual_seed(3)))
    b_idx, d_idx = (rows // D).cuda(), (rows % D).cuda()
    ref, ref_fin = oracle_conv(np_(d["x"][b_idx, d_idx][None]), np_(d["w"][d_idx]),
                               np_(d["bias"][d_idx]), np_(d["conv_state"][b_idx, d_idx][None]))
    check(out[b_idx, d_idx].cpu().numpy()[None], ref, f"{name} {len(rows)} rows")
    np.testing.assert_array_equal(fin[b_idx, d_idx].cpu().numpy()[None],
                                  ref_fin.astype(np.float32))
    del d, out, fin
    torch.cuda.empty_cache()
