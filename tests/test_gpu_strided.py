"""The SSD forward and the token-major conv on strided views, as they leave
the input projection (page "ops-transformer MambaV2 算子套件", §1.4: one
projection row per token holds z, x, B, C and dt side by side, and the conv
runs over x, B and C before the SSD splits them).

x, B and C are column ranges of one [B, L, H*P + 2*G*N] conv output; z and
dt are column ranges of wider rows.  Each strided call must equal the call
on dense copies of the same values bit for bit (the kernels read the same
numbers and do the same arithmetic; only addresses differ) and the fp64
oracle to the parity bar: max|gpu - oracle| <= 2e-3 * max|oracle| on the
fp16-operand path, 8x that for bf16 operands, 1e-4 on the fp32 path.
"""
import sys

import numpy as np
import pytest
import torch

from oracle import causal_conv1d as oracle_conv
from oracle import ssd_recurrence
from workloads import conv_inputs, random_inputs

pytestmark = pytest.mark.gpu

TOL = {"f16": 2e-3, "bf16": 8 * 2e-3, "f32": 1e-4}


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def rel_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    assert got.shape == ref.shape and np.isfinite(got).all()
    return float(np.abs(got - ref).max() / np.abs(ref).max())


def strided_views(d, pad_x=0, pad_z=8, pad_dt=4, dtype=torch.float32):
    """Places x, B, C in one conv-output row [x | B | C | pad_x], z in the
    second half of a [z_other | z] row and dt at column 1 of a wider row;
    returns the strided GPU views and the dense GPU tensors."""
    Bsz, L, H, P = d["x"].shape
    G, N = d["B"].shape[2:]
    hp, gn = H * P, G * N
    row = torch.full((Bsz, L, hp + 2 * gn + pad_x), float("nan"), device="cuda", dtype=dtype)
    row[..., :hp] = d["x"].reshape(Bsz, L, hp).to(dtype).cuda()
    row[..., hp:hp + gn] = d["B"].reshape(Bsz, L, gn).to(dtype).cuda()
    row[..., hp + gn:hp + 2 * gn] = d["C"].reshape(Bsz, L, gn).to(dtype).cuda()
    v = {"x": row[..., :hp].view(Bsz, L, H, P),
         "B": row[..., hp:hp + gn].view(Bsz, L, G, N),
         "C": row[..., hp + gn:hp + 2 * gn].view(Bsz, L, G, N)}
    if d.get("z") is not None:
        zrow = torch.full((Bsz, L, 2 * hp + pad_z), float("nan"), device="cuda")
        zrow[..., hp + pad_z:] = d["z"].reshape(Bsz, L, hp).cuda()
        v["z"] = zrow[..., hp + pad_z:].view(Bsz, L, H, P)
    dtrow = torch.full((Bsz, L, H + pad_dt), float("nan"), device="cuda")
    dtrow[..., 1:1 + H] = d["dt"].cuda()
    v["dt"] = dtrow[..., 1:1 + H]
    dense = {k: (None if t is None else t.contiguous()) for k, t in v.items()}
    return v, dense


def call(ssd, d, v, chunk, mma, **kw):
    g = lambda k: None if d.get(k) is None else d[k].cuda()
    out, fin = ssd.ssd_fwd(v["x"], v["dt"], g("A"), v["B"], v["C"], chunk, D=g("D"), z=v.get("z"),
                           dt_bias=g("dt_bias"), initial_states=g("initial_states"),
                           dt_softplus=True, return_final_state=True, mma=mma, **kw)
    torch.cuda.synchronize()
    return out, fin


# (B, L, H, N, G, chunk, mma, io dtype)
CASES = [(2, 300, 4, 64, 2, 64, "f16", torch.float32),
         (1, 700, 4, 128, 1, 128, "f16", torch.float32),
         (2, 600, 8, 128, 2, 256, "f16", torch.float32),
         (1, 513, 4, 64, 2, 256, "bf16", torch.bfloat16),
         (2, 130, 2, 64, 1, 64, "f32", torch.float32),
         (3, 1, 4, 64, 2, 64, "f16", torch.float32)]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "_".join(map(str, c[:7])))
def test_strided_views_equal_dense_and_oracle(gpu_lib, case):
    Bsz, L, H, N, G, Q, mma, io = case
    _say(f"  strided SSD B={Bsz} L={L} H={H} N={N} G={G} Q={Q} mma={mma} io={io}")
    d = random_inputs(Bsz, L, H, 64, N, G, seed=3000 + L + Q, has_D=True, has_z=True,
                      has_h0=True, dt_bias=True)
    v, dense = strided_views(d, pad_x=8, dtype=io)   # rows of 16-byte multiples
    out_s, fin_s = call(gpu_lib, d, v, Q, mma)
    out_d, fin_d = call(gpu_lib, d, dense, Q, mma)
    assert torch.equal(out_s, out_d) and torch.equal(fin_s, fin_d)
    # the oracle sees the values as stored (bf16-rounded where io is bf16)
    xs = {k: dense[k].float().cpu() for k in ("x", "B", "C")}
    ref, ref_fin = ssd_recurrence(xs["x"], d["dt"], d["A"], xs["B"], xs["C"], D=d["D"], z=d["z"],
                                  dt_bias=d["dt_bias"], initial_states=d["initial_states"],
                                  dt_softplus=True)
    e, ef = rel_err(out_s.cpu().numpy(), ref), rel_err(fin_s.cpu().numpy(), ref_fin)
    _say(f"    out {e:.3e} final {ef:.3e} (tol {TOL[mma]:g})")
    assert e <= TOL[mma] and ef <= TOL[mma]


def test_strided_packed_sequences_equal_dense(gpu_lib):
    """Variable-length sequences packed along one token axis (cu_seqlens),
    read through strided views."""
    lens = [1, 200, 64, 333]
    T = sum(lens)
    d = random_inputs(1, T, 4, 64, 64, 2, seed=3100, has_D=True, has_z=True, has_h0=False)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device="cuda")
    v, dense = strided_views(d)
    kw = dict(cu_seqlens=cu, max_seqlen=max(lens))
    g = lambda k: None if d.get(k) is None else d[k].cuda()
    outs = []
    for t in (v, dense):
        o, f = gpu_lib.ssd_fwd(t["x"], t["dt"], g("A"), t["B"], t["C"], 128, D=g("D"), z=t["z"],
                               dt_softplus=True, return_final_state=True, **kw)
        outs.append((o, f))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    a = 0
    for i, n in enumerate(lens):
        sl = slice(a, a + n)
        ref, ref_fin = ssd_recurrence(d["x"][:, sl], d["dt"][:, sl], d["A"], d["B"][:, sl],
                                      d["C"][:, sl], D=d["D"], z=d["z"][:, sl], dt_softplus=True)
        e = rel_err(outs[0][0][:, sl].cpu().numpy(), ref)
        ef = rel_err(outs[0][1][i:i + 1].cpu().numpy(), ref_fin)
        _say(f"    sequence {i} (len {n}): out {e:.3e} final {ef:.3e}")
        assert e <= TOL["f16"] and ef <= TOL["f16"]
        a += n


# ------------------------------------------------------------ token-major conv

def conv_tok(ssd, x_tok, d, act=True, final=True, state=None, out=None):
    g = lambda k: None if d.get(k) is None else d[k].cuda()
    return ssd.causal_conv1d_tokmajor(x_tok, g("w"), g("bias"),
                                      g("conv_state") if state is None else state,
                                      activation="silu" if act else None, out=out,
                                      return_final_state=final,
                                      final_state=state if state is not None else None)


# (B, D, S, W, extra columns around x in its row)
TOK_SHAPES = [(1, 4, 1, 4, 0), (2, 8, 3, 3, 4), (1, 256, 33, 4, 0), (2, 260, 129, 2, 8),
              (1, 516, 1000, 4, 12), (3, 64, 4097, 4, 0), (1, 1024, 31, 4, 256),
              (2, 12, 2, 4, 4)]


@pytest.mark.parametrize("opts", [dict(act=True, bias=True, state=True),
                                  dict(act=False, bias=False, state=False)],
                         ids=["silu_bias_state", "plain"])
@pytest.mark.parametrize("shape", TOK_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_tokmajor_conv_matches_oracle(gpu_lib, shape, opts):
    B, D, S, W, extra = shape
    _say(f"  token-major conv1d B={B} D={D} S={S} W={W} row +{extra} {opts}")
    d = conv_inputs(B, D, S, W, seed=B * 1000 + D * 37 + S + W + 5, has_bias=opts["bias"],
                    has_state=opts["state"])
    lo = extra // 2 // 4 * 4
    row = torch.full((B, S, D + extra), float("nan"), device="cuda")
    row[..., lo:lo + D] = d["x"].transpose(1, 2).cuda()
    x_tok = row[..., lo:lo + D]
    out, fin = conv_tok(gpu_lib, x_tok, d, act=opts["act"])
    torch.cuda.synchronize()
    ref, ref_fin = oracle_conv(d["x"].numpy(), d["w"].numpy(),
                               None if d["bias"] is None else d["bias"].numpy(),
                               None if d["conv_state"] is None else d["conv_state"].numpy(),
                               activation=opts["act"])
    got = out.transpose(1, 2).cpu().double().numpy()
    scale = float(np.abs(ref).max())
    _say(f"    out: max_err/max_ref={np.abs(got - ref).max() / scale:.3e}")
    np.testing.assert_allclose(got, ref, rtol=1e-5, atol=1e-5 * scale)
    np.testing.assert_array_equal(fin.cpu().numpy(), ref_fin.astype(np.float32))


# [2, 264, 777] takes 16-step waves (a grid under two workgroups per CU),
# [4, 1024, 4100] 32-step ones (528 workgroups), with a ragged last block
@pytest.mark.parametrize("shape", [(2, 264, 777, 4), (4, 1024, 4100, 4)],
                         ids=lambda s: "x".join(map(str, s)))
def test_tokmajor_conv_equals_the_channel_major_conv(gpu_lib, shape):
    """Both layouts compute each output with the same taps in the same order:
    the results agree bit for bit."""
    B, D, S, W = shape
    _say(f"  token-major vs channel-major conv1d B={B} D={D} S={S} W={W}")
    d = conv_inputs(B, D, S, W, seed=77 + S, has_state=True)
    g = {k: v.cuda() for k, v in d.items()}
    ref, ref_fin = gpu_lib.causal_conv1d(g["x"], g["w"], g["bias"], g["conv_state"],
                                         return_final_state=True)
    out, fin = conv_tok(gpu_lib, g["x"].transpose(1, 2).contiguous(), d)
    torch.cuda.synchronize()
    assert torch.equal(out.transpose(1, 2), ref) and torch.equal(fin, ref_fin)


def test_tokmajor_decode_steps_update_the_state_in_place(gpu_lib):
    """Token-by-token and short pieces (S <= 32), each updating the conv
    state in place, equal one call over the whole sequence."""
    B, D, S, W = 2, 64, 70, 4
    d = conv_inputs(B, D, S, W, seed=78, has_state=True)
    g = {k: v.cuda() for k, v in d.items()}
    x_tok = g["x"].transpose(1, 2).contiguous()
    whole, fin_whole = conv_tok(gpu_lib, x_tok, d)
    state = g["conv_state"].clone()
    pieces = []
    for a, b in [(0, 1), (1, 2), (2, 34), (34, 35), (35, 60), (60, 70)]:
        o, _ = conv_tok(gpu_lib, x_tok[:, a:b].contiguous(), d, state=state)
        pieces.append(o)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat(pieces, dim=1), whole)
    assert torch.equal(state, fin_whole)


def test_tokmajor_rejects_bad_layouts(gpu_lib):
    d = conv_inputs(1, 8, 64, 4, seed=79, has_state=True)
    g = {k: v.cuda() for k, v in d.items()}
    x_tok = g["x"].transpose(1, 2).contiguous()
    with pytest.raises(ValueError):                  # out over x
        conv_tok(gpu_lib, x_tok, d, final=False, out=x_tok)
    with pytest.raises(ValueError):                  # in-place state beyond 32 steps
        conv_tok(gpu_lib, x_tok, d, state=g["conv_state"])
    with pytest.raises(ValueError):                  # channel-major x
        conv_tok(gpu_lib, g["x"].transpose(1, 2), d, final=False)
    d6 = conv_inputs(1, 6, 16, 4, seed=80)
    with pytest.raises(NotImplementedError):         # D not a multiple of 4
        conv_tok(gpu_lib, d6["x"].transpose(1, 2).contiguous().cuda(), d6, final=False)
