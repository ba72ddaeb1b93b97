"""GPU parity: the HIP path through the C ABI against the fp64 CPU oracle.

Bar (per output tensor): max|gpu - oracle| <= tol * max|oracle|, with
tol = 2e-3 on the fp16-operand MFMA path and 1e-4 on the all-fp32 check
path; the same bound applies to final_state against max|final_state|.
The bf16-operand path gets 8 x the fp16 bound, 1.6e-2: the same multiple
of its unit roundoff (2^-8 for bf16's 8 significant bits against 2^-11 for
fp16's 11), since every operand rounding scales with it.
NRMSE and cosine similarity are printed alongside.
"""
import math
import sys

import numpy as np
import pytest
import torch

from oracle import ssd_recurrence
from workloads import WORKLOADS, make_inputs, random_inputs

pytestmark = pytest.mark.gpu

TOL = {"f16": 2e-3, "bf16": 8 * 2e-3, "f32": 1e-4}


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def metrics(got: np.ndarray, ref: np.ndarray):
    diff = np.abs(got - ref)
    scale = float(np.abs(ref).max())
    rel = float(diff.max()) / scale if scale > 0 else float(diff.max())
    nrmse = float(np.sqrt(np.mean((got - ref) ** 2)) / (np.sqrt(np.mean(ref ** 2)) + 1e-300))
    cos = float(np.sum(got * ref) / (np.linalg.norm(got) * np.linalg.norm(ref) + 1e-300))
    return rel, nrmse, cos


def assert_close(got, ref, tol, what):
    got = np.asarray(got, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite values"
    rel, nrmse, cos = metrics(got, ref)
    _say(f"    {what}: max_err/max_ref={rel:.3e} nrmse={nrmse:.3e} cos={cos:.9f} (tol {tol:g})")
    assert rel <= tol, f"{what}: max_err/max_ref={rel:.3e} > {tol:g}"


def to_gpu(d):
    return {k: (None if v is None else v.cuda()) for k, v in d.items()}


def gpu_run(ssd, d, chunk, mma="f16", softplus=True, limit=(0.0, math.inf), chunks_per_wg=0,
            ret_final=True, out_dtype=None):
    g = to_gpu(d)
    res = ssd.ssd_fwd(g["x"], g["dt"], g["A"], g["B"], g["C"], chunk, D=g.get("D"), z=g.get("z"),
                      dt_bias=g.get("dt_bias"), initial_states=g.get("initial_states"),
                      dt_softplus=softplus, dt_limit=limit, return_final_state=ret_final, mma=mma,
                      out_dtype=out_dtype, chunks_per_wg=chunks_per_wg)
    torch.cuda.synchronize()
    if ret_final:
        out, fin = res
        return out.float().cpu().numpy(), fin.cpu().numpy()
    return res.float().cpu().numpy(), None


def oracle_run(d, softplus=True, limit=(0.0, math.inf)):
    return ssd_recurrence(d["x"], d["dt"], d["A"], d["B"], d["C"], D=d.get("D"), z=d.get("z"),
                          dt_bias=d.get("dt_bias"), initial_states=d.get("initial_states"),
                          dt_softplus=softplus, dt_limit=limit)


# (name, B, L, H, N, G, chunk, D, z, h0, dt_bias, io, limit)
SMALL = [
    ("q64_tail", 2, 300, 4, 64, 2, 64, False, False, False, False, "f32", None),
    ("q128_tail_D_h0", 1, 700, 3, 128, 1, 128, True, False, True, False, "f32", None),
    ("q256_tail_all", 2, 600, 8, 128, 2, 256, True, True, True, True, "f32", None),
    ("q64_n128_bf16", 1, 257, 4, 128, 4, 64, True, True, True, False, "bf16", None),
    ("q128_n64_limit", 2, 390, 2, 64, 1, 128, False, False, False, True, "f32", (0.8, 1.1)),
    ("q256_n64_bf16_gate", 1, 513, 4, 64, 2, 256, True, True, False, False, "bf16", None),
    # eight or more heads per B/C group: C.B^T formed once per group
    ("q64_g1_h8_tail_D_h0", 1, 300, 8, 64, 1, 64, True, False, True, False, "f32", None),
    ("q128_g1_h8_bf16_gate", 2, 400, 8, 128, 1, 128, True, True, True, True, "bf16", None),
    ("q256_g2_h16_tail", 1, 700, 16, 128, 2, 256, False, False, False, False, "f32", None),
    ("q128_h4_g2_D_h0_bias", 2, 700, 4, 128, 2, 128, True, False, True, True, "f32", None),
    ("q128_n64_bf16_limit", 1, 333, 8, 64, 2, 128, True, False, True, False, "bf16", (0.8, 1.2)),
]


@pytest.mark.parametrize("mma", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_shapes(gpu_lib, case, mma):
    name, Bsz, L, H, N, G, Q, hD, hz, hh, hb, io, limit = case
    limit = limit or (0.0, math.inf)
    _say(f"[case] {name} mma={mma} shape=[{Bsz},{L},{H},64,{N},{Q},{G}]")
    d = random_inputs(Bsz, L, H, 64, N, G, seed=100 + len(name), has_D=hD, has_z=hz, has_h0=hh,
                      io_dtype=io, dt_bias=hb)
    ref_out, ref_fin = oracle_run(d, limit=limit)
    for cpw in (0, 1, 2):
        out, fin = gpu_run(gpu_lib, d, Q, mma=mma, limit=limit, chunks_per_wg=cpw)
        assert_close(out, ref_out, TOL[mma], f"out (chunks_per_wg={cpw})")
        assert_close(fin, ref_fin, TOL[mma], f"final_state (chunks_per_wg={cpw})")


@pytest.mark.parametrize("mma", ["f16", "bf16", "f32"])
def test_tiny_workload(gpu_lib, mma):
    w = WORKLOADS["tiny"]
    _say(f"[case] tiny workload {w.shape_str()} mma={mma}")
    d = make_inputs(w)
    ref_out, ref_fin = oracle_run(d)
    out, fin = gpu_run(gpu_lib, d, w.chunk, mma=mma)
    assert_close(out, ref_out, TOL[mma], "out")
    assert_close(fin, ref_fin, TOL[mma], "final_state")


@pytest.mark.parametrize("L", [1, 5, 16, 63, 65, 129])
def test_short_and_ragged_sequences(gpu_lib, L):
    _say(f"[case] short L={L}")
    d = random_inputs(2, L, 4, 64, 64, 2, seed=300 + L, has_D=True, has_h0=True)
    ref_out, ref_fin = oracle_run(d)
    for Q in (64, 128, 256):
        out, fin = gpu_run(gpu_lib, d, Q)
        assert_close(out, ref_out, TOL["f16"], f"out Q={Q}")
        assert_close(fin, ref_fin, TOL["f16"], f"final Q={Q}")


@pytest.mark.parametrize("ngroups", [9, 10])
def test_group_chaining_either_side_of_the_fold_limit(gpu_lib, ngroups):
    """One chunk per group: 9 groups are chained inside the main pass (8
    aggregates before the last), 10 by the separate passing pass."""
    _say(f"[case] {ngroups} chunk groups")
    d = random_inputs(1, 64 * ngroups - 17, 3, 64, 128, 1, seed=700 + ngroups, has_D=True,
                      has_h0=True)
    ref_out, ref_fin = oracle_run(d)
    out, fin = gpu_run(gpu_lib, d, 64, chunks_per_wg=1)
    assert_close(out, ref_out, TOL["f16"], "out")
    assert_close(fin, ref_fin, TOL["f16"], "final_state")


def test_no_final_state_and_bf16_out(gpu_lib):
    d = random_inputs(1, 200, 2, 64, 128, 1, seed=401, has_z=True)
    ref_out, _ = oracle_run(d)
    out, fin = gpu_run(gpu_lib, d, 128, ret_final=False, out_dtype=torch.bfloat16)
    assert fin is None
    # bf16 storage adds up to 2^-9 relative rounding per element
    assert_close(out, ref_out, TOL["f16"] + 2 ** -8, "out (bf16 storage)")


@pytest.mark.parametrize("cpw", [1, 2])
def test_final_state_request_does_not_change_out(gpu_lib, cpw):
    """Without the final state the main pass skips the state work after each
    chunk group's last chunk; out is the same, bit for bit, as with the final
    state, and both match the oracle (8 groups of one chunk or 4 of two, the
    last one ragged)."""
    _say(f"[case] final state on and off, chunks_per_wg={cpw}")
    d = random_inputs(2, 900, 4, 64, 128, 2, seed=404, has_D=True, has_z=True)
    ref_out, ref_fin = oracle_run(d)
    out_f, fin = gpu_run(gpu_lib, d, 128, chunks_per_wg=cpw)
    out_n, none = gpu_run(gpu_lib, d, 128, chunks_per_wg=cpw, ret_final=False)
    assert none is None
    assert np.array_equal(out_f, out_n)
    assert_close(out_n, ref_out, TOL["f16"], f"out (chunks_per_wg={cpw})")
    assert_close(fin, ref_fin, TOL["f16"], f"final_state (chunks_per_wg={cpw})")


def test_determinism(gpu_lib):
    d = random_inputs(2, 700, 8, 64, 128, 2, seed=402, has_D=True, has_z=True, has_h0=True)
    a_out, a_fin = gpu_run(gpu_lib, d, 256, chunks_per_wg=1)
    b_out, b_fin = gpu_run(gpu_lib, d, 256, chunks_per_wg=1)
    np.testing.assert_array_equal(a_out, b_out)
    np.testing.assert_array_equal(a_fin, b_fin)


def test_guard_bands_untouched(gpu_lib):
    d = random_inputs(1, 333, 4, 64, 128, 2, seed=403, has_h0=True)
    g = to_gpu(d)
    n_out = 1 * 333 * 4 * 64
    n_fin = 1 * 4 * 64 * 128
    pad = 1024
    big = torch.full((n_out + 2 * pad,), float("nan"), device="cuda")
    bigf = torch.full((n_fin + 2 * pad,), float("nan"), device="cuda")
    out = big[pad:pad + n_out].view(1, 333, 4, 64)
    fin = bigf[pad:pad + n_fin].view(1, 4, 64, 128)
    call, _, _, _ = gpu_lib.prepare(g["x"], g["dt"], g["A"], g["B"], g["C"], 128,
                                    initial_states=g["initial_states"], dt_softplus=True,
                                    return_final_state=True, out=out, final_state=fin)
    call.launch(torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert torch.isnan(big[:pad]).all() and torch.isnan(big[pad + n_out:]).all()
    assert torch.isnan(bigf[:pad]).all() and torch.isnan(bigf[pad + n_fin:]).all()
    ref_out, ref_fin = oracle_run(d)
    assert_close(out.cpu().numpy(), ref_out, TOL["f16"], "out")
    assert_close(fin.cpu().numpy(), ref_fin, TOL["f16"], "final_state")


@pytest.mark.parametrize("N", [64, 128])
def test_workspace_reuse_and_stale_contents(gpu_lib, N):
    """Many chunk groups (one chunk each); the workspace starts as garbage and
    is then reused by calls with other inputs: nothing a call reads from it
    may depend on what an earlier call left there."""
    _say(f"[case] workspace reuse N={N}")
    d1 = random_inputs(2, 1300, 3, 64, N, 1, seed=500 + N, has_D=True, has_h0=True)
    d2 = random_inputs(2, 1300, 3, 64, N, 1, seed=600 + N, has_h0=True)
    g1, g2 = to_gpu(d1), to_gpu(d2)
    st = torch.cuda.current_stream().cuda_stream

    def prep(g, ws):
        return gpu_lib.prepare(g["x"], g["dt"], g["A"], g["B"], g["C"], 64, D=g["D"],
                               initial_states=g["initial_states"], dt_softplus=True,
                               return_final_state=True, chunks_per_wg=1, workspace=ws)

    call1, out1, fin1, ws = prep(g1, None)
    assert ws is not None and gpu_lib.plan(call1.desc, 64) == (1, 21)
    ws.fill_(255)
    ref1, ref2 = oracle_run(d1), oracle_run(d2)
    call2, out2, fin2, _ = prep(g2, ws)
    for k, (call, out, fin, ref) in enumerate([(call1, out1, fin1, ref1), (call2, out2, fin2, ref2),
                                               (call1, out1, fin1, ref1)]):
        out.fill_(float("nan"))
        call.launch(st)
        torch.cuda.synchronize()
        assert_close(out.cpu().numpy(), ref[0], TOL["f16"], f"out (call {k})")
        assert_close(fin.cpu().numpy(), ref[1], TOL["f16"], f"final_state (call {k})")


@pytest.mark.parametrize("cpw", [0, 1])
def test_graph_capture_replays_match_eager(gpu_lib, cpw):
    """One call captured in a HIP graph (the entry point allocates and
    synchronises nothing) and replayed several times with other eager work
    in between; every replay must equal the eager result bit for bit."""
    _say(f"[case] graph capture chunks_per_wg={cpw}")
    d = to_gpu(random_inputs(2, 900, 4, 64, 128, 2, seed=800 + cpw, has_D=True, has_z=True,
                             has_h0=True))
    s = torch.cuda.Stream()
    call, out, fin, ws = gpu_lib.prepare(d["x"], d["dt"], d["A"], d["B"], d["C"], 128, D=d["D"],
                                         z=d["z"], initial_states=d["initial_states"],
                                         dt_softplus=True, return_final_state=True,
                                         chunks_per_wg=cpw)
    with torch.cuda.stream(s):
        call.launch(s.cuda_stream)
    torch.cuda.synchronize()
    ref_out, ref_fin = out.clone(), fin.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call.launch(s.cuda_stream)
    for k in range(4):
        out.fill_(float("nan"))
        fin.fill_(float("nan"))
        junk = torch.randn(1 << 20, device="cuda").sum()  # unrelated eager work
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), f"replay {k}: out differs"
        assert torch.equal(fin, ref_fin), f"replay {k}: final_state differs"
        del junk


def test_largest_row_under_the_32bit_offset_limit(gpu_lib):
    """One batch row whose x and out slices are one token short of 2 GiB, the
    largest the 32-bit buffer offsets address (131071 tokens of 64 heads,
    a ragged last chunk, eight chunk groups): sampled heads, first and last,
    against the oracle, output and final state."""
    H, P, N, G, Q = 64, 64, 128, 1, 128
    L = (2 ** 31 - 1) // (H * P * 4)
    _say(f"[case] largest row [1,{L},{H},{P},{N},{Q},{G}] (x bytes {L * H * P * 4})")
    assert L * H * P * 4 < 2 ** 31 <= (L + 1) * H * P * 4
    g = torch.Generator(device="cuda").manual_seed(20260 + 99)
    x = torch.randn(1, L, H, P, device="cuda", generator=g)
    dt = torch.rand(1, L, H, device="cuda", generator=g)
    A = -torch.rand(H, device="cuda", generator=g)
    Bm = torch.randn(1, L, G, N, device="cuda", generator=g)
    Cm = torch.randn(1, L, G, N, device="cuda", generator=g)
    out, fin = gpu_lib.ssd_fwd(x, dt, A, Bm, Cm, Q, dt_softplus=True, return_final_state=True)
    torch.cuda.synchronize()
    Bc, Cc = Bm.cpu(), Cm.cpu()
    for h in (0, H - 1):
        ref_out, ref_fin = oracle_run({"x": x[:, :, h:h + 1].cpu(), "dt": dt[:, :, h:h + 1].cpu(),
                                       "A": A[h:h + 1].cpu(), "B": Bc, "C": Cc})
        assert_close(out[:, :, h:h + 1].cpu().numpy(), ref_out, TOL["f16"], f"out (h={h})")
        assert_close(fin[:, h:h + 1].cpu().numpy(), ref_fin, TOL["f16"], f"final (h={h})")
        # the last tokens, whose byte offsets are the largest of the row
        assert_close(out[:, -200:, h:h + 1].cpu().numpy(), ref_out[:, -200:], TOL["f16"],
                     f"last 200 rows (h={h})")
    del x, dt, A, Bm, Cm, out, fin
    torch.cuda.empty_cache()


def test_invalid_calls_raise(gpu_lib):
    d = to_gpu(random_inputs(1, 64, 2, 64, 64, 1, seed=404))
    with pytest.raises(NotImplementedError):
        gpu_lib.ssd_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], 32)
    with pytest.raises(ValueError):
        gpu_lib.ssd_fwd(d["x"].cpu(), d["dt"], d["A"], d["B"], d["C"], 64)


# ------------------------------------------------------------------ full-size workloads

def _pair_slice(d, b, h, H, G):
    g = h // (H // G)
    s = {"x": d["x"][b:b + 1, :, h:h + 1], "dt": d["dt"][b:b + 1, :, h:h + 1],
         "A": d["A"][h:h + 1], "B": d["B"][b:b + 1, :, g:g + 1], "C": d["C"][b:b + 1, :, g:g + 1]}
    s["D"] = None if d["D"] is None else d["D"][h:h + 1]
    s["z"] = None if d["z"] is None else d["z"][b:b + 1, :, h:h + 1]
    s["initial_states"] = None if d["initial_states"] is None else d["initial_states"][b:b + 1, h:h + 1]
    return s


@pytest.mark.parametrize("name", ["same_device", "h256", "long", "gated"])
def test_full_workload_sampled_pairs(gpu_lib, name):
    """Full-size workload in the launch configuration the benchmark times;
    the oracle recomputes a sample of (b, h) sequences end to end."""
    w = WORKLOADS[name]
    _say(f"[case] full workload {name} {w.shape_str()}")
    d = make_inputs(w)
    out, fin = gpu_run(gpu_lib, d, w.chunk)
    Bsz, H = w.batch, w.nheads
    pairs = sorted({(0, 0), (Bsz - 1, H - 1), (Bsz // 2, H // 2), (0, H - 1), (Bsz - 1, 1 % H),
                    (Bsz // 3, (2 * H) // 3)})
    for b, h in pairs:
        s = _pair_slice(d, b, h, H, w.ngroups)
        ref_out, ref_fin = oracle_run(s)
        assert_close(out[b:b + 1, :, h:h + 1], ref_out, TOL["f16"], f"out (b={b}, h={h})")
        assert_close(fin[b:b + 1, h:h + 1], ref_fin, TOL["f16"], f"final (b={b}, h={h})")
    del d, out, fin
    torch.cuda.empty_cache()


# ------------------------------------------------------------------ bf16 operands and storage

@pytest.mark.parametrize("mma", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("x_io,bc_io", [("f32", "bf16"), ("bf16", "f32")])
def test_mixed_storage_dtypes(gpu_lib, mma, x_io, bc_io):
    """x in one storage dtype, B and C in another (the descriptor's x_dtype
    and bc_dtype): the oracle reads the same stored values."""
    _say(f"[case] mixed storage x={x_io} B/C={bc_io} mma={mma}")
    d = random_inputs(2, 333, 4, 64, 128, 2, seed=1300, has_D=True, has_z=True, has_h0=True,
                      dt_bias=True)
    dt = {"f32": torch.float32, "bf16": torch.bfloat16}
    d["x"] = d["x"].to(dt[x_io])
    d["B"], d["C"] = d["B"].to(dt[bc_io]), d["C"].to(dt[bc_io])
    ref_out, ref_fin = oracle_run(d)
    for Q, cpw in ((64, 1), (128, 0), (256, 0)):
        out, fin = gpu_run(gpu_lib, d, Q, mma=mma, chunks_per_wg=cpw)
        assert_close(out, ref_out, TOL[mma], f"out Q={Q}")
        assert_close(fin, ref_fin, TOL[mma], f"final_state Q={Q}")


@pytest.mark.parametrize("scale", [1e5, 1e-5])
def test_bf16_operands_cover_magnitudes_outside_fp16(gpu_lib, scale):
    """bf16 inputs scaled by 1e5 (values and products far above fp16's 65504)
    or 1e-5 (products below fp16's smallest subnormal, 6e-8): the bf16-operand
    path keeps its bound; the fp16-operand path, whose operands must lie in
    fp16's range, overflows (1e5) or loses the products (1e-5)."""
    _say(f"[case] bf16 storage scaled by {scale:g}")
    d = random_inputs(1, 300, 4, 64, 128, 2, seed=1310, has_D=False, has_h0=False,
                      io_dtype="bf16", scale=scale)
    ref_out, ref_fin = oracle_run(d)
    for Q in (64, 128, 256):
        out, fin = gpu_run(gpu_lib, d, Q, mma="bf16")
        assert_close(out, ref_out, TOL["bf16"], f"out Q={Q} (bf16 operands)")
        assert_close(fin, ref_fin, TOL["bf16"], f"final_state Q={Q} (bf16 operands)")
    out, _ = gpu_run(gpu_lib, d, 128, mma="f16")
    if scale > 1:
        assert not np.isfinite(out).all(), "fp16 operands were expected to overflow"
    else:
        rel = float(np.abs(out - ref_out).max() / np.abs(ref_out).max())
        _say(f"    fp16 operands: max_err/max_ref={rel:.3e}")
        assert rel > 10 * TOL["f16"], "fp16 operands were expected to lose these products"


def test_gated_workload_on_bf16_operands(gpu_lib):
    """The gated bf16 workload [2,8192,128,64,128,256,8] on bf16 MFMA operands,
    in the plan the benchmark uses, with sampled (b, h) sequences."""
    w = WORKLOADS["gated"]
    _say(f"[case] gated workload {w.shape_str()} mma=bf16")
    d = make_inputs(w)
    out, fin = gpu_run(gpu_lib, d, w.chunk, mma="bf16")
    for b, h in sorted({(0, 0), (1, 127), (1, 64), (0, 17)}):
        s = _pair_slice(d, b, h, w.nheads, w.ngroups)
        ref_out, ref_fin = oracle_run(s)
        assert_close(out[b:b + 1, :, h:h + 1], ref_out, TOL["bf16"], f"out (b={b}, h={h})")
        assert_close(fin[b:b + 1, h:h + 1], ref_fin, TOL["bf16"], f"final (b={b}, h={h})")
    del d, out, fin
    torch.cuda.empty_cache()
