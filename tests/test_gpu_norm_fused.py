"""GPU parity of the SSD forward with the gated RMSNorm fused into its
epilogue (page "ops-transformer MambaV2 算子套件", §4.6 mamba2_rmsnormgated,
in the chain order of its §2: chunk_scan, then rmsnormgated), against the
chain of fp64 oracles: ssd_recurrence without the gate, then rmsnorm_gated
with the gate z, the weight, the group count and eps.

Bar: the SSD's own tolerance (2e-3 on the fp16-operand path, 8x that for
bf16 operands, 1e-4 on the fp32 path) carried through the norm.  The scan
meets |dy| <= tol * max|y| on the gated output y; the norm divides token t's
group by r_t = sqrt(mean(y^2) + eps) and scales channel c by w_c, so to first
order its output moves by w_c (dy_c / r_t - y_c dr / r_t^2) with |dr| <=
max|dy|.  The test therefore bounds, element by element,
  |out - oracle| <= tol * max|y| * |w_c| / r_t * (1 + |y_c| / r_t)
                    + 2e-6 * max|oracle|
(r_t and y from the oracle; the last term is the norm's own fp32 rounding),
i.e. the fused output is the oracle's norm of a y within the scan's
tolerance.  Tokens whose group has a small root mean square get a looser
absolute bound, exactly as the norm magnifies their errors.

The heads of a norm group run in different workgroups that exchange partial
sums through the workspace; the tests cover one to 32 heads per group, chunk
groups split over several workgroups (the first pass and the fold), packed
sequences, repeated launches of one prepared call (the exchange counters
must come back to zero), graph replays and the static scratch of
ssd_fwd_noalloc.
"""
import sys

import numpy as np
import pytest
import torch

from oracle import rmsnorm_gated, ssd_recurrence
from workloads import NORM_EPS, WORKLOADS, make_inputs, random_inputs

pytestmark = pytest.mark.gpu

TOL = {"f16": 2e-3, "bf16": 8 * 2e-3, "f32": 1e-4}


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def rel_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    assert got.shape == ref.shape and np.isfinite(got).all()
    return float(np.abs(got - ref).max() / np.abs(ref).max())


def norm_weight(n, seed):
    g = torch.Generator().manual_seed(seed)
    return 1.0 + 0.25 * torch.randn(n, generator=g)


class Chain:
    """The oracle chain's output, final state and the norm's input and
    scale, for the propagated bound."""

    def __init__(self, d, w, ngroups, xs=None, Bm=None, Cm=None):
        x = d["x"] if xs is None else xs
        y, self.fin = ssd_recurrence(x, d["dt"], d["A"], d["B"] if Bm is None else Bm,
                                     d["C"] if Cm is None else Cm, D=d.get("D"),
                                     dt_bias=d.get("dt_bias"),
                                     initial_states=d.get("initial_states"), dt_softplus=True)
        Bsz, L, H, P = y.shape
        z = d.get("z")
        zz = None if z is None else np.asarray(z, dtype=np.float64).reshape(Bsz * L, H * P)
        y2 = y.reshape(Bsz * L, H * P)
        self.out = rmsnorm_gated(y2, zz, w.numpy(), ngroups, NORM_EPS).reshape(y.shape)
        g = y2 if zz is None else y2 * (zz / (1.0 + np.exp(-zz)))       # the gated y
        grouped = g.reshape(Bsz * L, ngroups, -1)
        r = np.sqrt(np.mean(grouped * grouped, axis=-1, keepdims=True) + NORM_EPS)
        self.r = np.broadcast_to(r, grouped.shape).reshape(y.shape)     # r_t per element
        self.g = np.abs(g).reshape(y.shape)
        self.ymax = float(self.g.max())
        self.w = np.broadcast_to(np.abs(w.numpy().astype(np.float64)).reshape(H, P), y.shape)

    def check(self, got, tol, what="out", sl=None):
        ref, r, w, g = self.out, self.r, self.w, self.g
        if sl is not None:
            ref, r, w, g = ref[sl], r[sl], w[sl], g[sl]
        got = np.asarray(got, dtype=np.float64)
        assert got.shape == ref.shape and np.isfinite(got).all()
        bound = tol * self.ymax * w / r * (1.0 + g / r) + 2e-6 * np.abs(ref).max()
        ratio = float((np.abs(got - ref) / bound).max())
        plain = float(np.abs(got - ref).max() / np.abs(ref).max())
        _say(f"    {what}: err/bound={ratio:.3f} (max_err/max_ref={plain:.3e}, tol {tol:g})")
        assert ratio <= 1.0


def fused(ssd, d, w, ngroups, chunk, mma="f16", **kw):
    g = {k: (None if v is None else v.cuda()) for k, v in d.items()}
    out, fin = ssd.ssd_fwd(g["x"], g["dt"], g["A"], g["B"], g["C"], chunk, D=g.get("D"),
                           z=g.get("z"), dt_bias=g.get("dt_bias"),
                           initial_states=g.get("initial_states"), dt_softplus=True,
                           return_final_state=True, mma=mma, norm_weight=w.cuda(),
                           norm_eps=NORM_EPS, norm_groups=ngroups, **kw)
    torch.cuda.synchronize()
    return out, fin


# (B, L, H, N, G, chunk, norm groups, z, D, h0, mma, io, chunks per workgroup)
CASES = [
    (2, 300, 4, 64, 2, 64, 2, True, True, False, "f16", "f32", 0),     # k = 2, ragged
    (1, 700, 8, 128, 2, 128, 2, False, True, True, "f16", "f32", 0),   # k = 4
    (2, 600, 8, 64, 1, 256, 1, True, False, False, "f16", "f32", 0),   # k = 8, 256-token chunks
    (1, 257, 4, 128, 4, 64, 4, True, True, True, "f16", "f32", 0),     # k = 1: no exchange
    (2, 513, 16, 64, 2, 128, 1, True, True, False, "f16", "f32", 0),   # k = 16
    (1, 200, 32, 64, 1, 64, 1, False, False, False, "f16", "f32", 0),  # k = 32
    (1, 513, 16, 128, 4, 256, 1, True, True, True, "f16", "f32", 0),   # k = 16 at 256
    (1, 2048, 4, 128, 1, 128, 1, True, True, True, "f16", "f32", 2),   # 8 chunk groups (fold)
    (1, 4160, 2, 64, 1, 64, 1, False, True, False, "f16", "f32", 2),   # 33 groups (passing pass)
    (2, 390, 4, 64, 2, 128, 2, True, True, True, "bf16", "bf16", 0),
    (1, 300, 4, 64, 2, 64, 1, True, True, True, "f32", "f32", 0),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "_".join(map(str, c)))
def test_fused_norm_matches_the_oracle_chain(gpu_lib, case):
    Bsz, L, H, N, G, Q, ng, has_z, has_D, has_h0, mma, io, cpg = case
    _say(f"  fused norm B={Bsz} L={L} H={H} N={N} G={G} Q={Q} norm_groups={ng} z={has_z} "
         f"D={has_D} h0={has_h0} mma={mma} io={io} cpg={cpg}")
    d = random_inputs(Bsz, L, H, 64, N, G, seed=4000 + L + H + Q, has_D=has_D, has_z=has_z,
                      has_h0=has_h0, dt_bias=True)
    if io == "bf16":
        for k in ("x", "B", "C"):
            d[k] = d[k].to(torch.bfloat16)
    w = norm_weight(H * 64, 4100 + H)
    out, fin = fused(gpu_lib, d, w, ng, Q, mma=mma, chunks_per_wg=cpg)
    f = {k: (None if d[k] is None else d[k].float()) for k in ("x", "B", "C")}
    ch = Chain(d, w, ng, xs=f["x"], Bm=f["B"], Cm=f["C"])
    ch.check(out.float().cpu().numpy(), TOL[mma])
    ef = rel_err(fin.cpu().numpy(), ch.fin)
    _say(f"    final {ef:.3e}")
    assert ef <= TOL[mma]


def test_fused_norm_bf16_output(gpu_lib):
    d = random_inputs(2, 333, 8, 64, 128, 2, seed=4200, has_D=True, has_z=True, has_h0=False)
    w = norm_weight(8 * 64, 4201)
    out, _ = fused(gpu_lib, d, w, 2, 128, out_dtype=torch.bfloat16)
    assert out.dtype == torch.bfloat16
    ch = Chain(d, w, 2)
    got = out.float().cpu().numpy()
    # the stored value is rounded to bf16 (half an ulp, 2^-9 relative) after
    # the norm: compare the rest against the bound
    slack = np.abs(ch.out) * 2.0 ** -8
    got = np.where(np.abs(got - ch.out) <= slack, ch.out, got - np.sign(got - ch.out) * slack)
    ch.check(got, TOL["f16"], "bf16 out")


def test_fused_norm_packed_sequences(gpu_lib):
    lens = [1, 300, 64, 517, 129]
    T = sum(lens)
    H, G = 8, 2
    d = random_inputs(1, T, H, 64, 64, G, seed=4300, has_D=True, has_z=True, has_h0=False)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device="cuda")
    w = norm_weight(H * 64, 4301)
    g = {k: (None if v is None else v.cuda()) for k, v in d.items()}
    out, fin = gpu_lib.ssd_fwd(g["x"], g["dt"], g["A"], g["B"], g["C"], 128, D=g["D"], z=g["z"],
                               dt_softplus=True, return_final_state=True, cu_seqlens=cu,
                               max_seqlen=max(lens), norm_weight=w.cuda(), norm_eps=NORM_EPS,
                               norm_groups=G)
    torch.cuda.synchronize()
    a = 0
    for i, n in enumerate(lens):
        sl = slice(a, a + n)
        di = {"x": d["x"][:, sl], "dt": d["dt"][:, sl], "A": d["A"], "B": d["B"][:, sl],
              "C": d["C"][:, sl], "D": d["D"], "z": d["z"][:, sl]}
        ch = Chain(di, w, G)
        ch.check(out[:, sl].cpu().numpy(), TOL["f16"], f"sequence {i} (len {n})")
        ef = rel_err(fin[i:i + 1].cpu().numpy(), ch.fin)
        assert ef <= TOL["f16"]
        a += n


def test_repeated_launches_and_graph_replays_are_identical(gpu_lib):
    """The exchange counters return to zero after every call: one prepared
    call launched eagerly several times, then captured and replayed, gives
    the same bits each time and never reports a time-out."""
    d = random_inputs(2, 640, 8, 64, 128, 2, seed=4400, has_D=True, has_z=True, has_h0=True)
    w = norm_weight(8 * 64, 4401).cuda()
    g = {k: (None if v is None else v.cuda()) for k, v in d.items()}
    call, out, fin, ws = gpu_lib.prepare(g["x"], g["dt"], g["A"], g["B"], g["C"], 128, D=g["D"],
                                         z=g["z"], initial_states=g["initial_states"],
                                         dt_softplus=True, return_final_state=True,
                                         norm_weight=w, norm_eps=NORM_EPS, norm_groups=2)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        call.launch(s.cuda_stream)
    torch.cuda.synchronize()
    call.check()
    ref = out.clone()
    for k in range(3):
        out.fill_(float("nan"))
        with torch.cuda.stream(s):
            call.launch(s.cuda_stream)
        torch.cuda.synchronize()
        call.check()
        assert torch.equal(out, ref), f"eager launch {k} differs"
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        call.launch(s.cuda_stream)
    for k in range(3):
        out.fill_(float("nan"))
        junk = torch.randn(1 << 20, device="cuda").sum()   # unrelated eager work
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        call.check()
        assert torch.equal(out, ref), f"replay {k} differs"
        del junk
    # the exchange's epoch (the workspace's first word) advanced once per
    # launch, and the count of finished workgroups is back at zero
    epoch, done = ws[:16].view(torch.int64).tolist()
    assert (epoch, done) == (7, 0)               # 4 eager launches, 3 replays


def test_noalloc_fused_equals_the_workspace_call(gpu_lib):
    d = random_inputs(2, 700, 8, 64, 128, 2, seed=4500, has_D=True, has_z=True, has_h0=False)
    w = norm_weight(8 * 64, 4501)
    ref, ref_fin = fused(gpu_lib, d, w, 2, 128)
    for _ in range(2):
        out, fin = fused(gpu_lib, d, w, 2, 128, noalloc=True)
        assert torch.equal(out, ref) and torch.equal(fin, ref_fin)


def test_fused_equals_scan_then_separate_norm(gpu_lib):
    """The fused epilogue and the separate norm kernel compute the same
    thing; their results agree to fp32 rounding."""
    d = random_inputs(2, 512, 8, 64, 128, 2, seed=4600, has_D=True, has_z=True, has_h0=True)
    w = norm_weight(8 * 64, 4601)
    out, _ = fused(gpu_lib, d, w, 2, 128)
    g = {k: (None if v is None else v.cuda()) for k, v in d.items()}
    y, _ = gpu_lib.ssd_fwd(g["x"], g["dt"], g["A"], g["B"], g["C"], 128, D=g["D"],
                           initial_states=g["initial_states"], dt_softplus=True,
                           return_final_state=True)
    sep = gpu_lib.rmsnorm_gated(y.view(-1, 8 * 64), g["z"].view(-1, 8 * 64), w.cuda(), 2, NORM_EPS)
    torch.cuda.synchronize()
    e = float((out.view(-1, 8 * 64) - sep).abs().max() / sep.abs().max())
    _say(f"    fused vs separate: {e:.3e}")
    assert e <= 1e-5


@pytest.mark.parametrize("name", ["same_device", "h256"])
def test_full_size_sampled(gpu_lib, name):
    """The fused call at a workload's full size, in the launch the benchmark
    times; one batch row's norm group (all its heads) checked against the
    oracle chain."""
    w0 = WORKLOADS[name]
    _say(f"  fused norm full size {name}: {w0.shape_str()}")
    d = make_inputs(w0, device="cuda")
    H, P, G = w0.nheads, w0.headdim, w0.ngroups
    wt = norm_weight(H * P, 4700)
    out, fin = gpu_lib.ssd_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], w0.chunk, D=d.get("D"),
                               z=d.get("z"), initial_states=d.get("initial_states"),
                               dt_softplus=True, return_final_state=True,
                               norm_weight=wt.cuda(), norm_eps=NORM_EPS, norm_groups=G)
    torch.cuda.synchronize()
    b, grp = w0.batch - 1, G // 2                   # one row, one norm group
    k = H // G
    hs = slice(grp * k, (grp + 1) * k)
    L = min(w0.seqlen, 2048)
    # norm group grp holds heads grp*k .. (grp+1)*k-1, which read B/C group grp
    sub = {"x": d["x"][b:b + 1, :L, hs].cpu(), "dt": d["dt"][b:b + 1, :L, hs].cpu(),
           "A": d["A"][hs].cpu(), "B": d["B"][b:b + 1, :L, grp:grp + 1].cpu(),
           "C": d["C"][b:b + 1, :L, grp:grp + 1].cpu(),
           "D": None if d.get("D") is None else d["D"][hs].cpu(),
           "z": None if d.get("z") is None else d["z"][b:b + 1, :L, hs].cpu(),
           "initial_states": None if d.get("initial_states") is None
           else d["initial_states"][b:b + 1, hs].cpu()}
    ch = Chain(sub, wt[grp * k * P:(grp + 1) * k * P], 1)
    ch.check(out[b:b + 1, :L, hs].float().cpu().numpy(), TOL["f16"],
             f"row {b}, heads {hs.start}..{hs.stop - 1}, {L} tokens")
    del d, out, fin
    torch.cuda.empty_cache()
