"""SSD chunked forward benchmark on one MI355X.

A step is one full SSD forward (all kernels of the path) over one batch of
synthetic inputs already resident in HBM.  Inputs and outputs rotate over
several buffer sets whose total exceeds the 256 MB Infinity Cache, so each
step reads its inputs from HBM rather than from a cache warmed by the
previous step.

Prints ONE JSON line: whole-step throughput (tokens/s), plus
  roofline     -- the whole ssd_fwd call (every kernel it launches), timed
                  live by a HIP event pair on the launch stream around the K
                  back-to-back timed calls; achieved = algorithmic bytes /
                  the mean GPU time of one call.  A sampling phase after the
                  timed region splits a call over its kernels (``split``);
  cpu_baseline -- the oracle's recurrence on this host's cores over a bounded
                  sample (the fp32 instance; the fp64 oracle and one-thread
                  runs alongside).

``--op rmsnorm_gated`` instead times the gated grouped RMSNorm that follows
the SSD forward (page "ops-transformer MambaV2 算子套件", section 4.6) on the
configuration's output shape [B*L, H*P] with G groups: a step is one launch.
``--op ssd_bwd`` times the SSD backward (fp32; P = N = chunk = 64, so the
training-shape workload h256 by default): a step is the whole backward.
``--op causal_conv1d`` times the depthwise causal conv1d + bias + SiLU before
it (that page, §1.4 and §4.1) on [B, H*P + 2*G*N, L], or with ``--config
page`` on the page's own test shape [1, 10240, 1024]: a step is one launch.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

import torch

from workloads import (CONV_WIDTH, NORM_EPS, WORKLOADS, Workload, conv_inputs, conv_shape,
                       make_inputs, norm_inputs, norm_shape)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
METRIC = "SSD fwd ms & tokens/s at [B,L,H,P,N,chunk,G]; % of MFMA/HBM roofline"
NORM_METRIC = "gated RMSNorm ms & tokens/s at [B*L, H*P], G groups; % of HBM roofline"
FUSED_METRIC = ("SSD fwd with the gated RMSNorm fused into its epilogue, ms & tokens/s at "
                "[B,L,H,P,N,chunk,G], G norm groups; % of HBM roofline")
CONV_METRIC = "causal conv1d ms & tokens/s at [B, D, S], width 4; % of HBM roofline"
BWD_METRIC = "SSD bwd ms & tokens/s at [B,L,H,P,N,chunk,G] (fp32, P=N=chunk=64); % of fp32 roofline"
FP32_PEAK_TFLOPS = 157.3       # MI355X fp32 vector, published
# Published figure for [4,2048,16,64,128,128,4]: 0.632 ms on Ascend 910B3
# (page "Mamba-2 SSD for Ascend NPU", Benchmark table) = 4*2048/0.632e-3 tokens/s.
PAGE_TOKENS_PER_S = {"same_device": 4 * 2048 / 0.632e-3,
                     "h256": 8 * 4096 / 31.888e-3}


def quantile(v, q: float) -> float:
    """Linear-interpolated quantile of a non-empty list."""
    v = sorted(v)
    x = q * (len(v) - 1)
    i = int(math.floor(x))
    j = min(i + 1, len(v) - 1)
    return v[i] + (v[j] - v[i]) * (x - i)


def algorithmic_bytes(w: Workload, ret_final: bool = True) -> int:
    """Bytes the forward must move at least once: every input read once,
    every output written once."""
    s_io = 2 if w.io_dtype == "bf16" else 4
    T, H, P, N, G = w.tokens, w.nheads, w.headdim, w.dstate, w.ngroups
    b = T * H * P * s_io                     # x
    b += T * H * P * 4                       # out (fp32)
    b += (T * H * P * 4) if w.has_z else 0   # z (fp32)
    b += 2 * T * G * N * s_io                # B, C
    b += 4 * T * H                           # dt
    b += 4 * H * (1 + (1 if w.has_D else 0))  # A, D
    b += 4 * w.nseq * H * P * N * ((1 if ret_final else 0) + (1 if w.has_h0 else 0))
    b += 4 * (w.nseq + 1) if w.packed else 0  # cu_seqlens
    return b


def algorithmic_flops(w: Workload) -> int:
    """Dense-tile MFMA flops of the chunked form: C.B^T, M.X, C.S^T, X^T.B."""
    nc = -(-w.seqlen // w.chunk)
    Q, N, P, G, H = w.chunk, w.dstate, w.headdim, w.ngroups, w.nheads
    return 2 * w.batch * nc * (G * Q * Q * N + H * Q * Q * P + 2 * H * Q * N * P)


def measured_traffic(name: str, kernel: str = "ssd_chunk_scan_kernel",
                     record: str = "traffic.json"):
    """HBM bytes per launch of ``kernel`` on workload ``name``, measured with
    rocprofv3 counters (FETCH_SIZE + WRITE_SIZE, copy-calibrated; a record
    under profiles/), or None when the kernel source changed since the
    counters were taken."""
    import hashlib
    here = os.path.dirname(os.path.abspath(__file__))
    path = os.path.join(here, "profiles", record)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    src = os.path.join(here, rec.get("kernel_source", ""))
    if not os.path.exists(src):
        return None
    with open(src, "rb") as f:
        if hashlib.sha256(f.read()).hexdigest() != rec.get("kernel_source_sha256"):
            return None
    wl = rec.get("workloads", {}).get(name, {})
    if kernel == "ssd_fwd":
        # every kernel of one call; None unless the record lists the whole call
        if not wl.get("whole_call"):
            return None
        ks = [v for v in wl.values() if isinstance(v, dict) and "fetch_bytes" in v]
        return int(sum(k["fetch_bytes"] + k["write_bytes"] for k in ks)) if ks else None
    k = wl.get(kernel)
    return None if k is None else int(k["fetch_bytes"] + k["write_bytes"])


def kernel_list(ngroups: int) -> str:
    """The kernels one ssd_fwd call launches for a plan with `ngroups` chunk
    groups per (b, h) (the group passes only when a sequence is cut)."""
    if ngroups <= 1:
        return "ssd_chunk_scan_kernel"
    if ngroups - 1 > 8:
        return "ssd_group_state_kernel, ssd_group_passing_kernel, ssd_chunk_scan_kernel"
    return "ssd_group_state_kernel, ssd_chunk_scan_kernel"


class HipEvents:
    """Raw HIP events via the HIP runtime (recorded inside the library)."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    def create(self) -> ctypes.c_void_p:
        ev = ctypes.c_void_p()
        rc = self.hip.hipEventCreate(ctypes.byref(ev))
        if rc != 0:
            raise RuntimeError(f"hipEventCreate failed: {rc}")
        return ev

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {rc}")
        return float(ms.value)

    def record(self, ev, stream: int):
        rc = self.hip.hipEventRecord(ev, ctypes.c_void_p(stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed: {rc}")

    def destroy(self, ev):
        self.hip.hipEventDestroy(ev)


def gpu_input_set(w: Workload, seed: int, device: str):
    """One more input set drawn directly on the GPU (same distributions)."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    f32 = torch.float32
    io = torch.bfloat16 if w.io_dtype == "bf16" else f32
    Bsz, L, H, P, N, G = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups
    d = {"x": torch.randn(Bsz, L, H, P, generator=g, device=device, dtype=f32).to(io),
         "dt": torch.rand(Bsz, L, H, generator=g, device=device, dtype=f32),
         "A": -torch.rand(H, generator=g, device=device, dtype=f32),
         "B": torch.randn(Bsz, L, G, N, generator=g, device=device, dtype=f32).to(io),
         "C": torch.randn(Bsz, L, G, N, generator=g, device=device, dtype=f32).to(io)}
    d["D"] = torch.randn(H, generator=g, device=device, dtype=f32) if w.has_D else None
    d["z"] = torch.randn(Bsz, L, H, P, generator=g, device=device, dtype=f32) if w.has_z else None
    d["initial_states"] = (0.1 * torch.randn(w.nseq, H, P, N, generator=g, device=device, dtype=f32)
                           if w.has_h0 else None)
    if w.packed:
        d["cu_seqlens"] = w.cu_seqlens().to(device)
    return d


def host_cpu() -> dict:
    """The host's CPU model and the cores this process may run on."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count()
    return {"model": model, "logical_cpus": os.cpu_count(), "usable_cpus": usable}


def _time_pairs(fn, d, pairs, threads: int, budget_s: float):
    """Seconds per run of the recurrence over `pairs`, repeated until about
    `budget_s` (at least once); returns (seconds per run, repetitions)."""
    t, reps = 0.0, 0
    while reps == 0 or t + t / reps <= budget_s:
        t0 = time.perf_counter()
        fn(d["x"], d["dt"], d["A"], d["B"], d["C"], D=d["D"], z=d["z"],
           initial_states=d["initial_states"], dt_softplus=True, pairs=pairs, nthreads=threads)
        t += time.perf_counter() - t0
        reps += 1
    return t / reps, reps


def cpu_baseline(w: Workload, budget_s: float):
    """The oracle's token recurrence, as it stands, on this host's cores over a
    bounded sample of the same workload (whole (b, h) sequences), scaled to
    tokens/s of the whole workload.  ``value`` is its float instance (the
    precision of the public tensors); the fp64 oracle itself and one-thread
    runs (this workload's sample and the tiny workload) are reported
    alongside."""
    from oracle import oracle_max_threads, ssd_recurrence, ssd_recurrence_f32
    d = make_inputs(w)
    threads = oracle_max_threads()
    if w.packed:
        rec = packed_cpu_baseline(w, d, budget_s, threads)
        rec["host"] = host_cpu()
        return rec
    BH = w.batch * w.nheads
    all_pairs = [(b, h) for b in range(w.batch) for h in range(w.nheads)]
    # probe: one sequence per thread, spread over the workload
    n = min(BH, threads)
    stride = max(1, BH // n)
    t_probe, _ = _time_pairs(ssd_recurrence_f32, d, all_pairs[::stride][:n], threads, 0.0)
    share = 0.5 * budget_s                   # fp32 at full width; the rest below
    rounds = max(1, int(share / max(t_probe, 1e-9)))
    n_pairs = min(BH, rounds * n)
    pairs = all_pairs[::max(1, BH // n_pairs)][:n_pairs]
    t32, reps32 = _time_pairs(ssd_recurrence_f32, d, pairs, threads, share)
    t64, reps64 = _time_pairs(ssd_recurrence, d, pairs, threads, 0.25 * budget_s)
    scale = BH / len(pairs)
    # one thread: this workload (one sequence) and the tiny workload (whole)
    one = {}
    t1, _ = _time_pairs(ssd_recurrence_f32, d, all_pairs[:1], 1, 0.1 * budget_s)
    one[w.name] = w.tokens / (t1 * BH)
    tw = WORKLOADS["tiny"]
    dt_ = make_inputs(tw)
    tt, _ = _time_pairs(ssd_recurrence_f32, dt_, None, 1, 0.05 * budget_s)
    one["tiny"] = tw.tokens / tt
    return {"value": w.tokens / (t32 * scale), "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{len(pairs)} of {BH} (b,h) sequences of the {w.shape_str()} workload "
                      f"through the oracle's token recurrence in fp32 (its float instance), "
                      f"{reps32} repetition(s) on {threads} OpenMP threads; scaled to the whole "
                      f"workload",
            "fp64_value": w.tokens / (t64 * scale), "fp64_reps": reps64,
            "one_thread_fp32": one, "host": host_cpu()}


def calibrate(dev: str) -> dict:
    """What this GPU delivers, next to the published peaks: a 1 GiB device
    copy (torch), a 1 GiB streaming read and back-to-back fp16 MFMAs (the
    calibration kernels of libssd_calib.so), each timed with events on the
    current stream after a warm-up."""
    from mamba_ssd_chunked_04_amd.build import CALIB_LIB
    lib = ctypes.CDLL(CALIB_LIB)
    lib.ssd_calib_mfma_f16.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.ssd_calib_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int,
                                   ctypes.c_void_p]
    lib.ssd_calib_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_void_p]
    stream = torch.cuda.current_stream().cuda_stream
    nbytes = 1 << 30
    src = torch.ones(nbytes // 4, device=dev)
    dst = torch.empty_like(src)
    blocks_read, blocks_mfma, iters = 2048, 1024, 2000
    out = torch.empty(max(blocks_read, blocks_mfma) * 256, device=dev)

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps * 1e-3

    def check(rc):
        if rc != 0:
            raise RuntimeError(f"calibration kernel failed: HIP error {rc}")

    t_copy = timed(lambda: dst.copy_(src), 5)
    t_read = timed(lambda: check(lib.ssd_calib_read(src.data_ptr(), nbytes, out.data_ptr(),
                                                    blocks_read, ctypes.c_void_p(stream))), 5)
    t_mfma = timed(lambda: check(lib.ssd_calib_mfma_f16(out.data_ptr(), blocks_mfma, iters,
                                                        ctypes.c_void_p(stream))), 3)
    # the other matrix shapes: (kind, flops per wave per iteration)
    shapes = {"mfma_f16_32x32x16_tflops": (1, 4 * 2 * 32 * 32 * 16),
              "mfma_bf16_16x16x32_tflops": (2, 8 * 2 * 16 * 16 * 32),
              "mfma_f32_16x16x4_tflops": (3, 8 * 2 * 16 * 16 * 4)}
    per_shape = {}
    for key, (kind, fpw) in shapes.items():
        n_it = iters if kind != 3 else iters // 4
        t = timed(lambda: check(lib.ssd_calib_mfma(out.data_ptr(), blocks_mfma, n_it, kind,
                                                   ctypes.c_void_p(stream))), 3)
        per_shape[key] = blocks_mfma * 4 * n_it * fpw / t / 1e12
    del src, dst, out
    flops = blocks_mfma * 4 * iters * 8 * 2 * 16 * 16 * 32
    return {"hbm_copy_gbs": 2 * nbytes / t_copy / 1e9, "hbm_read_gbs": nbytes / t_read / 1e9,
            "mfma_f16_tflops": flops / t_mfma / 1e12, **per_shape,
            "how": "1 GiB device copy (read + write bytes), 1 GiB streaming read, "
                   f"{blocks_mfma} x 256-thread blocks of back-to-back MFMAs on registers "
                   "(16x16x32 fp16 with 8 accumulators per wave; also 32x32x16 fp16 with 4, "
                   "16x16x32 bf16 and 16x16x4 fp32 with 8)"}


def copy_calibration(mb: int, dev: str) -> None:
    """A plain device copy of known size, run three times: the reference
    kernel that scales the HBM byte counters."""
    if mb <= 0:
        return
    n = mb * (1 << 20) // 4
    src = torch.ones(n, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"[bench] copy calibration: {n * 4} bytes read + {n * 4} written per copy",
          file=sys.stderr, flush=True)
    del src, dst


def norm_bytes(rows: int, dim: int, gate: bool = True) -> int:
    """x, z and out once each, plus the weight."""
    return (3 if gate else 2) * 4 * rows * dim + 4 * dim


def norm_cpu_baseline(rows: int, dim: int, G: int, seed: int, budget_s: float):
    """The fp64 norm oracle on a bounded sample of rows, scaled to tokens/s."""
    from oracle import rmsnorm_gated as oracle_norm
    n = min(rows, 256)
    d = norm_inputs(n, dim, seed)
    x, z, wt = d["x"].numpy(), d["z"].numpy(), d["w"].numpy()
    reps, t = 0, 0.0
    while t < budget_s:
        t0 = time.perf_counter()
        oracle_norm(x, z, wt, G, NORM_EPS)
        t += time.perf_counter() - t0
        reps += 1
    return {"value": n * reps / t, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{n} rows of [{rows}, {dim}] (G={G}), {reps} repetition(s), {t:.1f} s of "
                      f"fp64 numpy on one thread; tokens/s = rows/s"}


def norm_main(args, w: Workload) -> int:
    import mamba_ssd_chunked_04_amd as ssd
    rows, dim, G = norm_shape(w)
    dev = "cuda:0"
    abytes = norm_bytes(rows, dim)
    n_sets = args.sets or max(1, min(16, math.ceil(2 * 512e6 / abytes)))
    print(f"[bench] gated RMSNorm after {w.name}: rows={rows} dim={dim} G={G} sets={n_sets}",
          file=sys.stderr, flush=True)
    sets = []
    for k in range(n_sets):
        d = norm_inputs(rows, dim, w.seed * 1000 + 500 + k, device=dev)
        d["out"] = torch.empty_like(d["x"])
        sets.append(d)
    stream = torch.cuda.current_stream().cuda_stream
    ev = HipEvents()

    copy_calibration(args.copy_calibration_mb, dev)

    def step(k):
        d = sets[k % n_sets]
        ssd.rmsnorm_gated(d["x"], d["z"], d["w"], G, NORM_EPS, out=d["out"])

    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    # A step is one launch, so the kernel's mean duration is taken over the
    # back-to-back launches between two events (an event pair around each
    # launch of a ~17 us kernel would add its own ~3 us to every sample).
    K = args.steps
    e0, e1 = ev.create(), ev.create()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev.record(e0, stream)
    for k in range(K):
        step(k)
    ev.record(e1, stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kmean = ev.elapsed_ms(e0, e1) / K
    ev.destroy(e0)
    ev.destroy(e1)
    achieved = abytes / (kmean * 1e-3) / 1e9
    rec = {
        "metric": NORM_METRIC,
        "value": rows / (wall / K),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": wall / K * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"gated RMSNorm after {w.name} {w.shape_str()}", "rows": rows,
                   "dim": dim, "G": G, "group_size": dim // G, "eps": NORM_EPS, "z": True,
                   "input_sets": n_sets},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": measured_traffic(w.name, "gated_rmsnorm_kernel",
                                                 "traffic_rmsnorm.json"),
                     "kernel": "gated_rmsnorm_kernel", "kernel_ms": kmean,
                     "algorithmic_bytes": abytes},
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle baseline", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = norm_cpu_baseline(rows, dim, G, w.seed, args.cpu_baseline_seconds)
    print(json.dumps(rec), flush=True)
    return 0


def fused_main(args, w: Workload) -> int:
    """The forward with the gated RMSNorm fused into its epilogue (norm groups
    = G, the chain's), against the same chain as two launches: the forward
    without the gate, then the gated RMSNorm kernel over its output."""
    import mamba_ssd_chunked_04_amd as ssd
    dev = "cuda:0"
    if args.mma == "auto":
        args.mma = "bf16" if w.io_dtype == "bf16" else "f16"
    abytes = algorithmic_bytes(w) + 4 * w.nheads * w.headdim       # + the norm weight
    n_sets = args.sets or max(1, min(16, math.ceil(2 * 512e6 / abytes)))
    print(f"[bench] fused norm after {w.name} {w.shape_str()} mma={args.mma} sets={n_sets}",
          file=sys.stderr, flush=True)
    sets = [{k: (None if v is None else v.to(dev)) for k, v in make_inputs(w).items()}]
    for k in range(1, n_sets):
        sets.append(gpu_input_set(w, w.seed * 1000 + k, dev))
    g = torch.Generator().manual_seed(w.seed + 77)
    wt = (1.0 + 0.1 * torch.randn(w.nheads * w.headdim, generator=g)).to(dev)
    rows, dim = w.tokens, w.nheads * w.headdim
    fused, sep = [], []
    for d in sets:
        kw = dict(D=d["D"], initial_states=d["initial_states"], dt_softplus=True,
                  return_final_state=True, mma=args.mma, chunks_per_wg=args.chunks_per_wg,
                  cu_seqlens=d.get("cu_seqlens"), max_seqlen=w.max_len if w.packed else None)
        call, _, _, _ = ssd.prepare(d["x"], d["dt"], d["A"], d["B"], d["C"], w.chunk, z=d["z"],
                                    norm_weight=wt, norm_eps=NORM_EPS, norm_groups=w.ngroups, **kw)
        fused.append(call)
        scall, out, _, _ = ssd.prepare(d["x"], d["dt"], d["A"], d["B"], d["C"], w.chunk, **kw)
        zv = None if d["z"] is None else d["z"].view(rows, dim)
        sep.append((scall, out.view(rows, dim), zv, torch.empty(rows, dim, device=dev)))
    stream = torch.cuda.current_stream().cuda_stream
    ev = HipEvents()
    copy_calibration(args.copy_calibration_mb, dev)

    def run_sep(k):
        scall, y, zv, nout = sep[k % n_sets]
        scall.launch(stream)
        ssd.rmsnorm_gated(y, zv, wt, w.ngroups, NORM_EPS, out=nout)

    def timed(step, K):
        for k in range(args.warmup):
            step(k)
        torch.cuda.synchronize()
        e0, e1 = ev.create(), ev.create()
        t0 = time.perf_counter()
        ev.record(e0, stream)
        for k in range(K):
            step(k)
        ev.record(e1, stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ms = ev.elapsed_ms(e0, e1) / K
        ev.destroy(e0)
        ev.destroy(e1)
        return ms, wall / K

    K = args.steps
    fused_ms, fused_wall = timed(lambda k: fused[k % n_sets].launch(stream), K)
    for c in fused:
        c.check()                     # raises if an exchange timed out
    sep_ms, _ = timed(run_sep, K)
    achieved = abytes / (fused_ms * 1e-3) / 1e9
    rec = {
        "metric": FUSED_METRIC,
        "value": w.tokens / fused_wall,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": fused_wall * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.mma,
        "data": "synthetic",
        "config": {"workload": f"{w.name} {w.shape_str()} + fused gated RMSNorm",
                   "norm_groups": w.ngroups, "group_size": dim // w.ngroups, "eps": NORM_EPS,
                   "z": w.has_z, "io_dtype": w.io_dtype, "input_sets": n_sets},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": measured_traffic(w.name + "+norm", "ssd_fwd"),
                     "kernel": "ssd_fwd with norm_weight (every kernel of one call)",
                     "kernel_ms": fused_ms, "algorithmic_bytes": abytes},
        "separate_chain": {"kernels": "ssd_fwd without the gate, then gated_rmsnorm_kernel",
                           "ms": sep_ms, "fused_speedup": sep_ms / fused_ms},
    }
    print(json.dumps(rec), flush=True)
    return 0


def packed_cpu_baseline(w: Workload, d, budget_s: float, threads: int):
    """The fp64 packed oracle (each sequence through the recurrence) over the
    whole packed workload, repeated to about ``budget_s`` seconds."""
    from oracle import ssd_varlen
    reps, t = 0, 0.0
    while t < budget_s:
        t0 = time.perf_counter()
        ssd_varlen(d["x"], d["dt"], d["A"], d["B"], d["C"], d["cu_seqlens"], D=d["D"], z=d["z"],
                   initial_states=d["initial_states"], dt_softplus=True)
        t += time.perf_counter() - t0
        reps += 1
    return {"value": w.tokens * reps / t, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"the whole packed {w.shape_str()} workload ({w.nseq} sequences), {reps} "
                      f"repetition(s), {t:.1f} s of fp64 recurrence on {threads} OpenMP threads"}


def conv_bytes(B: int, D: int, S: int, W: int) -> int:
    """x read and out written once, the taps and bias, the conv state read and
    the final state written."""
    return 8 * B * D * S + 4 * D * (W + 1) + 8 * B * D * (W - 1)


def conv_cpu_baseline(B: int, D: int, S: int, seed: int, budget_s: float):
    """The fp64 conv oracle on a bounded sample of channels, scaled to tokens/s
    (a token is one step of all B*D channels)."""
    from oracle import causal_conv1d as oracle_conv
    n = min(D, 64)
    d = conv_inputs(1, n, S, CONV_WIDTH, seed, has_state=True)
    x, wt, b, st = (d[k].numpy() for k in ("x", "w", "bias", "conv_state"))
    reps, t = 0, 0.0
    while t < budget_s:
        t0 = time.perf_counter()
        oracle_conv(x, wt, b, st)
        t += time.perf_counter() - t0
        reps += 1
    chan_steps_per_s = n * S * reps / t
    return {"value": chan_steps_per_s / D, "unit": "tokens/s", "cores": 1,
            "kind": "oracle",
            "sample": f"{n} of {B * D} channel rows of {S} steps, {reps} repetition(s), {t:.1f} s "
                      f"of fp64 numpy on one thread; scaled to B*S tokens of all D channels"}


def conv_main(args) -> int:
    import mamba_ssd_chunked_04_amd as ssd
    name = args.config
    B, D, S = conv_shape(name)
    W = CONV_WIDTH
    dev = "cuda:0"
    abytes = conv_bytes(B, D, S, W)
    n_sets = args.sets or max(1, min(16, math.ceil(2 * 512e6 / abytes)))
    print(f"[bench] causal conv1d {name}: B={B} D={D} S={S} W={W} sets={n_sets}",
          file=sys.stderr, flush=True)
    seed0 = (WORKLOADS[name].seed if name in WORKLOADS else 20269) * 1000 + 700
    tok = args.conv_layout == "tokmajor"
    sets = []
    for k in range(n_sets):
        d = conv_inputs(B, D, S, W, seed0 + k, device=dev, has_state=True)
        if tok:   # the same values, token-major [B, S, D]
            d["x"] = d["x"].transpose(1, 2).contiguous()
        d["out"] = torch.empty_like(d["x"])
        d["fin"] = torch.empty_like(d["conv_state"])
        sets.append(d)
    stream = torch.cuda.current_stream().cuda_stream
    ev = HipEvents()
    copy_calibration(args.copy_calibration_mb, dev)
    conv = ssd.causal_conv1d_tokmajor if tok else ssd.causal_conv1d
    kernel = "causal_conv1d_tok_kernel" if tok else "causal_conv1d_vec_kernel"

    def step(k):
        d = sets[k % n_sets]
        conv(d["x"], d["w"], d["bias"], d["conv_state"], out=d["out"], return_final_state=True,
             final_state=d["fin"])

    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    # one launch per step: the kernel's mean duration over the back-to-back
    # timed launches, between two events on the launch stream
    K = args.steps
    e0, e1 = ev.create(), ev.create()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev.record(e0, stream)
    for k in range(K):
        step(k)
    ev.record(e1, stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kmean = ev.elapsed_ms(e0, e1) / K
    ev.destroy(e0)
    ev.destroy(e1)
    achieved = abytes / (kmean * 1e-3) / 1e9
    rec = {
        "metric": CONV_METRIC,
        "value": B * S / (wall / K),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": wall / K * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"causal conv1d {name} [B={B}, D={D}, S={S}]"
                               + (" token-major [B, S, D]" if tok else ""), "B": B, "D": D,
                   "S": S, "W": W, "bias": True, "conv_state": True, "activation": "silu",
                   "layout": args.conv_layout, "input_sets": n_sets},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": measured_traffic(name, kernel, "traffic_conv1d.json"),
                     "kernel": kernel, "kernel_ms": kmean,
                     "algorithmic_bytes": abytes},
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle baseline", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = conv_cpu_baseline(B, D, S, seed0, args.cpu_baseline_seconds)
    print(json.dumps(rec), flush=True)
    return 0


def bwd_flops_per_chunk() -> int:
    """fp32 flops of the backward main kernel per (b, h, 64-token chunk): nine
    64x64x64 products (C B^T, dy x^T, W1^T dy, B G^T, W2^T C, x G, W2 B, dy S,
    dy^T diag C)."""
    return 9 * 2 * 64 ** 3


def bwd_main(args) -> int:
    import mamba_ssd_chunked_04_amd as ssd
    name = args.config if args.config != "same_device" else "h256"
    w = WORKLOADS[name]
    if (w.headdim, w.dstate, w.chunk) != (64, 64, 64) or w.packed or w.has_z:
        print(f"--op ssd_bwd needs P = N = chunk = 64 without z: {name} is not", file=sys.stderr)
        return 2
    dev = "cuda:0"
    print(f"[bench] SSD backward {w.name} {w.shape_str()}", file=sys.stderr, flush=True)
    copy_calibration(args.copy_calibration_mb, dev)
    d = {k: (None if v is None else v.to(dev)) for k, v in make_inputs(w).items()}
    g = torch.Generator(device=dev)
    g.manual_seed(w.seed * 1000 + 900)
    dout = torch.randn(w.batch, w.seqlen, w.nheads, 64, generator=g, device=dev)
    dfin = torch.randn(w.batch, w.nheads, 64, 64, generator=g, device=dev)
    call = ssd.prepare_bwd(d["x"], d["dt"], d["A"], d["B"], d["C"], dout, 64, D=d["D"],
                           initial_states=d["initial_states"], dfinal_state=dfin,
                           dt_softplus=True)
    stream = torch.cuda.current_stream().cuda_stream
    ev = HipEvents()
    for _ in range(args.warmup):
        call.launch(stream)
    torch.cuda.synchronize()
    K = args.steps
    evs = [(ev.create(), ev.create()) for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(K):
        call.desc.ev_main_begin, call.desc.ev_main_end = evs[k][0].value, evs[k][1].value
        call.launch(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    call.desc.ev_main_begin = call.desc.ev_main_end = None
    main_ms = [ev.elapsed_ms(a, b) for a, b in evs]
    for a, b in evs:
        ev.destroy(a)
        ev.destroy(b)
    kmean = sum(main_ms) / len(main_ms)
    nc = -(-w.seqlen // 64)
    flops = bwd_flops_per_chunk() * w.batch * w.nheads * nc
    achieved = flops / (kmean * 1e-3) / 1e12
    rec = {
        "metric": BWD_METRIC,
        "value": w.tokens / (wall / K),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": wall / K * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"SSD backward {w.name} {w.shape_str()}", "B": w.batch,
                   "L": w.seqlen, "H": w.nheads, "P": 64, "N": 64, "chunk": 64, "G": w.ngroups,
                   "D": w.has_D, "initial_state": w.has_h0, "dfinal_state": True},
        "roofline": {"bound": "alu", "achieved": achieved, "peak": FP32_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / FP32_PEAK_TFLOPS, "traffic": None,
                     "kernel": "ssd_bwd_chunk_kernel", "kernel_ms": kmean,
                     "algorithmic_flops": flops},
    }
    if not args.no_calibration:
        print("[bench] calibrating the GPU's delivered peaks", file=sys.stderr, flush=True)
        try:
            cal = calibrate(dev)
        except (OSError, RuntimeError) as e:
            cal = {"error": str(e)}
        if "mfma_f32_16x16x4_tflops" in cal:
            rec["roofline"]["calibrated"] = {
                "peak": cal["mfma_f32_16x16x4_tflops"], "unit": "TFLOP/s",
                "frac": achieved / cal["mfma_f32_16x16x4_tflops"],
                "of": "this GPU's measured back-to-back 16x16x4 fp32 MFMA rate"}
        rec["calibration"] = cal
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle baseline", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = bwd_cpu_baseline(w, args.cpu_baseline_seconds)
    print(json.dumps(rec), flush=True)
    return 0


def bwd_cpu_baseline(w: Workload, budget_s: float):
    """The fp64 autograd backward oracle on one sequence of one group's heads
    (one batch row, H/G heads) of the workload, repeated to about budget_s,
    scaled to tokens/s of the whole workload."""
    from oracle import ssd_grads
    from workloads import random_inputs
    hpg = w.nheads // w.ngroups
    L = min(w.seqlen, 512)
    d = random_inputs(1, L, hpg, 64, 64, 1, seed=w.seed, has_D=w.has_D, has_h0=w.has_h0)
    g = torch.Generator().manual_seed(5)
    dout = torch.randn(1, L, hpg, 64, generator=g)
    reps, t = 0, 0.0
    while t < budget_s:
        t0 = time.perf_counter()
        ssd_grads(d["x"], d["dt"], d["A"], d["B"], d["C"], dout, D=d["D"],
                  initial_states=d["initial_states"], dt_softplus=True)
        t += time.perf_counter() - t0
        reps += 1
    heads_tokens_per_s = hpg * L * reps / t
    return {"value": heads_tokens_per_s / w.nheads, "unit": "tokens/s",
            "cores": torch.get_num_threads(), "kind": "oracle",
            "sample": f"{L} tokens of one sequence of the {hpg} heads of one group (same "
                      f"distributions), "
                      f"{reps} repetition(s), {t:.1f} s of fp64 autograd; scaled to tokens/s "
                      f"of all {w.nheads} heads"}


def multi_process(args, argv) -> int:
    """Run bench.py in args.processes independent child processes in turn
    (the first one also times the CPU baseline and the calibration) and print
    the record of the child with the median value, with every child's value
    and per-call time under ``processes``."""
    import subprocess
    base, skip = [], False
    for a in argv:                      # drop --processes N / --processes=N
        if skip:
            skip = False
            continue
        if a == "--processes":
            skip = True
            continue
        if a.startswith("--processes="):
            continue
        base.append(a)
    recs = []
    for i in range(args.processes):
        extra = [] if i == 0 else ["--no-cpu-baseline", "--no-calibration"]
        cmd = [sys.executable, os.path.abspath(__file__), *base, *extra]
        print(f"[bench] process {i + 1} of {args.processes}", file=sys.stderr, flush=True)
        r = subprocess.run(cmd, stdout=subprocess.PIPE, text=True)
        if r.returncode != 0:
            print(f"[bench] process {i + 1} failed with exit code {r.returncode}",
                  file=sys.stderr)
            return r.returncode
        lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
        recs.append(json.loads(lines[-1]))
    order = sorted(range(len(recs)), key=lambda i: recs[i]["value"])
    med = dict(recs[order[len(order) // 2]])
    for k in ("cpu_baseline", "calibration"):
        if k in recs[0] and k not in med:
            med[k] = recs[0][k]
    if "calibrated" in recs[0].get("roofline", {}) and "calibrated" not in med["roofline"]:
        cal = dict(recs[0]["roofline"]["calibrated"])
        cal["frac"] = med["roofline"]["achieved"] / cal["peak"]
        med["roofline"] = dict(med["roofline"], calibrated=cal)
    vals = [r["value"] for r in recs]
    med["processes"] = {"n": len(recs), "values": vals,
                        "kernel_ms": [r["roofline"].get("kernel_ms") for r in recs],
                        "spread": (max(vals) - min(vals)) / med["value"],
                        "reported": "the process with the median value"}
    print(json.dumps(med), flush=True)
    return 0


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="same_device", choices=sorted(WORKLOADS) + ["page"],
                    help="workload; 'page' is the conv1d test shape of --op causal_conv1d")
    ap.add_argument("--op", default="ssd_fwd", choices=["ssd_fwd", "ssd_bwd", "rmsnorm_gated",
                                                        "causal_conv1d", "ssd_fwd_norm"],
                    help="ssd_fwd_norm: the forward with the gated RMSNorm fused into its "
                         "epilogue, timed against the forward and the norm kernel in sequence")
    ap.add_argument("--conv-layout", default="channel", choices=["channel", "tokmajor"],
                    help="--op causal_conv1d: [B, D, S] (channel) or token-major [B, S, D]")
    ap.add_argument("--mma", default="auto", choices=["auto", "f16", "bf16", "f32"],
                    help="MFMA operand precision; auto = bf16 for bf16 storage, else f16")
    ap.add_argument("--chunks-per-wg", type=int, default=0)
    ap.add_argument("--sets", type=int, default=0, help="rotating input sets (0 = auto)")
    ap.add_argument("--split-samples", type=int, default=20,
                    help="calls sampled after the timed region with event pairs around the "
                         "whole call and its main-pass kernel (the per-kernel split)")
    ap.add_argument("--cpu-baseline-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-calibration", action="store_true",
                    help="skip measuring the GPU's own copy, read and MFMA peaks")
    ap.add_argument("--copy-calibration-mb", type=int, default=0,
                    help="before warmup, run a plain device copy of this many MB three times "
                         "(a known-size reference kernel for HBM byte counters)")
    ap.add_argument("--processes", type=int, default=1,
                    help="run the measurement in this many independent processes, one after "
                         "another, and report the one with the median value (with every "
                         "process's value alongside)")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): there is no "
              f"multi-GPU path; the forward would shard over (b, h) with no exchange, or "
              f"over L with one exchange of per-span states.", file=sys.stderr)
        return 2
    if args.processes > 1:
        # before this process touches the GPU: each run is a child process
        return multi_process(args, sys.argv[1:] if argv is None else list(argv))
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2

    import mamba_ssd_chunked_04_amd as ssd
    ssd.load_library()
    torch.cuda.set_device(0)
    if args.op == "causal_conv1d":
        return conv_main(args)
    if args.op == "ssd_bwd":
        return bwd_main(args)
    if args.config not in WORKLOADS:
        print(f"--config {args.config} is a conv1d shape only", file=sys.stderr)
        return 2
    w = WORKLOADS[args.config]
    dev = "cuda:0"
    if args.op == "rmsnorm_gated":
        return norm_main(args, w)
    if args.op == "ssd_fwd_norm":
        return fused_main(args, w)
    if args.mma == "auto":
        args.mma = "bf16" if w.io_dtype == "bf16" else "f16"
    print(f"[bench] workload {w.name} {w.shape_str()} mma={args.mma}", file=sys.stderr, flush=True)

    # rotating input/output sets: total footprint > 2 x 256 MB Infinity Cache
    abytes = algorithmic_bytes(w)
    n_sets = args.sets or max(1, min(16, math.ceil(2 * 512e6 / abytes)))
    sets = [{k: (None if v is None else v.to(dev)) for k, v in make_inputs(w).items()}]
    for s in range(1, n_sets):
        sets.append(gpu_input_set(w, w.seed * 1000 + s, dev))
    ev = HipEvents()
    calls = []
    for d in sets:
        call, out, fin, wsp = ssd.prepare(d["x"], d["dt"], d["A"], d["B"], d["C"], w.chunk,
                                          D=d["D"], z=d["z"], initial_states=d["initial_states"],
                                          dt_softplus=True, return_final_state=True, mma=args.mma,
                                          chunks_per_wg=args.chunks_per_wg,
                                          cu_seqlens=d.get("cu_seqlens"),
                                          max_seqlen=w.max_len if w.packed else None)
        calls.append(call)
    cpg, ngroups = ssd.plan(calls[0].desc, w.chunk)
    stream = torch.cuda.current_stream().cuda_stream

    copy_calibration(args.copy_calibration_mb, dev)

    for k in range(args.warmup):
        calls[k % n_sets].launch(stream)
    torch.cuda.synchronize()

    # Timed region: K back-to-back calls (every launch of each call) between
    # two HIP events on the launch stream; their mean is the GPU time of one
    # whole call, which the roofline divides the algorithmic bytes by.
    K = args.steps
    e0, e1 = ev.create(), ev.create()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev.record(e0, stream)
    for k in range(K):
        calls[k % n_sets].launch(stream)
    ev.record(e1, stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    call_ms = ev.elapsed_ms(e0, e1) / K
    ev.destroy(e0)
    ev.destroy(e1)

    # Split of a call over its kernels, outside the timed region: event pairs
    # around whole calls and around their main-pass kernel (each pair costs
    # the stream a few microseconds, so these samples are not the headline).
    S = max(1, args.split_samples)
    evs = [tuple(ev.create() for _ in range(4)) for _ in range(S)]
    torch.cuda.synchronize()
    for k in range(S):
        c = calls[k % n_sets]
        a, m0, m1, b = evs[k]
        c.desc.ev_main_begin, c.desc.ev_main_end = m0.value, m1.value
        ev.record(a, stream)
        c.launch(stream)
        ev.record(b, stream)
    torch.cuda.synchronize()
    for c in calls:
        c.desc.ev_main_begin = c.desc.ev_main_end = None
    main_ms = [ev.elapsed_ms(m0, m1) for _, m0, m1, _ in evs]
    pre_ms = [ev.elapsed_ms(a, m0) for a, m0, _, _ in evs]
    one_ms = [ev.elapsed_ms(a, b) for a, _, _, b in evs]
    for e in evs:
        for x in e:
            ev.destroy(x)

    ms_per_step = wall / K * 1e3
    tok_s = w.tokens / (wall / K)
    achieved = abytes / (call_ms * 1e-3) / 1e9
    flops = algorithmic_flops(w)
    main_mean = sum(main_ms) / len(main_ms)
    rec = {
        "metric": METRIC,
        "value": tok_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": (tok_s / PAGE_TOKENS_PER_S[w.name]) if w.name in PAGE_TOKENS_PER_S else None,
        "dtype": args.mma,
        "data": "synthetic",
        "config": {"workload": f"{w.name} {w.shape_str()}", "B": w.batch, "L": w.seqlen,
                   "H": w.nheads, "P": w.headdim, "N": w.dstate, "chunk": w.chunk,
                   "G": w.ngroups, "io_dtype": w.io_dtype, "D": w.has_D, "z": w.has_z,
                   "initial_state": w.has_h0, "final_state": True,
                   "seqlens": list(w.seqlens) if w.packed else None,
                   "chunks_per_wg": cpg, "chunk_groups": ngroups, "input_sets": n_sets},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": measured_traffic(w.name, "ssd_fwd"),
                     "kernel": "ssd_fwd (every kernel of one call: " + kernel_list(ngroups) + ")",
                     "kernel_ms": call_ms,
                     "algorithmic_bytes": abytes,
                     "split": {"samples": S,
                               "main_kernel": "ssd_chunk_scan_kernel",
                               "call_ms_p20_p50_p80": [quantile(one_ms, q) for q in (0.2, 0.5, 0.8)],
                               "main_ms_p20_p50_p80": [quantile(main_ms, q) for q in (0.2, 0.5, 0.8)],
                               "main_hbm_frac": abytes / (main_mean * 1e-3) / 1e9 / HBM_PEAK_GBS,
                               "before_main_ms_p50": quantile(pre_ms, 0.5)}},
        "path": {"ms": ms_per_step, "gbs": abytes / (wall / K) / 1e9,
                 "hbm_frac": abytes / (wall / K) / 1e9 / HBM_PEAK_GBS,
                 "tflops": flops / (wall / K) / 1e12},
    }
    if not args.no_calibration:
        print("[bench] calibrating the GPU's delivered peaks", file=sys.stderr, flush=True)
        try:
            cal = calibrate(dev)
        except (OSError, RuntimeError) as e:          # library missing or a kernel refused
            cal = {"error": str(e)}
        if "hbm_read_gbs" in cal:
            rec["roofline"]["calibrated"] = {
                "peak": cal["hbm_read_gbs"], "unit": "GB/s", "frac": achieved / cal["hbm_read_gbs"],
                "of": "this GPU's measured streaming-read rate"}
        rec["calibration"] = cal
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle baseline", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = cpu_baseline(w, args.cpu_baseline_seconds)
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
