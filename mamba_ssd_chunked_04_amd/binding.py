"""Python binding of libssd_mi355x.so (include/ssd_mi355x.h), via ctypes.

Argument marshalling only: every step of the SSD forward runs in the HIP
kernels behind ``ssd_fwd``.  PyTorch provides device memory and the stream.
There is no CPU fallback: a missing library or a non-GPU tensor raises.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

from .build import LIB

SSD_OK, SSD_ERR_INVALID_ARG, SSD_ERR_UNSUPPORTED, SSD_ERR_WORKSPACE, SSD_ERR_LAUNCH = range(5)
SSD_F32, SSD_F16, SSD_BF16 = 0, 1, 2
SSD_MMA_F16, SSD_MMA_BF16, SSD_MMA_F32 = 0, 1, 2

# Every symbol include/ssd_mi355x.h declares.
EXPORTED_SYMBOLS = ("ssd_desc_init", "ssd_fwd_workspace_size", "ssd_fwd_plan", "ssd_fwd",
                    "ssd_fwd_noalloc", "ssd_bwd_workspace_size", "ssd_bwd", "ssd_rmsnorm_gated",
                    "ssd_causal_conv1d", "ssd_causal_conv1d_tokmajor", "ssd_status_str",
                    "ssd_abi_version")
# include/ssd_mi355x.h: SSD_FWD_NOALLOC_MAX_SCRATCH, SSD_FWD_NOALLOC_SYNC_BYTES
NOALLOC_MAX_SCRATCH = 64 << 20
NOALLOC_SYNC_BYTES = 24 << 20


class SsdDesc(ctypes.Structure):
    """Mirror of ``ssd_desc``."""
    _fields_ = [
        ("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("nheads", ctypes.c_int64),
        ("headdim", ctypes.c_int64), ("dstate", ctypes.c_int64), ("ngroups", ctypes.c_int64),
        ("x_dtype", ctypes.c_int32), ("z_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
        ("mma", ctypes.c_int32),
        ("dt_min", ctypes.c_float), ("dt_max", ctypes.c_float),
        ("z", ctypes.c_void_p), ("dt_bias", ctypes.c_void_p), ("initial_state", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
        ("chunks_per_wg", ctypes.c_int32), ("bc_dtype", ctypes.c_int32),
        ("ev_main_begin", ctypes.c_void_p), ("ev_main_end", ctypes.c_void_p),
        ("cu_seqlens", ctypes.c_void_p), ("packed_tokens", ctypes.c_int64),
        ("error_flag", ctypes.c_void_p),
        ("x_stride", ctypes.c_int64), ("bc_stride", ctypes.c_int64),
        ("z_stride", ctypes.c_int64), ("dt_stride", ctypes.c_int64),
        ("norm_weight", ctypes.c_void_p), ("norm_eps", ctypes.c_float),
        ("norm_groups", ctypes.c_int32),
    ]


class SsdError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


_lib = None


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load the HIP library (built in-tree by ``build.build_library``)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or os.environ.get("SSD_MI355X_LIB", LIB)
    if not os.path.exists(p):
        raise RuntimeError(f"HIP library {p} is missing: build it first with "
                           f"python -m mamba_ssd_chunked_04_amd.build")
    lib = ctypes.CDLL(p)
    vp, i64, c_int = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    dp = ctypes.POINTER(SsdDesc)
    lib.ssd_desc_init.argtypes = [dp, i64, i64, i64, i64, i64, i64]
    lib.ssd_desc_init.restype = None
    lib.ssd_fwd_workspace_size.argtypes = [dp, i64, ctypes.POINTER(ctypes.c_size_t)]
    lib.ssd_fwd_workspace_size.restype = c_int
    lib.ssd_fwd_plan.argtypes = [dp, i64, ctypes.POINTER(i64), ctypes.POINTER(i64)]
    lib.ssd_fwd_plan.restype = c_int
    lib.ssd_fwd.argtypes = [vp, vp, vp, vp, vp, vp, i64, c_int, c_int, vp, vp, vp, dp]
    lib.ssd_fwd.restype = c_int
    lib.ssd_fwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, i64, c_int, c_int, vp, vp, vp, dp]
    lib.ssd_fwd_noalloc.restype = c_int
    lib.ssd_rmsnorm_gated.argtypes = [vp, vp, vp, i64, i64, i64, ctypes.c_float, vp, vp]
    lib.ssd_rmsnorm_gated.restype = c_int
    lib.ssd_bwd_workspace_size.argtypes = [dp, i64, ctypes.POINTER(ctypes.c_size_t)]
    lib.ssd_bwd_workspace_size.restype = c_int
    lib.ssd_bwd.argtypes = [vp] * 6 + [i64, c_int] + [vp] * 11 + [vp, dp]
    lib.ssd_bwd.restype = c_int
    lib.ssd_causal_conv1d.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, c_int, vp, vp, vp]
    lib.ssd_causal_conv1d.restype = c_int
    lib.ssd_causal_conv1d_tokmajor.argtypes = [vp, i64, vp, vp, vp, i64, i64, i64, i64, c_int, vp,
                                               vp, vp]
    lib.ssd_causal_conv1d_tokmajor.restype = c_int
    lib.ssd_status_str.argtypes = [c_int]
    lib.ssd_status_str.restype = ctypes.c_char_p
    lib.ssd_abi_version.argtypes = []
    lib.ssd_abi_version.restype = c_int
    if path is None:
        _lib = lib
    return lib


def status_str(status: int) -> str:
    return load_library().ssd_status_str(int(status)).decode()


def _raise_for(status: int, what: str):
    if status == SSD_OK:
        return
    msg = f"{what}: {status_str(status)}"
    if status == SSD_ERR_UNSUPPORTED:
        raise NotImplementedError(msg)
    if status in (SSD_ERR_INVALID_ARG, SSD_ERR_WORKSPACE):
        raise ValueError(msg)
    raise SsdError(status, msg)


def make_desc(batch, seqlen, nheads, headdim, dstate, ngroups) -> SsdDesc:
    d = SsdDesc()
    load_library().ssd_desc_init(ctypes.byref(d), batch, seqlen, nheads, headdim, dstate, ngroups)
    return d


def workspace_size(desc: SsdDesc, chunk: int) -> int:
    n = ctypes.c_size_t(0)
    _raise_for(load_library().ssd_fwd_workspace_size(ctypes.byref(desc), int(chunk), ctypes.byref(n)),
               "ssd_fwd_workspace_size")
    return int(n.value)


def plan(desc: SsdDesc, chunk: int) -> Tuple[int, int]:
    """(chunks walked per workgroup, chunk groups per (b, h))."""
    a, b = ctypes.c_int64(0), ctypes.c_int64(0)
    _raise_for(load_library().ssd_fwd_plan(ctypes.byref(desc), int(chunk), ctypes.byref(a),
                                           ctypes.byref(b)), "ssd_fwd_plan")
    return int(a.value), int(b.value)


def _dtype_code(t) -> int:
    import torch
    return {torch.float32: SSD_F32, torch.bfloat16: SSD_BF16, torch.float16: SSD_F16}[t]


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _token_stride(t, name: str) -> int:
    """Elements between consecutive tokens of a [B, L, ...] tensor whose
    per-token dims are dense and whose batch rows lie L tokens apart (a
    column range of wider token-major rows, such as x, B or C inside a conv
    output); 0 when the tensor is contiguous."""
    if t.is_contiguous():
        return 0
    shp, st = t.shape, t.stride()
    expect = 1
    for dim in range(t.dim() - 1, 1, -1):
        if shp[dim] != 1 and st[dim] != expect:
            raise ValueError(f"{name}: the dims after the token dim must be dense")
        expect *= shp[dim]
    # a size-1 axis carries no stride of its own: with one token per row the
    # batch stride is the token stride
    ts = st[1] if shp[1] > 1 else (st[0] if shp[0] > 1 else expect)
    if ts < expect or (shp[0] > 1 and st[0] != shp[1] * ts):
        raise ValueError(f"{name}: tokens must be at least one row apart and batch rows "
                         f"L tokens apart")
    return int(ts)


class SsdCall:
    """One prepared ``ssd_fwd`` call over fixed tensors (for repeated launches).

    Built by ``prepare``; ``launch(stream)`` enqueues the kernels on the given
    stream handle (an int from ``torch.cuda.Stream.cuda_stream``).
    """

    def __init__(self, args, desc: SsdDesc, keep, error_flag=None, noalloc: bool = False):
        self._args = args
        self.desc = desc
        self._keep = keep        # tensors whose storage the pointers refer to
        self.error_flag = error_flag   # packed or fused-norm calls: the device flag the kernels set
        self.noalloc = noalloc   # launch through ssd_fwd_noalloc

    def launch(self, stream: int) -> None:
        if self.noalloc:
            self.launch_noalloc(stream)
            return
        a = self._args
        st = load_library().ssd_fwd(a[0], a[1], a[2], a[3], a[4], a[5], a[6], a[7], a[8], a[9],
                                    a[10], ctypes.c_void_p(stream), ctypes.byref(self.desc))
        _raise_for(st, "ssd_fwd")

    def launch_noalloc(self, stream: int) -> None:
        """The same call through ``ssd_fwd_noalloc`` (the library's static
        scratch instead of this call's workspace, which is not read)."""
        a = self._args
        st = load_library().ssd_fwd_noalloc(a[0], a[1], a[2], a[3], a[4], a[5], a[6], a[7], a[8],
                                            a[9], a[10], ctypes.c_void_p(stream),
                                            ctypes.byref(self.desc))
        _raise_for(st, "ssd_fwd_noalloc")

    def check(self) -> None:
        """Packed or fused-norm calls: synchronise and raise if any launch of
        this call set the device flag -- ValueError when cu_seqlens broke its
        contract (a sequence longer than max_seqlen, decreasing offsets or one
        past the packed tokens), SsdError when the fused norm's exchange
        between workgroups timed out (the workspace's synchronisation words
        are then zeroed again here); the flag is then cleared.  A no-op for
        other calls."""
        if self.error_flag is None:
            return
        v = int(self.error_flag.item())
        if v == 0:
            return
        self.error_flag.zero_()
        if v == 2:
            ws = self._keep[11]
            if ws is not None:
                ws.zero_()
            raise SsdError(SSD_ERR_LAUNCH, "ssd_fwd: the fused norm's exchange between "
                           "workgroups timed out; `out` is undefined")
        raise ValueError("ssd_fwd: cu_seqlens breaks the call's contract (a sequence longer "
                         "than max_seqlen, decreasing offsets or an offset past the packed "
                         "tokens); the results of those sequences are undefined")


def prepare(x, dt, A, B, C, chunk_size: int, D=None, z=None, dt_bias=None, initial_states=None,
            dt_softplus: bool = False, dt_limit: Tuple[float, float] = (0.0, math.inf),
            return_final_state: bool = False, mma: str = "f16", out_dtype=None,
            chunks_per_wg: int = 0, out=None, final_state=None, workspace=None,
            cu_seqlens=None, max_seqlen: Optional[int] = None, noalloc: bool = False,
            norm_weight=None, norm_eps: float = 1e-5, norm_groups: Optional[int] = None):
    """Validate torch tensors, allocate outputs/workspace, and build an SsdCall.

    With ``norm_weight`` ([H*P] float32) the gated RMSNorm that follows the
    scan is fused into its epilogue: out = rmsnorm(y) * norm_weight over
    ``norm_groups`` groups of each token's H*P channels (default: G), where y
    already carries D and the z gate.  The workspace is then allocated zeroed
    (it holds the exchange's synchronisation words); a caller-given one must
    be zeroed before its first fused call.

    With ``noalloc`` no workspace is allocated and the call launches through
    ``ssd_fwd_noalloc`` (the library's static scratch; ValueError from the
    launch when the plan needs more than NOALLOC_MAX_SCRATCH bytes).

    ``out`` is float32 unless ``out_dtype`` (float32 or bfloat16) says
    otherwise, whatever the dtype of x, B and C.

    x, B, C, z and dt may be token-strided views (dense per-token dims,
    batch rows L tokens apart), read in place -- e.g. x, B and C as column
    ranges of one token-major conv output [B, L, H*P + 2*G*N]; the other
    tensors must be contiguous.

    Packed variable-length sequences: x [1, T, H, P] (dt [1, T, H], B/C
    [1, T, G, N], z like x) with ``cu_seqlens`` an int32 GPU tensor of
    nseq+1 token offsets; initial and final states are then [nseq, H, P, N].
    ``max_seqlen`` (the longest sequence) is read from cu_seqlens when not
    given, which synchronises with the device and checks the offsets (0
    first, never decreasing, T last; ValueError otherwise).  When it is
    given nothing is read: offsets that break the contract are reported by
    the kernels through a device flag, which ``call.check()`` reads.
    Returns (call, out, final_state_or_None, workspace_or_None).
    """
    import torch
    for name, t in (("x", x), ("dt", dt), ("A", A), ("B", B), ("C", C)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
    dev = x.device
    Bsz, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    nrows, row_len = Bsz, L                     # batch rows of the call and their length
    if cu_seqlens is not None:
        if Bsz != 1:
            raise ValueError("packed sequences take x of shape [1, T, H, P]")
        if (not isinstance(cu_seqlens, torch.Tensor) or cu_seqlens.device != dev
                or cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1
                or cu_seqlens.numel() < 2 or not cu_seqlens.is_contiguous()):
            raise ValueError("cu_seqlens must be a contiguous int32 tensor of nseq+1 offsets "
                             "on the GPU of x")
        nrows = cu_seqlens.numel() - 1
        if max_seqlen is None:
            # reading the offsets synchronises anyway: check them whole here
            cu = cu_seqlens.cpu()
            lens = cu[1:] - cu[:-1]
            if int(cu[0]) != 0 or bool((lens < 0).any()) or int(cu[-1]) != L:
                raise ValueError(f"cu_seqlens must start at 0, never decrease and end at the "
                                 f"packed token count {L}")
            max_seqlen = int(lens.max())
        elif int(max_seqlen) < 1:
            raise ValueError("max_seqlen must be >= 1")
        row_len = max(1, int(max_seqlen))
    if dt.shape != (Bsz, L, H) or A.shape != (H,) or B.shape != (Bsz, L, G, N) or C.shape != B.shape:
        raise ValueError("shape mismatch: x[B,L,H,P], dt[B,L,H], A[H], B/C[B,L,G,N]")
    if C.dtype != B.dtype:
        raise ValueError("B and C must share one dtype")
    for name, t in (("dt", dt), ("A", A), ("D", D), ("dt_bias", dt_bias),
                    ("initial_states", initial_states)):
        if t is not None and t.dtype != torch.float32:
            raise ValueError(f"{name} must be float32")
    opt_shapes = (("D", D, (H,)), ("dt_bias", dt_bias, (H,)), ("z", z, (Bsz, L, H, P)),
                  ("initial_states", initial_states, (nrows, H, P, N)))
    for name, t, shp in opt_shapes:
        if t is not None and tuple(t.shape) != shp:
            raise ValueError(f"{name} must have shape {shp}")
    tensors = [x, dt, A, B, C, D, z, dt_bias, initial_states]
    for t in tensors:
        if t is not None and t.device != dev:
            raise ValueError("all tensors must be on the same GPU")
    # x, B, C, z and dt may be token-strided views; the rest dense
    strides = {"x": _token_stride(x, "x"), "B": _token_stride(B, "B"), "C": _token_stride(C, "C"),
               "z": _token_stride(z, "z") if z is not None else 0, "dt": _token_stride(dt, "dt")}
    bc_dense = G * N
    if (strides["B"] or bc_dense) != (strides["C"] or bc_dense):
        raise ValueError("B and C must have the same token stride")
    for t in (A, D, dt_bias, initial_states):
        if t is not None and not t.is_contiguous():
            raise ValueError("A, D, dt_bias and initial_states must be contiguous")
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty(Bsz, L, H, P, device=dev, dtype=out_dtype)
    if return_final_state and final_state is None:
        final_state = torch.empty(nrows, H, P, N, device=dev, dtype=torch.float32)
    desc = make_desc(nrows, row_len, H, P, N, G)
    error_flag = None
    if cu_seqlens is not None or norm_weight is not None:
        error_flag = torch.zeros(1, device=dev, dtype=torch.int32)
        desc.error_flag = error_flag.data_ptr()
    if cu_seqlens is not None:
        desc.cu_seqlens = cu_seqlens.data_ptr()
        desc.packed_tokens = L
    if norm_weight is not None:
        if (not isinstance(norm_weight, torch.Tensor) or norm_weight.device != dev
                or norm_weight.dtype != torch.float32 or tuple(norm_weight.shape) != (H * P,)
                or not norm_weight.is_contiguous()):
            raise ValueError("norm_weight must be a contiguous float32 [H*P] tensor on the GPU of x")
        desc.norm_weight = norm_weight.data_ptr()
        desc.norm_eps = float(norm_eps)
        desc.norm_groups = int(G if norm_groups is None else norm_groups)
    desc.x_dtype = _dtype_code(x.dtype)
    desc.bc_dtype = _dtype_code(B.dtype)
    desc.z_dtype = _dtype_code(z.dtype) if z is not None else SSD_F32
    desc.out_dtype = _dtype_code(out.dtype)
    if mma not in ("f16", "bf16", "f32"):
        raise ValueError(f"mma must be 'f16', 'bf16' or 'f32', got {mma!r}")
    desc.mma = {"f16": SSD_MMA_F16, "bf16": SSD_MMA_BF16, "f32": SSD_MMA_F32}[mma]
    desc.dt_min, desc.dt_max = float(dt_limit[0]), float(dt_limit[1])
    desc.z, desc.dt_bias, desc.initial_state = _ptr(z), _ptr(dt_bias), _ptr(initial_states)
    desc.chunks_per_wg = int(chunks_per_wg)
    desc.x_stride, desc.z_stride, desc.dt_stride = strides["x"], strides["z"], strides["dt"]
    desc.bc_stride = strides["B"] or strides["C"]
    nbytes = workspace_size(desc, chunk_size)
    if nbytes > 0 and workspace is None and not noalloc:
        alloc = torch.zeros if norm_weight is not None else torch.empty
        workspace = alloc(nbytes, device=dev, dtype=torch.uint8)
    if workspace is not None:
        desc.workspace, desc.workspace_bytes = workspace.data_ptr(), workspace.numel()
    args = (_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), int(chunk_size),
            int(bool(dt_softplus)), int(bool(return_final_state)), _ptr(out),
            _ptr(final_state) if return_final_state else None)
    keep = (x, dt, A, B, C, D, z, dt_bias, initial_states, out, final_state, workspace, cu_seqlens,
            error_flag, norm_weight)
    return (SsdCall(args, desc, keep, error_flag, noalloc=noalloc), out,
            (final_state if return_final_state else None), workspace)


def ssd_fwd(x, dt, A, B, C, chunk_size: int, D=None, z=None, dt_bias=None, initial_states=None,
            dt_softplus: bool = False, dt_limit: Tuple[float, float] = (0.0, math.inf),
            return_final_state: bool = False, mma: str = "f16", out_dtype=None,
            chunks_per_wg: int = 0, cu_seqlens=None, max_seqlen: Optional[int] = None,
            check_offsets: bool = True, noalloc: bool = False, norm_weight=None,
            norm_eps: float = 1e-5, norm_groups: Optional[int] = None):
    """SSD chunked forward on the current torch stream.

    Returns ``out`` or ``(out, final_state)`` when ``return_final_state``.
    With ``cu_seqlens`` the call runs packed variable-length sequences (see
    ``prepare``); when ``max_seqlen`` is given, ``check_offsets`` (default
    True) synchronises after the launch and raises ValueError if a sequence
    was longer than it (or the offsets were malformed).  Pass
    ``check_offsets=False`` to skip that synchronisation (then nothing
    reports such offsets; ``prepare`` and ``call.check()`` give control over
    when the check runs).  ``noalloc`` runs it through ``ssd_fwd_noalloc``
    (no workspace; the outputs are still allocated here unless the caller
    uses ``prepare`` with its own).  ``norm_weight`` fuses the gated RMSNorm
    into the epilogue (see ``prepare``); ``check_offsets`` then also
    synchronises to report a timed-out exchange.
    """
    import torch
    call, out, fin, _ws = prepare(x, dt, A, B, C, chunk_size, D=D, z=z, dt_bias=dt_bias,
                                  initial_states=initial_states, dt_softplus=dt_softplus,
                                  dt_limit=dt_limit, return_final_state=return_final_state,
                                  mma=mma, out_dtype=out_dtype, chunks_per_wg=chunks_per_wg,
                                  cu_seqlens=cu_seqlens, max_seqlen=max_seqlen, noalloc=noalloc,
                                  norm_weight=norm_weight, norm_eps=norm_eps,
                                  norm_groups=norm_groups)
    with torch.cuda.device(x.device):
        call.launch(torch.cuda.current_stream(x.device).cuda_stream)
        if check_offsets and ((cu_seqlens is not None and max_seqlen is not None)
                              or norm_weight is not None):
            call.check()
    return (out, fin) if return_final_state else out


def rmsnorm_gated(x, z, weight, ngroups: int, eps: float = 1e-5, out=None):
    """Gated grouped RMSNorm over the last dimension on the current torch stream.

    x, z: [..., D] float32 GPU tensors (z may be None: no gate); weight: [D].
    Returns ``out`` (allocated unless given; it may be ``x`` for in-place).
    """
    import torch
    for name, t in (("x", x), ("weight", weight)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
    D = x.shape[-1]
    if weight.shape != (D,) or (z is not None and z.shape != x.shape):
        raise ValueError("shape mismatch: x[..., D], z like x, weight[D]")
    if out is None:
        out = torch.empty_like(x)
    for t in (x, z, weight, out):
        if t is None:
            continue
        if t.dtype != torch.float32 or t.device != x.device or not t.is_contiguous():
            raise ValueError("x, z, weight and out must be contiguous float32 on one GPU")
    if out.shape != x.shape:
        raise ValueError("out must have the shape of x")
    rows = x.numel() // D if D else 0
    with torch.cuda.device(x.device):
        st = torch.cuda.current_stream(x.device).cuda_stream
        _raise_for(load_library().ssd_rmsnorm_gated(_ptr(x), _ptr(z), _ptr(weight), rows, D,
                                                    int(ngroups), float(eps), _ptr(out),
                                                    ctypes.c_void_p(st)), "ssd_rmsnorm_gated")
    return out


def causal_conv1d(x, weight, bias=None, conv_state=None, activation: str = "silu", out=None,
                  return_final_state: bool = False, final_state=None):
    """Depthwise causal conv1d (+ bias, + SiLU) over the last axis, on the
    current torch stream.

    x: [B, D, S] float32 GPU tensor; weight: [D, W] (W in 2..4); bias: [D]
    or None; conv_state: [B, D, W-1] steps before t = 0, or None (zeros).
    Returns ``out``, or ``(out, final_state)`` with ``return_final_state``
    (``final_state`` may be ``conv_state`` itself when S <= 1024).
    """
    import torch
    if not isinstance(x, torch.Tensor) or not x.is_cuda or x.dim() != 3:
        raise ValueError("x must be a [B, D, S] GPU tensor")
    Bsz, D, S = x.shape
    if weight.dim() != 2 or weight.shape[0] != D:
        raise ValueError("weight must be [D, W]")
    W = weight.shape[1]
    if activation not in ("silu", "none", None):
        raise ValueError(f"activation must be 'silu' or None, got {activation!r}")
    act = 1 if activation == "silu" else 0
    if out is None:
        out = torch.empty_like(x)
    if return_final_state and final_state is None:
        final_state = torch.empty(Bsz, D, W - 1, device=x.device, dtype=torch.float32)
    shapes = ((bias, (D,)), (conv_state, (Bsz, D, W - 1)), (out, (Bsz, D, S)),
              (final_state if return_final_state else None, (Bsz, D, W - 1)))
    for t, shp in shapes:
        if t is not None and tuple(t.shape) != shp:
            raise ValueError(f"expected shape {shp}, got {tuple(t.shape)}")
    for t in (x, weight, bias, conv_state, out, final_state):
        if t is None:
            continue
        if t.dtype != torch.float32 or t.device != x.device or not t.is_contiguous():
            raise ValueError("all tensors must be contiguous float32 on the GPU of x")
    with torch.cuda.device(x.device):
        st = torch.cuda.current_stream(x.device).cuda_stream
        _raise_for(load_library().ssd_causal_conv1d(
            _ptr(x), _ptr(weight), _ptr(bias), _ptr(conv_state), Bsz, D, S, W, act, _ptr(out),
            _ptr(final_state) if return_final_state else None, ctypes.c_void_p(st)),
            "ssd_causal_conv1d")
    return (out, final_state) if return_final_state else out


def causal_conv1d_tokmajor(x, weight, bias=None, conv_state=None, activation: str = "silu",
                           out=None, return_final_state: bool = False, final_state=None):
    """The same conv over token-major x: [B, S, D] float32 GPU tensor whose
    channels are contiguous and whose batches are S token rows apart (a
    column range x = proj[..., a:a + D] of a wider [B, S, *] tensor is
    taken as it is, without a copy).  out: [B, S, D] dense; weight, bias and
    conv_state as for causal_conv1d (``final_state`` may be ``conv_state``
    itself when S <= 32).
    """
    import torch
    if not isinstance(x, torch.Tensor) or not x.is_cuda or x.dim() != 3:
        raise ValueError("x must be a [B, S, D] GPU tensor")
    Bsz, S, D = x.shape
    if x.dtype != torch.float32:
        raise ValueError("x must be float32")
    # token row stride (a size-1 axis carries no stride of its own)
    xs = x.stride(1) if S > 1 else (x.stride(0) if Bsz > 1 else D)
    if (D > 1 and x.stride(2) != 1) or (Bsz > 1 and x.stride(0) != S * xs):
        raise ValueError("x must have contiguous channels and batches S token rows apart")
    if weight.dim() != 2 or weight.shape[0] != D:
        raise ValueError("weight must be [D, W]")
    W = weight.shape[1]
    if activation not in ("silu", "none", None):
        raise ValueError(f"activation must be 'silu' or None, got {activation!r}")
    act = 1 if activation == "silu" else 0
    if out is None:
        out = torch.empty(Bsz, S, D, device=x.device, dtype=torch.float32)
    if return_final_state and final_state is None:
        final_state = torch.empty(Bsz, D, W - 1, device=x.device, dtype=torch.float32)
    shapes = ((bias, (D,)), (conv_state, (Bsz, D, W - 1)), (out, (Bsz, S, D)),
              (final_state if return_final_state else None, (Bsz, D, W - 1)))
    for t, shp in shapes:
        if t is not None and tuple(t.shape) != shp:
            raise ValueError(f"expected shape {shp}, got {tuple(t.shape)}")
    for t in (weight, bias, conv_state, out, final_state):
        if t is None:
            continue
        if t.dtype != torch.float32 or t.device != x.device or not t.is_contiguous():
            raise ValueError("weight, bias, states and out must be contiguous float32 on the GPU of x")
    with torch.cuda.device(x.device):
        st = torch.cuda.current_stream(x.device).cuda_stream
        _raise_for(load_library().ssd_causal_conv1d_tokmajor(
            _ptr(x), xs, _ptr(weight), _ptr(bias), _ptr(conv_state), Bsz, D, S, W, act,
            _ptr(out), _ptr(final_state) if return_final_state else None, ctypes.c_void_p(st)),
            "ssd_causal_conv1d_tokmajor")
    return (out, final_state) if return_final_state else out


class SsdBwdCall:
    """One prepared ``ssd_bwd`` call over fixed tensors (for repeated launches)."""

    def __init__(self, args, desc: SsdDesc, keep, grads):
        self._args = args
        self.desc = desc
        self._keep = keep
        self.grads = grads

    def launch(self, stream: int) -> None:
        a = self._args
        st = load_library().ssd_bwd(*a, ctypes.c_void_p(stream), ctypes.byref(self.desc))
        _raise_for(st, "ssd_bwd")


def prepare_bwd(x, dt, A, B, C, dout, chunk_size: int = 64, D=None, z=None, dt_bias=None,
                initial_states=None, dfinal_state=None, dt_softplus: bool = False,
                dt_limit: Tuple[float, float] = (0.0, math.inf)):
    """Validate, allocate the gradients and the workspace, build an SsdBwdCall.

    fp32 tensors in the ssd_fwd layouts.  ``call.grads`` holds dx, ddt, dA,
    dB, dC and, for the optional inputs given, dD, dz, ddt_bias,
    dinitial_states.
    """
    import torch
    for name, t in (("x", x), ("dt", dt), ("A", A), ("B", B), ("C", C), ("dout", dout)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
    dev = x.device
    Bsz, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    shapes = (("dt", dt, (Bsz, L, H)), ("A", A, (H,)), ("B", B, (Bsz, L, G, N)),
              ("C", C, (Bsz, L, G, N)), ("dout", dout, (Bsz, L, H, P)), ("D", D, (H,)),
              ("z", z, (Bsz, L, H, P)),
              ("dt_bias", dt_bias, (H,)), ("initial_states", initial_states, (Bsz, H, P, N)),
              ("dfinal_state", dfinal_state, (Bsz, H, P, N)))
    for name, t, shp in shapes:
        if t is not None and tuple(t.shape) != shp:
            raise ValueError(f"{name} must have shape {shp}")
    for t in (x, dt, A, B, C, dout, D, z, dt_bias, initial_states, dfinal_state):
        if t is not None and (t.dtype != torch.float32 or t.device != dev or not t.is_contiguous()):
            raise ValueError("all tensors must be contiguous float32 on the same GPU")
    desc = make_desc(Bsz, L, H, P, N, G)
    desc.mma = SSD_MMA_F32
    desc.dt_min, desc.dt_max = float(dt_limit[0]), float(dt_limit[1])
    desc.dt_bias, desc.initial_state = _ptr(dt_bias), _ptr(initial_states)
    desc.z = _ptr(z)
    n = ctypes.c_size_t(0)
    _raise_for(load_library().ssd_bwd_workspace_size(ctypes.byref(desc), int(chunk_size),
                                                     ctypes.byref(n)), "ssd_bwd_workspace_size")
    ws = torch.empty(int(n.value), device=dev, dtype=torch.uint8)
    desc.workspace, desc.workspace_bytes = ws.data_ptr(), ws.numel()
    e = lambda *s: torch.empty(*s, device=dev, dtype=torch.float32)
    grads = {"dx": e(Bsz, L, H, P), "ddt": e(Bsz, L, H), "dA": e(H), "dB": e(Bsz, L, G, N),
             "dC": e(Bsz, L, G, N), "dD": e(H) if D is not None else None,
             "dz": e(Bsz, L, H, P) if z is not None else None,
             "ddt_bias": e(H) if dt_bias is not None else None,
             "dinitial_states": e(Bsz, H, P, N) if initial_states is not None else None}
    args = (_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), int(chunk_size),
            int(bool(dt_softplus)), _ptr(dout), _ptr(dfinal_state),
            *(_ptr(grads[k]) for k in ("dx", "ddt", "dA", "dB", "dC", "dD", "dz", "ddt_bias",
                                       "dinitial_states")))
    keep = (x, dt, A, B, C, dout, D, z, dt_bias, initial_states, dfinal_state, ws)
    return SsdBwdCall(args, desc, keep, grads)


def ssd_bwd(x, dt, A, B, C, dout, chunk_size: int = 64, D=None, z=None, dt_bias=None,
            initial_states=None, dfinal_state=None, dt_softplus: bool = False,
            dt_limit: Tuple[float, float] = (0.0, math.inf)):
    """SSD backward on the current torch stream; returns the dict of gradients."""
    import torch
    call = prepare_bwd(x, dt, A, B, C, dout, chunk_size, D=D, z=z, dt_bias=dt_bias,
                       initial_states=initial_states, dfinal_state=dfinal_state,
                       dt_softplus=dt_softplus, dt_limit=dt_limit)
    with torch.cuda.device(x.device):
        call.launch(torch.cuda.current_stream(x.device).cuda_stream)
    return call.grads
