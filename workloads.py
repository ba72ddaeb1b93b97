"""Seeded synthetic SSD-forward workloads.

This module only draws random numbers: it holds none of the method's
arithmetic, so both the HIP path and the CPU oracle can take their inputs
from it without sharing any computation.

Shapes are written [B, L, H, P, N, chunk, G] (batch, sequence length, heads,
head dim, state size, chunk size, B/C groups), the convention of the page
"Mamba-2 SSD for Ascend NPU" (Benchmark table and the tensor list under
"Implementation").  Value distributions follow the usage example on that
page: x, B, C ~ N(0,1); dt ~ U(0,1) fed through softplus; A = -U(0,1).
D and z ~ N(0,1); the initial state is 0.1 * N(0,1).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional, Sequence, Tuple

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    seqlen: int
    nheads: int
    headdim: int
    dstate: int
    chunk: int
    ngroups: int
    has_D: bool = False
    has_z: bool = False
    has_h0: bool = False
    io_dtype: str = "f32"       # dtype of x, B, C ("f32" or "bf16")
    seed: int = 20260
    # packed variable-length sequences: their lengths (batch is then 1 and
    # seqlen their sum, the packed token axis); empty for dense batches
    seqlens: Tuple[int, ...] = ()

    @property
    def tokens(self) -> int:
        return self.batch * self.seqlen

    @property
    def packed(self) -> bool:
        return len(self.seqlens) > 0

    @property
    def nseq(self) -> int:
        """Rows of the call: sequences when packed, else batch rows."""
        return len(self.seqlens) if self.packed else self.batch

    @property
    def max_len(self) -> int:
        return max(self.seqlens) if self.packed else self.seqlen

    def cu_seqlens(self) -> torch.Tensor:
        """int32 [nseq+1] start offsets of the packed sequences (CPU)."""
        cu = [0]
        for n in self.seqlens:
            cu.append(cu[-1] + n)
        return torch.tensor(cu, dtype=torch.int32)

    def shape_str(self) -> str:
        return (f"[{self.batch},{self.seqlen},{self.nheads},{self.headdim},"
                f"{self.dstate},{self.chunk},{self.ngroups}]")

    def scaled(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads, indexed like their seeds (20260 + index).
WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload("tiny", 1, 128, 2, 64, 128, 128, 1, seed=20260),
    "same_device": Workload("same_device", 4, 2048, 16, 64, 128, 128, 4, seed=20261),
    "h256": Workload("h256", 8, 4096, 256, 64, 64, 64, 64, seed=20262),
    "long": Workload("long", 1, 16384, 32, 64, 128, 256, 1, has_D=True, seed=20263),
    "gated": Workload("gated", 2, 8192, 128, 64, 128, 256, 8, has_D=True, has_z=True,
                      has_h0=True, io_dtype="bf16", seed=20264),
    # the headline's 8192 tokens and heads as 16 packed sequences with a
    # long-tailed length mix (most lengths not a multiple of the chunk)
    "varlen": Workload("varlen", 1, 8192, 16, 64, 128, 128, 4, has_D=True, has_h0=True,
                       seed=20265, seqlens=(2048, 1536, 1024, 768, 640, 512, 384, 256, 200, 180,
                                            160, 140, 130, 110, 64, 40)),
}

_TORCH_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def make_inputs(w: Workload, seed: Optional[int] = None, device: str = "cpu",
                z_dtype: torch.dtype = torch.float32) -> Dict[str, Optional[torch.Tensor]]:
    """Draw one batch of inputs for workload ``w``.

    Tensors are drawn on a CPU generator in the fixed order x, dt, A, B, C,
    D, z, h0 (so a given seed gives the same bits everywhere), then cast and
    moved to ``device``.  Optional tensors the workload lacks are None.
    """
    g = torch.Generator(device="cpu")
    g.manual_seed(w.seed if seed is None else seed)
    Bsz, L, H, P, N, G = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups
    f32 = torch.float32
    x = torch.randn(Bsz, L, H, P, generator=g, dtype=f32)
    dt = torch.rand(Bsz, L, H, generator=g, dtype=f32)
    A = -torch.rand(H, generator=g, dtype=f32)
    Bm = torch.randn(Bsz, L, G, N, generator=g, dtype=f32)
    Cm = torch.randn(Bsz, L, G, N, generator=g, dtype=f32)
    D = torch.randn(H, generator=g, dtype=f32) if w.has_D else None
    z = torch.randn(Bsz, L, H, P, generator=g, dtype=f32) if w.has_z else None
    h0 = 0.1 * torch.randn(w.nseq, H, P, N, generator=g, dtype=f32) if w.has_h0 else None
    io = _TORCH_DTYPES[w.io_dtype]
    x, Bm, Cm = x.to(io), Bm.to(io), Cm.to(io)
    if z is not None:
        z = z.to(z_dtype)
    out = {"x": x, "dt": dt, "A": A, "B": Bm, "C": Cm, "D": D, "z": z, "initial_states": h0}
    if w.packed:
        out["cu_seqlens"] = w.cu_seqlens()
    if device != "cpu":
        out = {k: (None if v is None else v.to(device)) for k, v in out.items()}
    return out


def packed_inputs(seqlens: Sequence[int], H: int, P: int, N: int, G: int, seed: int,
                  has_D: bool = False, has_z: bool = False, has_h0: bool = False,
                  io_dtype: str = "f32", dt_bias: bool = False) -> Dict[str, Optional[torch.Tensor]]:
    """Packed variable-length inputs of a small shape: x [1,T,H,P], dt
    [1,T,H], B/C [1,T,G,N], initial states [nseq,H,P,N], cu_seqlens int32
    [nseq+1]; same distributions as the workloads."""
    T = int(sum(seqlens))
    w = Workload("adhoc", 1, T, H, P, N, 64, G, has_D=has_D, has_z=has_z, has_h0=has_h0,
                 io_dtype=io_dtype, seed=seed, seqlens=tuple(int(n) for n in seqlens))
    d = make_inputs(w)
    if dt_bias:
        g = torch.Generator(device="cpu")
        g.manual_seed(seed + 7919)
        d["dt_bias"] = -torch.rand(H, generator=g, dtype=torch.float32)
    else:
        d["dt_bias"] = None
    return d


def random_inputs(Bsz: int, L: int, H: int, P: int, N: int, G: int, seed: int,
                  has_D: bool = False, has_z: bool = False, has_h0: bool = False,
                  io_dtype: str = "f32", dt_bias: bool = False,
                  bias_range: Optional[Tuple[float, float]] = None,
                  A_range: Optional[Tuple[float, float]] = None,
                  A_value: Optional[float] = None,
                  scale: Optional[float] = None) -> Dict[str, Optional[torch.Tensor]]:
    """Inputs of an arbitrary small shape, same distributions as the workloads.

    With ``dt_bias`` an extra per-head bias ~ U(-1, 0) is drawn after the
    other tensors; ``bias_range = (lo, hi)`` draws it ~ U(lo, hi) instead
    (the same generator).  ``A_range = (lo, hi)`` redraws A = -U(lo, hi) per
    head from a generator of its own; ``A_value`` sets every A[h] to that
    value.  ``scale`` multiplies x, B and C by it (before any cast), for
    magnitudes outside the standard normal's range.  Drawn after everything
    else, these leave the other tensors' bits unchanged.
    """
    w = Workload("adhoc", Bsz, L, H, P, N, 64, G, has_D=has_D, has_z=has_z,
                 has_h0=has_h0, io_dtype=io_dtype, seed=seed)
    if scale is not None:
        d = make_inputs(w.scaled(io_dtype="f32"))
        io = _TORCH_DTYPES[io_dtype]
        for k in ("x", "B", "C"):
            d[k] = (d[k] * scale).to(io)
    else:
        d = make_inputs(w)
    if dt_bias or bias_range is not None:
        g = torch.Generator(device="cpu")
        g.manual_seed(seed + 7919)
        if bias_range is None:
            d["dt_bias"] = -torch.rand(H, generator=g, dtype=torch.float32)
        else:
            lo, hi = bias_range
            d["dt_bias"] = lo + (hi - lo) * torch.rand(H, generator=g, dtype=torch.float32)
    else:
        d["dt_bias"] = None
    if A_range is not None:
        g = torch.Generator(device="cpu")
        g.manual_seed(seed + 104729)
        lo, hi = A_range
        d["A"] = -(lo + (hi - lo) * torch.rand(H, generator=g, dtype=torch.float32))
    if A_value is not None:
        d["A"] = torch.full((H,), float(A_value), dtype=torch.float32)
    return d


# ------------------------------------------------------------------ gated RMSNorm
# The norm that closes the SSD chain (page "ops-transformer MambaV2 算子套件",
# section 4.6) runs on out[B, S, D] with D = H * P, in G contiguous groups.
# Its workload for an SSD workload w is [w.batch, w.seqlen, w.nheads*w.headdim]
# with G = w.ngroups.  x stands in for the SSD output and z for the gate,
# both ~ N(0,1); the weight is 1 + 0.1 * N(0,1) (an RMSNorm weight near its
# initial value of one; the page gives no distribution); eps = 1e-5.
NORM_EPS = 1e-5


def norm_shape(w: Workload):
    """(rows, dim, ngroups) of the norm that follows workload ``w``."""
    return w.batch * w.seqlen, w.nheads * w.headdim, w.ngroups


def norm_inputs(rows: int, dim: int, seed: int, has_z: bool = True,
                device: str = "cpu") -> Dict[str, Optional[torch.Tensor]]:
    """x [rows, dim], z [rows, dim] (or None), w [dim], all fp32, drawn in the
    order x, z, w from a generator on ``device`` (CPU bits are reproducible
    everywhere; a GPU generator is used for inputs too large to draw on the
    host, and only its own draws are compared)."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    f32 = torch.float32
    x = torch.randn(rows, dim, generator=g, device=device, dtype=f32)
    z = torch.randn(rows, dim, generator=g, device=device, dtype=f32) if has_z else None
    wt = 1.0 + 0.1 * torch.randn(dim, generator=g, device=device, dtype=f32)
    return {"x": x, "z": z, "w": wt}


# ------------------------------------------------------------------ causal conv1d
# The depthwise causal conv1d before the SSD (page "ops-transformer MambaV2
# 算子套件", §1.4 and §4.1) runs on x [B, D, S] with D channels.  Its test
# shape on that page is B=1, D=10240, S=1024, W=4 ("page"); before an SSD
# workload w it runs over the channels that feed x, B and C,
# D = H*P + 2*G*N, with S = L.  x ~ N(0,1); weight and bias ~ U(-1/sqrt(W),
# 1/sqrt(W)) (the default initialisation of a grouped conv1d with W taps per
# channel; the page gives no distribution); conv state ~ N(0,1).
CONV_WIDTH = 4


def conv_shape(name: str):
    """(B, D, S) of the conv workload ``name``: "page" or an SSD workload."""
    if name == "page":
        return 1, 10240, 1024
    w = WORKLOADS[name]
    return w.batch, w.nheads * w.headdim + 2 * w.ngroups * w.dstate, w.seqlen


def conv_inputs(Bsz: int, D: int, S: int, W: int, seed: int, device: str = "cpu",
                has_bias: bool = True, has_state: bool = False) -> Dict[str, Optional[torch.Tensor]]:
    """x [B,D,S], weight [D,W], bias [D] (or None), conv_state [B,D,W-1] (or
    None), fp32, drawn in that order from a generator on ``device``."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    f32 = torch.float32
    bound = 1.0 / W ** 0.5
    x = torch.randn(Bsz, D, S, generator=g, device=device, dtype=f32)
    wt = (torch.rand(D, W, generator=g, device=device, dtype=f32) * 2 - 1) * bound
    b = (torch.rand(D, generator=g, device=device, dtype=f32) * 2 - 1) * bound if has_bias else None
    st = torch.randn(Bsz, D, W - 1, generator=g, device=device, dtype=f32) if has_state else None
    return {"x": x, "w": wt, "bias": b, "conv_state": st}
