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
from typing import Dict, Optional

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

    @property
    def tokens(self) -> int:
        return self.batch * self.seqlen

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
    h0 = 0.1 * torch.randn(Bsz, H, P, N, generator=g, dtype=f32) if w.has_h0 else None
    io = _TORCH_DTYPES[w.io_dtype]
    x, Bm, Cm = x.to(io), Bm.to(io), Cm.to(io)
    if z is not None:
        z = z.to(z_dtype)
    out = {"x": x, "dt": dt, "A": A, "B": Bm, "C": Cm, "D": D, "z": z, "initial_states": h0}
    if device != "cpu":
        out = {k: (None if v is None else v.to(device)) for k, v in out.items()}
    return out


def random_inputs(Bsz: int, L: int, H: int, P: int, N: int, G: int, seed: int,
                  has_D: bool = False, has_z: bool = False, has_h0: bool = False,
                  io_dtype: str = "f32", dt_bias: bool = False) -> Dict[str, Optional[torch.Tensor]]:
    """Inputs of an arbitrary small shape, same distributions as the workloads.

    With ``dt_bias`` an extra per-head bias ~ U(-1, 0) is drawn after the
    other tensors.
    """
    w = Workload("adhoc", Bsz, L, H, P, N, 64, G, has_D=has_D, has_z=has_z,
                 has_h0=has_h0, io_dtype=io_dtype, seed=seed)
    d = make_inputs(w)
    if dt_bias:
        g = torch.Generator(device="cpu")
        g.manual_seed(seed + 7919)
        d["dt_bias"] = -torch.rand(H, generator=g, dtype=torch.float32)
    else:
        d["dt_bias"] = None
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
