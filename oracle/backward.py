"""Gradients of the SSD forward (the backward pass), in fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The forward is the token recurrence of page "ops-transformer MambaV2 算子套件"
§1.1 with the tensor semantics of page "Mamba-2 SSD for Ascend NPU",
"Implementation"; that page's "AscendC training" section and "Limitations and
roadmap" describe a backward producing the gradients of x, dt, A, B, C (and
D, dt_bias, the initial state) for contiguous P = N = chunk = 64 in FP32.

ssd_grads writes the recurrence once more, here in plain PyTorch fp64 ops
(a loop over tokens, vectorised over batch, heads and the state), and takes
its gradients with torch.autograd: the definition of the backward, with no
chunking.  With z the output is gated as in the forward, out = y * silu(z),
and dz is returned.  Pinned by central finite differences of the fp64 C
recurrence in tests/test_oracle_backward.py.

Readings: the gradient of the clamp is zero
where dt is clamped (the inputs keep away from the edges); dA sums over all
batch rows and tokens; dD and ddt_bias likewise.
"""
from __future__ import annotations

import math
from typing import Dict, Optional, Tuple

import numpy as np


def _t(a, torch):
    if a is None:
        return None
    if hasattr(a, "detach"):
        return a.detach().to("cpu", torch.float64).clone()
    return torch.tensor(np.asarray(a, dtype=np.float64))


def ssd_grads(x, dt, A, B, C, dout, D=None, z=None, dt_bias=None, initial_states=None,
              dfinal_state=None, dt_softplus: bool = False,
              dt_limit: Tuple[float, float] = (0.0, math.inf)) -> Dict[str, Optional[np.ndarray]]:
    """Gradients of L = <dout, out> + <dfinal_state, final_state>.

    x [B,L,H,P], dt [B,L,H], A [H], B/C [B,L,G,N], dout [B,L,H,P],
    D [H], z [B,L,H,P], dt_bias [H], initial_states [B,H,P,N], dfinal_state
    [B,H,P,N] (optional ones may be None).  Returns a dict of fp64 arrays: dx,
    ddt, dA, dB, dC and, for the optional inputs given, dD, dz, ddt_bias,
    dinitial_states.
    """
    import torch
    xs = {"x": x, "dt": dt, "A": A, "B": B, "C": C, "D": D, "z": z, "dt_bias": dt_bias,
          "initial_states": initial_states}
    v = {k: _t(a, torch) for k, a in xs.items()}
    for k, a in v.items():
        if a is not None:
            a.requires_grad_(True)
    Bsz, L, H, P = v["x"].shape
    G, N = v["B"].shape[2], v["B"].shape[3]
    hpg = H // G
    u = v["dt"] + (v["dt_bias"][None, None, :] if v["dt_bias"] is not None else 0.0)
    if dt_softplus:
        u = torch.nn.functional.softplus(u)
    delta = torch.clamp(u, min=dt_limit[0], max=dt_limit[1])         # [B,L,H]
    Bh = v["B"].repeat_interleave(hpg, dim=2)                         # [B,L,H,N]
    Ch = v["C"].repeat_interleave(hpg, dim=2)
    S = (v["initial_states"] if v["initial_states"] is not None
         else torch.zeros(Bsz, H, P, N, dtype=torch.float64))
    ys = []
    for t in range(L):
        dA_t = torch.exp(delta[:, t] * v["A"][None, :])              # [B,H]
        S = dA_t[:, :, None, None] * S + (delta[:, t, :, None, None] * v["x"][:, t, :, :, None]
                                          * Bh[:, t, :, None, :])
        y = torch.einsum("bhpn,bhn->bhp", S, Ch[:, t])
        if v["D"] is not None:
            y = y + v["D"][None, :, None] * v["x"][:, t]
        ys.append(y)
    out = torch.stack(ys, dim=1)                                      # [B,L,H,P]
    if v["z"] is not None:
        out = out * (v["z"] * torch.sigmoid(v["z"]))
    loss = (out * _t(dout, torch)).sum()
    if dfinal_state is not None:
        loss = loss + (S * _t(dfinal_state, torch)).sum()
    loss.backward()
    names = {"x": "dx", "dt": "ddt", "A": "dA", "B": "dB", "C": "dC", "D": "dD", "z": "dz",
             "dt_bias": "ddt_bias", "initial_states": "dinitial_states"}
    return {names[k]: (None if a is None else a.grad.numpy()) for k, a in v.items()}
