"""Independent restatements of the SSD forward, in NumPy fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring).  These exist to pin
the C recurrence: each is derived from a different passage of the pages,
so an error in one of them does not repeat in the others.

  ssd_quadratic    -- the SSD "attention view": y = (L o C B^T) x with the
                      lower-triangular semiseparable decay mask
                      (page "ops-transformer MambaV2 算子套件" §1.3).
  ssd_chunked      -- the four-stage chunked algorithm in the order of that
                      page's §2 operator chain and §4.2-4.5 (chunk_cumsum ->
                      chunk_state -> chunk_state_passing -> chunk_scan),
                      returning the stage intermediates.
  ssd_linear_attention_closed_form -- A = 0, where the decay vanishes and
                      the SSM reduces to causal linear attention.

Conventions shared with the recurrence (readings of the pages): head h uses
group h // (H/G); softplus then clamp; D added before the z gate.
"""
from __future__ import annotations

import math
from typing import Dict, Optional, Tuple

import numpy as np


def _f64(a):
    if a is None:
        return None
    if hasattr(a, "detach"):
        import torch
        a = a.detach().to("cpu", torch.float64).numpy()
    return np.asarray(a, dtype=np.float64)


def discretize(dt, dt_bias=None, dt_softplus: bool = False,
               dt_limit: Tuple[float, float] = (0.0, math.inf)) -> np.ndarray:
    """delta = clamp(softplus(dt + dt_bias), dt_limit) -- page "Mamba-2 SSD for
    Ascend NPU", "Implementation" (Preprocess: softplus / clamp / decay)."""
    u = _f64(dt)
    if dt_bias is not None:
        u = u + _f64(dt_bias)
    if dt_softplus:
        # log(1 + e^u) without overflow: max(u,0) + log1p(e^-|u|)
        u = np.maximum(u, 0.0) + np.log1p(np.exp(-np.abs(u)))
    return np.clip(u, dt_limit[0], dt_limit[1])


def _expand_groups(M: np.ndarray, H: int) -> np.ndarray:
    """[B,L,G,N] -> [B,L,H,N], head h taking group h // (H/G)."""
    G = M.shape[2]
    return np.repeat(M, H // G, axis=2)


def _gate(y: np.ndarray, z) -> np.ndarray:
    if z is None:
        return y
    z = _f64(z)
    return y * (z / (1.0 + np.exp(-z)))


def ssd_quadratic(x, dt, A, B, C, D=None, z=None, dt_bias=None, initial_states=None,
                  dt_softplus: bool = False,
                  dt_limit: Tuple[float, float] = (0.0, math.inf)) -> Tuple[np.ndarray, np.ndarray]:
    """Quadratic (semiseparable-matrix) form, page "ops-transformer MambaV2 算子套件"
    §1.3: the whole sequence as one masked matrix product.

    With cs_t = sum_{s<=t} delta_s A_h,
      y_t = sum_{s<=t} (C_t . B_s) exp(cs_t - cs_s) delta_s x_s
            + exp(cs_t) C_t h0^T + D x_t, then the z gate;
      final = sum_s exp(cs_{L-1} - cs_s) delta_s x_s (outer) B_s + exp(cs_{L-1}) h0.
    O(L^2) memory per head: tiny shapes only.
    """
    x = _f64(x)
    Bsz, L, H, P = x.shape
    delta = discretize(dt, dt_bias, dt_softplus, dt_limit)          # [B,L,H]
    a = delta * _f64(A)[None, None, :]                               # [B,L,H]
    cs = np.cumsum(a, axis=1)                                        # [B,L,H]
    Bh = _expand_groups(_f64(B), H)                                  # [B,L,H,N]
    Ch = _expand_groups(_f64(C), H)
    CB = np.einsum("bthn,bshn->bhts", Ch, Bh)                        # [B,H,L,L]
    csh = np.transpose(cs, (0, 2, 1))                                # [B,H,L]
    diff = csh[:, :, :, None] - csh[:, :, None, :]                   # cs_t - cs_s
    causal = np.tril(np.ones((L, L), dtype=bool))
    decay = np.where(causal, np.exp(np.where(causal, diff, 0.0)), 0.0)
    Mmat = CB * decay * np.transpose(delta, (0, 2, 1))[:, :, None, :]
    y = np.einsum("bhts,bshp->bthp", Mmat, x)
    fin_w = np.exp(csh[:, :, -1:] - csh) * np.transpose(delta, (0, 2, 1))   # [B,H,L]
    final = np.einsum("bhs,bshp,bshn->bhpn", fin_w, x, Bh)
    if initial_states is not None:
        h0 = _f64(initial_states)                                    # [B,H,P,N]
        y = y + np.exp(cs)[..., None] * np.einsum("bthn,bhpn->bthp", Ch, h0)
        final = final + np.exp(csh[:, :, -1])[:, :, None, None] * h0
    if D is not None:
        y = y + _f64(D)[None, None, :, None] * x
    return _gate(y, z), final


def ssd_chunked(x, dt, A, B, C, chunk: int, D=None, z=None, dt_bias=None,
                initial_states=None, dt_softplus: bool = False,
                dt_limit: Tuple[float, float] = (0.0, math.inf)
                ) -> Tuple[np.ndarray, np.ndarray, Dict[str, np.ndarray]]:
    """The chunked algorithm, stage by stage, in the order of page
    "ops-transformer MambaV2 算子套件" §2 (chunk_cumsum -> chunk_state ->
    chunk_state_passing -> chunk_scan).

    The sequence is right-padded to a multiple of ``chunk`` with delta = 0
    and zero x, B, C (that page's §6 padding to whole chunks and the dt_mask
    input of §4.2); padded positions change no state and are dropped.

    Returns (out [B,L,H,P], final_state [B,H,P,N], intermediates) where the
    intermediates are
      delta    [B,H,nc,Q]   discretised step (dtout)
      Lam      [B,H,nc,Q]   inclusive in-chunk cumsum of delta*A (dacs)
      Lam_end  [B,H,nc]     chunk total (dacs_chunk)
      S_loc    [B,H,nc,P,N] state produced by each chunk from zero (states)
      S_in     [B,H,nc,P,N] state entering each chunk
    """
    x = _f64(x)
    Bsz, L, H, P = x.shape
    Q = int(chunk)
    nc = -(-L // Q)
    Lp = nc * Q
    pad = Lp - L
    delta = discretize(dt, dt_bias, dt_softplus, dt_limit)          # [B,L,H]
    Bh = _expand_groups(_f64(B), H)
    Ch = _expand_groups(_f64(C), H)
    N = Bh.shape[-1]
    if pad:
        delta = np.concatenate([delta, np.zeros((Bsz, pad, H))], axis=1)
        x = np.concatenate([x, np.zeros((Bsz, pad, H, P))], axis=1)
        Bh = np.concatenate([Bh, np.zeros((Bsz, pad, H, N))], axis=1)
        Ch = np.concatenate([Ch, np.zeros((Bsz, pad, H, N))], axis=1)
    # chunked views: [B,H,nc,Q,...]
    dl = np.transpose(delta.reshape(Bsz, nc, Q, H), (0, 3, 1, 2))
    xc = np.transpose(x.reshape(Bsz, nc, Q, H, P), (0, 3, 1, 2, 4))
    Bc = np.transpose(Bh.reshape(Bsz, nc, Q, H, N), (0, 3, 1, 2, 4))
    Cc = np.transpose(Ch.reshape(Bsz, nc, Q, H, N), (0, 3, 1, 2, 4))

    # 1. chunk_cumsum (§4.2): in-chunk inclusive prefix of delta*A, and its total
    a = dl * _f64(A)[None, :, None, None]
    Lam = np.cumsum(a, axis=-1)
    Lam_end = Lam[..., -1]

    # 2. chunk_state (§4.3): state each chunk builds from a zero start
    w = np.exp(Lam_end[..., None] - Lam) * dl                       # [B,H,nc,Q]
    S_loc = np.einsum("bhcq,bhcqp,bhcqn->bhcpn", w, xc, Bc)

    # 3. chunk_state_passing (§4.4): sequential over chunks
    S_in = np.empty_like(S_loc)
    S = (_f64(initial_states).copy() if initial_states is not None
         else np.zeros((Bsz, H, P, N)))
    for c in range(nc):
        S_in[:, :, c] = S
        S = np.exp(Lam_end[:, :, c])[:, :, None, None] * S + S_loc[:, :, c]
    final = S

    # 4. chunk_scan (§4.5): intra-chunk masked product + inter-chunk term
    G_cb = np.einsum("bhcin,bhcjn->bhcij", Cc, Bc)                  # C B^T per chunk
    causal = np.tril(np.ones((Q, Q), dtype=bool))
    seg = Lam[..., :, None] - Lam[..., None, :]                      # Lam_i - Lam_j
    Mmat = np.where(causal, G_cb * np.exp(np.where(causal, seg, 0.0)) * dl[..., None, :], 0.0)
    y_diag = np.einsum("bhcij,bhcjp->bhcip", Mmat, xc)
    y_off = np.exp(Lam)[..., None] * np.einsum("bhcin,bhcpn->bhcip", Cc, S_in)
    y = np.transpose((y_diag + y_off).reshape(Bsz, H, Lp, P), (0, 2, 1, 3))[:, :L]
    if D is not None:
        y = y + _f64(D)[None, None, :, None] * x[:, :L]
    inter = {"delta": dl, "Lam": Lam, "Lam_end": Lam_end, "S_loc": S_loc, "S_in": S_in}
    return _gate(y, z), final, inter


def ssd_linear_attention_closed_form(x, dt, B, C, D=None, dt_bias=None, initial_states=None,
                                     dt_softplus: bool = False,
                                     dt_limit: Tuple[float, float] = (0.0, math.inf)
                                     ) -> Tuple[np.ndarray, np.ndarray]:
    """A = 0: exp(delta*A) = 1, so the state is a running sum and
    y_t = C_t . (h0 + sum_{s<=t} delta_s x_s (outer) B_s) + D x_t
    (unnormalised causal linear attention), final = h0 + sum_s delta_s x_s (outer) B_s."""
    x = _f64(x)
    Bsz, L, H, P = x.shape
    delta = discretize(dt, dt_bias, dt_softplus, dt_limit)
    Bh = _expand_groups(_f64(B), H)
    Ch = _expand_groups(_f64(C), H)
    outer = (delta[..., None, None] * x[..., :, None]) * Bh[..., None, :]   # [B,L,H,P,N]
    S = np.cumsum(outer, axis=1)
    if initial_states is not None:
        S = S + _f64(initial_states)[:, None]
    y = np.einsum("blhpn,blhn->blhp", S, Ch)
    if D is not None:
        y = y + _f64(D)[None, None, :, None] * x
    return y, S[:, -1]
