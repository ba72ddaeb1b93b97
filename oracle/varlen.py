"""Packed variable-length sequences for the SSD forward (the cu_seqlens /
seq_idx form that page "Mamba-2 SSD for Ascend NPU", section "Limitations and
roadmap", lists as not yet implemented there, and that page "ops-transformer
MambaV2 算子套件" §1.4 describes for packed batches: sequences concatenated
along the token axis, delimited by cumulative start offsets).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Readings where the pages are silent:
  * the tokens of nseq sequences are concatenated along one token axis of
    length T; cu_seqlens [nseq+1] holds the start offset of each sequence
    and T last (cu_seqlens[0] = 0, non-decreasing); a sequence may be empty;
  * the state resets at every sequence start: the state entering sequence s
    is initial_states[s] (or zero), and no token of one sequence sees another
    sequence's tokens;
  * final_state and initial_states are per sequence, [nseq, H, P, N].

ssd_varlen is the definition: the token recurrence run on each sequence on
its own.  ssd_quadratic_seq_idx restates the same thing independently, as
one masked matrix over all T tokens (a cumulative decay over the whole
packed axis, the causal mask restricted to pairs in the same sequence); the
pins in tests/test_oracle_varlen.py hold the two against each other.
"""
from __future__ import annotations

import math
from typing import Tuple

import numpy as np

from .forms import _expand_groups, _f64, _gate, discretize
from .recurrence import ssd_recurrence


def _offsets(cu_seqlens, T: int) -> np.ndarray:
    cu = np.asarray(cu_seqlens.cpu() if hasattr(cu_seqlens, "cpu") else cu_seqlens,
                    dtype=np.int64).reshape(-1)
    if cu.size < 2 or cu[0] != 0 or cu[-1] != T or np.any(np.diff(cu) < 0):
        raise ValueError("cu_seqlens must start at 0, be non-decreasing and end at T")
    return cu


def _tokens_first(a):
    """[1, T, ...] -> [T, ...] (a leading batch of one is the packed axis)."""
    a = _f64(a)
    return None if a is None else (a[0] if a.shape[0] == 1 and a.ndim >= 3 else a)


def ssd_varlen(x, dt, A, B, C, cu_seqlens, D=None, z=None, dt_bias=None, initial_states=None,
               dt_softplus: bool = False,
               dt_limit: Tuple[float, float] = (0.0, math.inf)) -> Tuple[np.ndarray, np.ndarray]:
    """x [T,H,P] (or [1,T,H,P]), dt [T,H], B/C [T,G,N], z like x,
    initial_states [nseq,H,P,N].  Returns (out [T,H,P], final_state
    [nseq,H,P,N]) in fp64: each sequence through the token recurrence."""
    x, dt, B, C, z = (_tokens_first(v) for v in (x, dt, B, C, z))
    T, H, P = x.shape
    N = B.shape[-1]
    cu = _offsets(cu_seqlens, T)
    nseq = cu.size - 1
    h0 = None if initial_states is None else _f64(initial_states)
    out = np.zeros((T, H, P))
    fin = np.zeros((nseq, H, P, N))
    for s in range(nseq):
        a, e = int(cu[s]), int(cu[s + 1])
        if e == a:                                  # empty: the state passes through
            if h0 is not None:
                fin[s] = h0[s]
            continue
        sl = slice(a, e)
        o, f = ssd_recurrence(x[None, sl], dt[None, sl], A, B[None, sl], C[None, sl], D=D,
                              z=None if z is None else z[None, sl], dt_bias=dt_bias,
                              initial_states=None if h0 is None else h0[s:s + 1],
                              dt_softplus=dt_softplus, dt_limit=dt_limit)
        out[sl] = o[0]
        fin[s] = f[0]
    return out, fin


def ssd_quadratic_seq_idx(x, dt, A, B, C, cu_seqlens, D=None, z=None, dt_bias=None,
                          initial_states=None, dt_softplus: bool = False,
                          dt_limit: Tuple[float, float] = (0.0, math.inf)
                          ) -> Tuple[np.ndarray, np.ndarray]:
    """The packed forward as one matrix over all T tokens (page
    "ops-transformer MambaV2 算子套件" §1.3's semiseparable form with a
    per-token sequence index): with cs the cumulative sum of delta*A over the
    whole packed axis and seq(t) the sequence of token t,
      y_t = sum_{s<=t, seq(s)=seq(t)} (C_t.B_s) exp(cs_t - cs_s) delta_s x_s
            + exp(cs_t - cs_{start(t)-1}) C_t h0[seq(t)]^T + D x_t, then the gate.
    O(T^2) memory per head: tiny shapes only."""
    x, dt, B, C, z = (_tokens_first(v) for v in (x, dt, B, C, z))
    T, H, P = x.shape
    cu = _offsets(cu_seqlens, T)
    nseq = cu.size - 1
    seq = np.repeat(np.arange(nseq), np.diff(cu))                   # [T]
    start = cu[seq]                                                  # [T]
    delta = discretize(dt, dt_bias, dt_softplus, dt_limit)          # [T,H]
    a = delta * _f64(A)[None, :]
    cs = np.cumsum(a, axis=0)                                        # [T,H]
    cs_before = np.concatenate([np.zeros((1, H)), cs], axis=0)       # cs_{t-1}, cs_{-1} = 0
    Bh = _expand_groups(_f64(B)[None], H)[0]                         # [T,H,N]
    Ch = _expand_groups(_f64(C)[None], H)[0]
    CB = np.einsum("thn,shn->hts", Ch, Bh)                           # [H,T,T]
    same = (seq[:, None] == seq[None, :]) & np.tril(np.ones((T, T), dtype=bool))
    diff = cs.T[:, :, None] - cs.T[:, None, :]                       # cs_t - cs_s
    decay = np.where(same[None], np.exp(np.where(same[None], diff, 0.0)), 0.0)
    y = np.einsum("hts,sh,shp->thp", CB * decay, delta, x)
    N = Bh.shape[-1]
    fin = np.zeros((nseq, H, P, N))
    h0 = None if initial_states is None else _f64(initial_states)
    for s in range(nseq):
        a0, e0 = int(cu[s]), int(cu[s + 1])
        cs_end = cs_before[e0]                                       # cs at the last token
        w = np.exp(cs_end[None, :] - cs[a0:e0]) * delta[a0:e0]       # [len,H]
        fin[s] = np.einsum("sh,shp,shn->hpn", w, x[a0:e0], Bh[a0:e0])
        if h0 is not None:
            fin[s] += np.exp(cs_end - cs_before[a0])[:, None, None] * h0[s]
    if h0 is not None:
        into = np.exp(cs - cs_before[start])                        # decay since the start
        y = y + into[:, :, None] * np.einsum("thn,thpn->thp", Ch, h0[seq])
    if D is not None:
        y = y + _f64(D)[None, :, None] * x
    return _gate(y, z), fin
