"""Depthwise causal conv1d with bias and SiLU, the step before the SSD.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Page "ops-transformer MambaV2 算子套件": §1.4 (a short depthwise causal
convolution of width 4 over the time axis, then SiLU, feeding the SSM) and
§4.1 (mamba2_causal_conv1d: x [B,D,S] fp32, a per-channel weight of width W
and a per-channel bias; its test builds the reference as a grouped conv1d
with groups = D, stride 1, padding W-1, cut to the first S steps, then SiLU).

Readings where the page is silent or garbled:
  * w is [D, W] (the table's "w BDS" is an extraction garble; a depthwise
    kernel holds W taps per channel); tap k multiplies x[t - (W-1) + k], the
    cross-correlation of a conv1d padded by W-1 on the left, so w[:, W-1]
    weighs the current step;
  * bias is fp32 like x (the table's FP16 would not combine with the fp32
    reference conv); bias and activation are optional;
  * the W-1 steps before t = 0 are zeros, or the caller's conv state
    x_prev [B, D, W-1] (the cached-state form of §1.4); the final conv state
    is the last W-1 inputs of the padded sequence, [B, D, W-1].
"""
from __future__ import annotations

import numpy as np


def causal_conv1d(x, w, bias=None, x_prev=None, activation: bool = True):
    """out[b,d,t] = act(bias[d] + sum_k w[d,k] * xx[b,d,t+k]), xx = x_prev ++ x.

    x: [B, D, S]; w: [D, W]; bias: [D] or None; x_prev: [B, D, W-1] or None.
    Returns (out [B, D, S], final_state [B, D, W-1]) in fp64.
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    Bsz, D, S = x.shape
    W = w.shape[1]
    assert w.shape == (D, W) and W >= 1
    pre = (np.zeros((Bsz, D, W - 1)) if x_prev is None
           else np.asarray(x_prev, dtype=np.float64).reshape(Bsz, D, W - 1))
    xx = np.concatenate([pre, x], axis=2)                  # [B, D, S + W - 1]
    out = np.zeros((Bsz, D, S))
    for k in range(W):                                      # one tap at a time
        out += w[None, :, k, None] * xx[:, :, k:k + S]
    if bias is not None:
        out += np.asarray(bias, dtype=np.float64)[None, :, None]
    if activation:
        with np.errstate(over="ignore"):
            out = out / (1.0 + np.exp(-out))                # silu(v) = v * sigmoid(v)
    final = xx[:, :, S:].copy() if W > 1 else np.zeros((Bsz, D, 0))
    return out, final
