"""Gated grouped RMSNorm, the operator that closes the chunked SSD chain.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Page "ops-transformer MambaV2 算子套件", section 4.6 (mamba2_rmsnormgated):
the input x is gated by SiLU(z), normalised by an RMSNorm taken over groups
of the last dimension, and multiplied by a weight w.  x, z and out are
[B, S, D] fp32, w is [D]; the parameters are the group count G and eps.

Readings where the page is silent:
  * the G groups are contiguous blocks of D/G elements of the last dimension;
  * the RMS of a group is sqrt(mean(g^2) + eps), eps inside the root;
  * SiLU(v) = v * sigmoid(v);
  * without z there is no gate (a plain grouped RMSNorm).

Pinned by tests/test_oracle_rmsnorm.py (hand-derived fixtures in
tests/golden/, closed forms and invariants).
"""
import numpy as np


def rmsnorm_gated(x, z, w, ngroups: int, eps: float):
    """out = g / sqrt(mean over its group of g^2 + eps) * w, g = x * silu(z).

    x, z: [..., D]; w: [D].  Computed in fp64; returns an fp64 array.
    """
    g = np.asarray(x, dtype=np.float64)
    if z is not None:
        zz = np.asarray(z, dtype=np.float64)
        with np.errstate(over="ignore"):
            g = g * (zz / (1.0 + np.exp(-zz)))
    D = g.shape[-1]
    if ngroups < 1 or D % ngroups:
        raise ValueError("D must split into ngroups equal groups")
    grouped = g.reshape(g.shape[:-1] + (ngroups, D // ngroups))
    rms = np.sqrt(np.mean(grouped * grouped, axis=-1, keepdims=True) + eps)
    return (grouped / rms).reshape(g.shape) * np.asarray(w, dtype=np.float64)
