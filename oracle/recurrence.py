"""ctypes wrapper around the C fp64 recurrence in ``ssd_oracle.c``.

TEST INFRASTRUCTURE ONLY (see the package docstring).  The recurrence follows
page "ops-transformer MambaV2 算子套件" §1.1 (h(t) = A_bar h(t-1) + B_bar x(t),
y(t) = C h(t)) with the tensor semantics of page "Mamba-2 SSD for Ascend NPU",
section "Implementation" (x [B,L,H,P], dt [B,L,H], A [H], B/C [B,L,G,N],
states [B,H,P,N]; D, z, dt_bias, dt_softplus, dt_limit, initial_states).
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from typing import Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssd_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libssd_oracle.so")
_lib = None


def build_oracle(force: bool = False) -> str:
    """Compile ssd_oracle.c with gcc (-O2 -fopenmp, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH) or \
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-fopenmp",
                               "-fno-fast-math", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        build_oracle()
        lib = ctypes.CDLL(_LIB_PATH)
        i64, dp, c_int, c_dbl = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_double
        lib.ssd_oracle_f64.argtypes = [i64] * 6 + [dp] * 9 + [c_int, c_dbl, c_dbl, dp, i64,
                                                               dp, dp, c_int]
        lib.ssd_oracle_f64.restype = c_int
        f32 = ctypes.c_float
        lib.ssd_oracle_f32.argtypes = [i64] * 6 + [dp] * 9 + [c_int, f32, f32, dp, i64,
                                                               dp, dp, c_int]
        lib.ssd_oracle_f32.restype = c_int
        lib.ssd_oracle_max_threads.argtypes = []
        lib.ssd_oracle_max_threads.restype = c_int
        _lib = lib
    return _lib


def oracle_max_threads() -> int:
    return int(_load().ssd_oracle_max_threads())


def _f64(a) -> Optional[np.ndarray]:
    if a is None:
        return None
    if hasattr(a, "detach"):  # torch tensor: widen on the CPU, exactly
        import torch
        a = a.detach().to("cpu", torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def ssd_recurrence(x, dt, A, B, C, D=None, z=None, dt_bias=None, initial_states=None,
                   dt_softplus: bool = False,
                   dt_limit: Tuple[float, float] = (0.0, math.inf),
                   pairs: Optional[Sequence[Tuple[int, int]]] = None,
                   nthreads: int = 0) -> Tuple[np.ndarray, np.ndarray]:
    """Token-by-token SSD recurrence in fp64.

    Inputs may be numpy arrays or CPU torch tensors of any float dtype; they
    are widened to float64 exactly.  Returns ``(out [B,L,H,P], final_state
    [B,H,P,N])`` as float64.  With ``pairs`` only those (b, h) slices are
    computed; the rest of both outputs is NaN.
    """
    x, dt, A, B, C = (_f64(v) for v in (x, dt, A, B, C))
    D, z, dt_bias, h0 = (_f64(v) for v in (D, z, dt_bias, initial_states))
    Bsz, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    assert dt.shape == (Bsz, L, H) and A.shape == (H,)
    assert B.shape == (Bsz, L, G, N) and C.shape == (Bsz, L, G, N)
    assert D is None or D.shape == (H,)
    assert z is None or z.shape == x.shape
    assert dt_bias is None or dt_bias.shape == (H,)
    assert h0 is None or h0.shape == (Bsz, H, P, N)
    fill = np.nan if pairs is not None else 0.0
    out = np.full((Bsz, L, H, P), fill, dtype=np.float64)
    fin = np.full((Bsz, H, P, N), fill, dtype=np.float64)
    if pairs is not None:
        parr = np.ascontiguousarray(np.asarray(pairs, dtype=np.int64).reshape(-1, 2))
        pp, npairs = _ptr(parr), parr.shape[0]
    else:
        pp, npairs = None, 0
    rc = _load().ssd_oracle_f64(Bsz, L, H, P, N, G, _ptr(x), _ptr(dt), _ptr(A), _ptr(B),
                                _ptr(C), _ptr(D), _ptr(z), _ptr(dt_bias), _ptr(h0),
                                int(bool(dt_softplus)), float(dt_limit[0]), float(dt_limit[1]),
                                pp, npairs, _ptr(out), _ptr(fin), int(nthreads))
    if rc != 0:
        raise ValueError(f"ssd_oracle_f64 failed with code {rc}")
    return out, fin


def _f32(a) -> Optional[np.ndarray]:
    if a is None:
        return None
    if hasattr(a, "detach"):
        import torch
        a = a.detach().to("cpu", torch.float32).numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.float32))


def ssd_recurrence_f32(x, dt, A, B, C, D=None, z=None, dt_bias=None, initial_states=None,
                       dt_softplus: bool = False,
                       dt_limit: Tuple[float, float] = (0.0, math.inf),
                       pairs: Optional[Sequence[Tuple[int, int]]] = None,
                       nthreads: int = 0) -> Tuple[np.ndarray, np.ndarray]:
    """The same token recurrence in single precision (the C function's float
    instance).  Not a parity reference: the benchmark times it as the CPU
    baseline.  Arguments and results as ``ssd_recurrence``, in float32."""
    x, dt, A, B, C = (_f32(v) for v in (x, dt, A, B, C))
    D, z, dt_bias, h0 = (_f32(v) for v in (D, z, dt_bias, initial_states))
    Bsz, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    fill = np.nan if pairs is not None else 0.0
    out = np.full((Bsz, L, H, P), fill, dtype=np.float32)
    fin = np.full((Bsz, H, P, N), fill, dtype=np.float32)
    if pairs is not None:
        parr = np.ascontiguousarray(np.asarray(pairs, dtype=np.int64).reshape(-1, 2))
        pp, npairs = _ptr(parr), parr.shape[0]
    else:
        pp, npairs = None, 0
    rc = _load().ssd_oracle_f32(Bsz, L, H, P, N, G, _ptr(x), _ptr(dt), _ptr(A), _ptr(B),
                                _ptr(C), _ptr(D), _ptr(z), _ptr(dt_bias), _ptr(h0),
                                int(bool(dt_softplus)), float(dt_limit[0]), float(dt_limit[1]),
                                pp, npairs, _ptr(out), _ptr(fin), int(nthreads))
    if rc != 0:
        raise ValueError(f"ssd_oracle_f32 failed with code {rc}")
    return out, fin
