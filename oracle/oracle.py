"""ctypes front end of the float64 CPU oracle (``rsm_oracle.c``).

TEST INFRASTRUCTURE.  Only the test suite, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import this module.  It shares no code with the
HIP library or its Python binding, and imports nothing from the package.

``build()`` compiles ``rsm_oracle.c`` with gcc (``-O2 -fopenmp``, IEEE arithmetic, no FMA
contraction) into ``oracle/librsm_oracle.so``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "rsm_oracle.c")
_LIB = os.path.join(_HERE, "librsm_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle library in place; returns its path."""
    if not force and os.path.exists(_LIB):
        return _LIB
    tmp = _LIB + ".tmp"
    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
           "-std=c99", "-Wall", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build()
    lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    L = ctypes.c_long
    I = ctypes.c_int
    lib.rsm_oracle_route_topk.argtypes = [P, L, L, L, P, P]
    lib.rsm_oracle_route_ex.argtypes = [P, P, L, L, L, I, I, P, P]
    lib.rsm_oracle_forward.argtypes = [P, P, P, P, P, P, L, L, L, L, L, L, P, P, P, P, I]
    lib.rsm_oracle_forward_ex.argtypes = [P, P, P, P, P, P, I, P, L, L, L, L, L, L, I, I, P, P, P, P, I]
    lib.rsm_oracle_decode_step.argtypes = [P, P, P, P, P, P, L, L, L, L, L, P, P, I]
    lib.rsm_oracle_decode_ex.argtypes = [P, P, P, P, P, P, I, P, L, L, L, L, L, I, I, P, P, I]
    lib.rsm_oracle_backward.argtypes = [P, P, P, P, P, P, P, P, L, L, L, L, L, L, P, P, P, P, P, P, I]
    lib.rsm_oracle_backward.restype = ctypes.c_int
    for fn in (lib.rsm_oracle_route_topk, lib.rsm_oracle_route_ex, lib.rsm_oracle_forward,
               lib.rsm_oracle_forward_ex, lib.rsm_oracle_decode_step, lib.rsm_oracle_decode_ex):
        fn.restype = ctypes.c_int
    lib.rsm_oracle_max_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _f64(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float64)


def max_threads() -> int:
    return int(_load().rsm_oracle_max_threads())


_SCORES = {"sigmoid": 0, "softmax": 1}


def _score_kind(score: str) -> int:
    if score not in _SCORES:
        raise ValueError(f"score must be one of {sorted(_SCORES)}")
    return _SCORES[score]


def route_topk(z, K: int, noise=None, score: str = "sigmoid", normalize: bool = False):
    """z [..., M] float64 -> (idx [..., K] int32 ascending, score [..., K] float64).
    noise [..., M] (added to z in fp32 before routing) or None; score "sigmoid" or
    "softmax"; normalize divides the selected scores by their sum."""
    z, noise = _f64(z), _f64(noise)
    M = z.shape[-1]
    N = int(np.prod(z.shape[:-1]))
    if noise is not None and noise.shape != z.shape:
        raise ValueError("noise must have the shape of z")
    idx = np.empty(z.shape[:-1] + (K,), dtype=np.int32)
    sc = np.empty(z.shape[:-1] + (K,), dtype=np.float64)
    rc = _load().rsm_oracle_route_ex(_p(z), _p(noise), N, M, K, _score_kind(score), int(bool(normalize)),
                                     _p(idx), _p(sc))
    if rc != 0:
        raise ValueError(f"oracle route_topk failed ({rc})")
    return idx, sc


def forward(q, k, z, v, f, K: int, H0=None, trace: bool = False, nthreads: int = 0, noise=None,
            score: str = "sigmoid", normalize: bool = False):
    """Recurrent float64 forward.  Shapes: q,k,z [B,T,Hh,M], v [B,T,Hh,Dv], f [B,T,Hh] (one
    decay rate per token-head) or [B,T,Hh,M] (one per slot), H0 [B,Hh,M,Dv] or None, noise
    [B,T,Hh,M] or None.  Returns (o, H_final, idx[, H_trace])."""
    q, k, z, v, f, H0, noise = map(_f64, (q, k, z, v, f, H0, noise))
    B, T, Hh, M = q.shape
    Dv = v.shape[-1]
    per_slot = f.ndim == 4
    o = np.empty((B, T, Hh, Dv), dtype=np.float64)
    H = np.empty((B, Hh, M, Dv), dtype=np.float64)
    idx = np.empty((B, T, Hh, K), dtype=np.int32)
    Ht = np.empty((B, Hh, T, M, Dv), dtype=np.float64) if trace else None
    rc = _load().rsm_oracle_forward_ex(_p(q), _p(k), _p(z), _p(noise), _p(v), _p(f), int(per_slot), _p(H0),
                                       B, T, Hh, M, Dv, K, _score_kind(score), int(bool(normalize)), _p(o),
                                       _p(H), _p(idx), _p(Ht), int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle forward failed ({rc})")
    return (o, H, idx, Ht) if trace else (o, H, idx)


def decode_step(q, k, z, v, f, H, K: int, nthreads: int = 0, noise=None, score: str = "sigmoid",
                normalize: bool = False):
    """One token for all (b,h): q,k,z [B,Hh,M], v [B,Hh,Dv], f [B,Hh] or [B,Hh,M] (per slot),
    noise [B,Hh,M] or None, H [B,Hh,M,Dv] (float64, updated in place).
    Returns (o [B,Hh,Dv], idx [B,Hh,K])."""
    q, k, z, v, f, noise = map(_f64, (q, k, z, v, f, noise))
    if not (isinstance(H, np.ndarray) and H.dtype == np.float64 and H.flags.c_contiguous):
        raise TypeError("H must be a C-contiguous float64 array (updated in place)")
    B, Hh, M = q.shape
    Dv = v.shape[-1]
    o = np.empty((B, Hh, Dv), dtype=np.float64)
    idx = np.empty((B, Hh, K), dtype=np.int32)
    rc = _load().rsm_oracle_decode_ex(_p(q), _p(k), _p(z), _p(noise), _p(v), _p(f), int(f.ndim == 3), _p(H),
                                      B, Hh, M, Dv, K, _score_kind(score), int(bool(normalize)), _p(o),
                                      _p(idx), int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle decode_step failed ({rc})")
    return o, idx


def backward(q, k, z, v, f, K: int, dO, H0=None, dHT=None, nthreads: int = 0):
    """Float64 gradients of L = sum(dO * o) + sum(dHT * H_final) for the default router.
    Shapes as forward(); dO [B,T,Hh,Dv], dHT [B,Hh,M,Dv] or None (zero).
    Returns (dq, dk, dz, dv, df, dH0)."""
    q, k, z, v, f, H0, dO, dHT = map(_f64, (q, k, z, v, f, H0, dO, dHT))
    B, T, Hh, M = q.shape
    Dv = v.shape[-1]
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dz = np.empty_like(z)
    dv = np.empty_like(v)
    df = np.empty_like(f)
    dH0 = np.empty((B, Hh, M, Dv), dtype=np.float64)
    rc = _load().rsm_oracle_backward(_p(q), _p(k), _p(z), _p(v), _p(f), _p(H0), _p(dO), _p(dHT), B, T, Hh, M, Dv,
                                     K, _p(dq), _p(dk), _p(dz), _p(dv), _p(df), _p(dH0), int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle backward failed ({rc})")
    return dq, dk, dz, dv, df, dH0
