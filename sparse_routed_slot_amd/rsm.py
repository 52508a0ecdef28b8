"""Python binding of ``librsm.so`` (ctypes): argument marshalling only.

Every step of the mixer runs in the HIP kernels behind the C ABI declared in
``include/rsm.h``; this module only turns torch tensors into device pointers, allocates
outputs and the forward workspace with torch, and passes torch's current HIP stream.
If the library has not been built, every call raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

__all__ = ["RSMError", "lib_path", "load", "route_topk", "forward_chunked", "forward_chunked_noalloc",
           "noalloc_scratch_bytes", "backward", "decode_step",
           "forward_workspace_bytes", "abi_version", "DTYPE_CODES", "SCORE_KINDS"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "librsm.so")
_lib = None

DTYPE_CODES = {torch.float32: 0, torch.bfloat16: 1}
SCORE_KINDS = {"sigmoid": 0, "softmax": 1}


class _RouterOpts(ctypes.Structure):
    """rsm_router_opts of include/rsm.h."""
    _fields_ = [("score", ctypes.c_int), ("normalize", ctypes.c_int), ("f_per_slot", ctypes.c_int),
                ("noise", ctypes.c_void_p)]


class RSMError(RuntimeError):
    """A librsm call returned a non-zero status."""


def lib_path() -> str:
    return _LIB_PATH


def load():
    """Load librsm.so (raises if it is missing: build it with sparse_routed_slot_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is not built; run `python -m sparse_routed_slot_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.rsm_status_string.argtypes = [I]
    lib.rsm_status_string.restype = ctypes.c_char_p
    lib.rsm_abi_version.restype = I
    lib.rsm_route_topk.argtypes = [P, I, I64, I64, I64, I64, I64, P, P, P]
    lib.rsm_route_topk.restype = I
    lib.rsm_forward_workspace_bytes.argtypes = [I, I64, I64, I64, I64, I64, I64, I64]
    lib.rsm_forward_workspace_bytes.restype = ctypes.c_size_t
    lib.rsm_forward_chunked.argtypes = [P, P, P, P, I, P, P, I64, I64, I64, I64, I64, I64, I64, P, P, P, P,
                                        ctypes.c_size_t, P]
    lib.rsm_forward_chunked.restype = I
    lib.rsm_decode_step.argtypes = [P, P, P, P, I, P, P, I64, I64, I64, I64, I64, P, P, P]
    lib.rsm_decode_step.restype = I
    O = ctypes.POINTER(_RouterOpts)
    lib.rsm_route_topk_ex.argtypes = [P, I, O, I64, I64, I64, I64, I64, P, P, P]
    lib.rsm_route_topk_ex.restype = I
    lib.rsm_forward_chunked_ex.argtypes = [P, P, P, P, I, P, P, I64, I64, I64, I64, I64, I64, I64, P, P, P, P,
                                           ctypes.c_size_t, O, P]
    lib.rsm_forward_chunked_ex.restype = I
    lib.rsm_decode_step_ex.argtypes = [P, P, P, P, I, P, P, I64, I64, I64, I64, I64, P, P, O, P]
    lib.rsm_decode_step_ex.restype = I
    lib.rsm_backward_workspace_bytes.argtypes = [I, I64, I64, I64, I64, I64, I64]
    lib.rsm_backward_workspace_bytes.restype = ctypes.c_size_t
    lib.rsm_backward.argtypes = [P, P, P, P, I, P, P, P, P, I64, I64, I64, I64, I64, I64, P, P, P, P, P, P, P,
                                 ctypes.c_size_t, P]
    lib.rsm_backward.restype = I
    lib.rsm_noalloc_scratch_bytes.argtypes = []
    lib.rsm_noalloc_scratch_bytes.restype = ctypes.c_size_t
    lib.rsm_forward_chunked_noalloc.argtypes = [P, P, P, P, I, P, P, I64, I64, I64, I64, I64, I64, I64, P, P, P, P]
    lib.rsm_forward_chunked_noalloc.restype = I
    _lib = lib
    return lib


def abi_version() -> int:
    return int(load().rsm_abi_version())


def _check(status: int):
    if status != 0:
        raise RSMError(f"librsm status {status}: {load().rsm_status_string(status).decode()}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev(t: torch.Tensor, name: str) -> torch.Tensor:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    return t.contiguous()


def _code(t: torch.Tensor) -> int:
    if t.dtype not in DTYPE_CODES:
        raise ValueError(f"unsupported dtype {t.dtype}; use float32 or bfloat16")
    return DTYPE_CODES[t.dtype]


def _router(score: str, normalize: bool, f_per_slot: bool, noise: Optional[torch.Tensor], zshape):
    """(opts struct or None for the default router, the contiguous noise tensor)."""
    if score not in SCORE_KINDS:
        raise ValueError(f"score must be one of {sorted(SCORE_KINDS)}")
    if noise is not None:
        noise = _dev(noise, "noise")
        if noise.dtype != torch.float32 or tuple(noise.shape) != tuple(zshape):
            raise ValueError(f"noise must be float32 of shape {tuple(zshape)}")
    if score == "sigmoid" and not normalize and not f_per_slot and noise is None:
        return None, None
    return _RouterOpts(SCORE_KINDS[score], int(bool(normalize)), int(bool(f_per_slot)),
                       None if noise is None else noise.data_ptr()), noise


def route_topk(z: torch.Tensor, K: int, want_score: bool = True, score: str = "sigmoid",
               normalize: bool = False, noise: Optional[torch.Tensor] = None
               ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """z [B,T,Hh,M] -> idx [B,T,Hh,K] int32 (ascending slots), score [B,T,Hh,K] fp32 (the
    routing weight: sigmoid or softmax, renormalised over the selected slots if asked).
    noise: fp32 [B,T,Hh,M] added to z before routing, or None."""
    z = _dev(z, "z")
    B, T, Hh, M = z.shape
    opts, noise = _router(score, normalize, False, noise, z.shape)
    idx = torch.empty((B, T, Hh, K), dtype=torch.int32, device=z.device)
    sc = torch.empty((B, T, Hh, K), dtype=torch.float32, device=z.device) if want_score else None
    if opts is None:
        _check(load().rsm_route_topk(_ptr(z), _code(z), B, T, Hh, M, K, _ptr(idx), _ptr(sc), _stream()))
    else:
        _check(load().rsm_route_topk_ex(_ptr(z), _code(z), ctypes.byref(opts), B, T, Hh, M, K, _ptr(idx), _ptr(sc),
                                        _stream()))
    return idx, sc


def forward_workspace_bytes(dtype: torch.dtype, B: int, T: int, Hh: int, M: int, Dv: int, C: int, K: int) -> int:
    return int(load().rsm_forward_workspace_bytes(DTYPE_CODES[dtype], B, T, Hh, M, Dv, C, K))


def forward_chunked(q, k, z, v, f, K: int, C: int = 64, H0: Optional[torch.Tensor] = None,
                    want_state: bool = True, want_idx: bool = False,
                    workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                    state_out: Optional[torch.Tensor] = None, score: str = "sigmoid", normalize: bool = False,
                    noise: Optional[torch.Tensor] = None):
    """Chunked forward.  q,k,z [B,T,Hh,M], v [B,T,Hh,Dv] (same dtype), f [B,T,Hh] fp32 (or
    [B,T,Hh,M]: one decay rate per slot), H0 [B,Hh,M,Dv] fp32 or None; router variant:
    score "sigmoid"/"softmax", normalize, noise fp32 [B,T,Hh,M] or None.
    Returns (o [B,T,Hh,Dv] fp32, H_out or None, idx or None)."""
    q, k, z, v, f = (_dev(t, n) for t, n in zip((q, k, z, v, f), "qkzvf"))
    if not (q.dtype == k.dtype == z.dtype == v.dtype):
        raise ValueError("q, k, z, v must share one dtype")
    if f.dtype != torch.float32:
        raise ValueError("f must be float32")
    B, T, Hh, M = q.shape
    Dv = v.shape[-1]
    if tuple(f.shape) not in ((B, T, Hh), (B, T, Hh, M)):
        raise ValueError("f must be [B,T,Hh] or [B,T,Hh,M]")
    opts, noise = _router(score, normalize, f.dim() == 4, noise, q.shape)
    dev = q.device
    if H0 is not None:
        H0 = _dev(H0, "H0")
        if H0.dtype != torch.float32:
            raise ValueError("H0 must be float32")
    o = out if out is not None else torch.empty((B, T, Hh, Dv), dtype=torch.float32, device=dev)
    H = None
    if want_state:
        H = state_out if state_out is not None else torch.empty((B, Hh, M, Dv), dtype=torch.float32, device=dev)
    idx = torch.empty((B, T, Hh, K), dtype=torch.int32, device=dev) if want_idx else None
    need = forward_workspace_bytes(q.dtype, B, T, Hh, M, Dv, C, K)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    if opts is None:
        _check(load().rsm_forward_chunked(
            _ptr(q), _ptr(k), _ptr(z), _ptr(v), _code(q), _ptr(f), _ptr(H0), B, T, Hh, M, Dv, K, C,
            _ptr(o), _ptr(H), _ptr(idx), _ptr(workspace), workspace.numel(), _stream()))
    else:
        _check(load().rsm_forward_chunked_ex(
            _ptr(q), _ptr(k), _ptr(z), _ptr(v), _code(q), _ptr(f), _ptr(H0), B, T, Hh, M, Dv, K, C,
            _ptr(o), _ptr(H), _ptr(idx), _ptr(workspace), workspace.numel(), ctypes.byref(opts), _stream()))
    return o, H, idx


def noalloc_scratch_bytes() -> int:
    """Size of the library's fixed scratch array used by forward_chunked_noalloc."""
    return int(load().rsm_noalloc_scratch_bytes())


def forward_chunked_noalloc(q, k, z, v, f, K: int, C: int = 64, H0: Optional[torch.Tensor] = None,
                            want_idx: bool = False, out: Optional[torch.Tensor] = None,
                            state_out: Optional[torch.Tensor] = None):
    """forward_chunked through rsm_forward_chunked_noalloc: the library allocates nothing;
    its workspace is the library's fixed per-device scratch array.  out and state_out (and
    the idx buffer, when want_idx) are the caller's; pass preallocated ones to allocate
    nothing here either.  Returns (o, H_out, idx or None)."""
    q, k, z, v, f = (_dev(t, n) for t, n in zip((q, k, z, v, f), "qkzvf"))
    if not (q.dtype == k.dtype == z.dtype == v.dtype) or f.dtype != torch.float32:
        raise ValueError("q, k, z, v must share one dtype; f must be float32")
    B, T, Hh, M = q.shape
    Dv = v.shape[-1]
    if tuple(f.shape) != (B, T, Hh):
        raise ValueError("f must be [B,T,Hh]")
    if H0 is not None:
        H0 = _dev(H0, "H0")
    dev = q.device
    o = out if out is not None else torch.empty((B, T, Hh, Dv), dtype=torch.float32, device=dev)
    H = state_out if state_out is not None else torch.empty((B, Hh, M, Dv), dtype=torch.float32, device=dev)
    idx = torch.empty((B, T, Hh, K), dtype=torch.int32, device=dev) if want_idx else None
    _check(load().rsm_forward_chunked_noalloc(
        _ptr(q), _ptr(k), _ptr(z), _ptr(v), _code(q), _ptr(f), _ptr(H0), B, T, Hh, M, Dv, K, C,
        _ptr(o), _ptr(H), _ptr(idx), _stream()))
    return o, H, idx


def backward(q, k, z, v, f, K: int, dO, H0: Optional[torch.Tensor] = None, dHT: Optional[torch.Tensor] = None,
             want_dH0: bool = True, workspace: Optional[torch.Tensor] = None):
    """Gradients of L = sum(dO * o) + sum(dHT * H_final) for the default router (the
    vector-Jacobian product of forward_chunked).  dO fp32 [B,T,Hh,Dv]; dHT fp32 [B,Hh,M,Dv]
    or None.  Returns (dq, dk, dz, dv, df, dH0 or None), all fp32."""
    q, k, z, v, f, dO = (_dev(t, n) for t, n in zip((q, k, z, v, f, dO), ("q", "k", "z", "v", "f", "dO")))
    if not (q.dtype == k.dtype == z.dtype == v.dtype) or f.dtype != torch.float32 or dO.dtype != torch.float32:
        raise ValueError("q, k, z, v must share one dtype; f and dO must be float32")
    B, T, Hh, M = q.shape
    Dv = v.shape[-1]
    if H0 is not None:
        H0 = _dev(H0, "H0")
    if dHT is not None:
        dHT = _dev(dHT, "dHT")
    dev = q.device
    dq = torch.empty((B, T, Hh, M), dtype=torch.float32, device=dev)
    dk = torch.empty_like(dq)
    dz = torch.empty_like(dq)
    dv = torch.empty((B, T, Hh, Dv), dtype=torch.float32, device=dev)
    df = torch.empty((B, T, Hh), dtype=torch.float32, device=dev)
    dH0 = torch.empty((B, Hh, M, Dv), dtype=torch.float32, device=dev) if want_dH0 else None
    need = int(load().rsm_backward_workspace_bytes(_code(q), B, T, Hh, M, Dv, K))
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _check(load().rsm_backward(_ptr(q), _ptr(k), _ptr(z), _ptr(v), _code(q), _ptr(f), _ptr(H0), _ptr(dO),
                               _ptr(dHT), B, T, Hh, M, Dv, K, _ptr(dq), _ptr(dk), _ptr(dz), _ptr(dv), _ptr(df),
                               _ptr(dH0), _ptr(workspace), workspace.numel(), _stream()))
    return dq, dk, dz, dv, df, dH0


def decode_step(q, k, z, v, f, H: torch.Tensor, K: int, want_idx: bool = False,
                out: Optional[torch.Tensor] = None, score: str = "sigmoid", normalize: bool = False,
                noise: Optional[torch.Tensor] = None):
    """One token for B x Hh heads.  q,k,z [B,Hh,M], v [B,Hh,Dv], f [B,Hh] fp32 (or [B,Hh,M]:
    per slot), H [B,Hh,M,Dv] fp32 contiguous (updated in place); router variant as in
    forward_chunked (noise [B,Hh,M]).  Returns (o [B,Hh,Dv], idx or None)."""
    q, k, z, v, f = (_dev(t, n) for t, n in zip((q, k, z, v, f), "qkzvf"))
    if not (H.is_cuda and H.is_contiguous() and H.dtype == torch.float32):
        raise ValueError("H must be a contiguous float32 device tensor (updated in place)")
    B, Hh, M = q.shape
    Dv = v.shape[-1]
    if f.dtype != torch.float32 or tuple(f.shape) not in ((B, Hh), (B, Hh, M)):
        raise ValueError("f must be float32 [B,Hh] or [B,Hh,M]")
    opts, noise = _router(score, normalize, f.dim() == 3, noise, q.shape)
    o = out if out is not None else torch.empty((B, Hh, Dv), dtype=torch.float32, device=q.device)
    idx = torch.empty((B, Hh, K), dtype=torch.int32, device=q.device) if want_idx else None
    if opts is None:
        _check(load().rsm_decode_step(_ptr(q), _ptr(k), _ptr(z), _ptr(v), _code(q), _ptr(f), _ptr(H), B, Hh, M,
                                      Dv, K, _ptr(o), _ptr(idx), _stream()))
    else:
        _check(load().rsm_decode_step_ex(_ptr(q), _ptr(k), _ptr(z), _ptr(v), _code(q), _ptr(f), _ptr(H), B, Hh, M,
                                         Dv, K, _ptr(o), _ptr(idx), ctypes.byref(opts), _stream()))
    return o, idx
