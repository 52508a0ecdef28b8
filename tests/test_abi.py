"""The C ABI library loads, exports every symbol ``include/rsm.h`` declares, and rejects
bad arguments with the documented status codes before any GPU work (CPU-only: no call
here reaches a kernel launch)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HDR = os.path.join(ROOT, "include", "rsm.h")
LIB = os.path.join(ROOT, "sparse_routed_slot_amd", "librsm.so")

OK, NULL, SHAPE, KERR, DTYPE, UNSUP, WS, HIP, ALIAS = 0, -1, -2, -3, -4, -5, -6, -7, -8
P = ctypes.c_void_p
I64 = ctypes.c_int64


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        from sparse_routed_slot_amd import build
        build.build_library()
    L = ctypes.CDLL(LIB)
    L.rsm_status_string.restype = ctypes.c_char_p
    L.rsm_route_topk.argtypes = [P, ctypes.c_int, I64, I64, I64, I64, I64, P, P, P]
    L.rsm_forward_workspace_bytes.argtypes = [ctypes.c_int, I64, I64, I64, I64, I64, I64, I64]
    L.rsm_forward_workspace_bytes.restype = ctypes.c_size_t
    L.rsm_forward_chunked.argtypes = [P, P, P, P, ctypes.c_int, P, P, I64, I64, I64, I64, I64, I64, I64,
                                      P, P, P, P, ctypes.c_size_t, P]
    L.rsm_decode_step.argtypes = [P, P, P, P, ctypes.c_int, P, P, I64, I64, I64, I64, I64, P, P, P]
    return L


def declared_functions():
    src = open(HDR).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(rsm_[a-z_0-9]+)\s*\(", src)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert {"rsm_route_topk", "rsm_forward_chunked", "rsm_decode_step"} <= set(names)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in rsm.h but not exported"


def test_status_strings(lib):
    for s in (OK, NULL, SHAPE, KERR, DTYPE, UNSUP, WS, HIP, ALIAS):
        assert lib.rsm_status_string(s)
    assert lib.rsm_status_string(12345) == b"unknown status"


A, B_, C_, D_, E_, F_, G_ = (P(0x10000 * (i + 1)) for i in range(7))


def route(lib, z=A, dtype=1, B=1, T=4, Hh=2, M=64, K=4, idx=B_, score=None):
    return lib.rsm_route_topk(z, dtype, B, T, Hh, M, K, idx, score, None)


def test_route_argument_errors(lib):
    assert route(lib, dtype=7) == DTYPE
    assert route(lib, M=48) == SHAPE
    assert route(lib, B=-1) == SHAPE
    assert route(lib, K=0) == KERR
    assert route(lib, K=65) == KERR
    assert route(lib, z=None) == NULL
    assert route(lib, idx=None) == NULL
    assert route(lib, idx=P(0x10000 + 8)) == ALIAS    # idx overlaps z
    assert route(lib, B=0) == OK                       # empty: nothing enqueued
    assert route(lib, T=0, z=None, idx=None) == OK


def fwd(lib, dtype=1, B=1, T=100, Hh=2, M=64, Dv=128, K=8, C=64, o=F_, H0=None, H_out=None, idx=None,
        ws=P(0x900000), wsb=1 << 30, q=A):
    return lib.rsm_forward_chunked(q, B_, C_, D_, dtype, E_, H0, B, T, Hh, M, Dv, K, C, o, H_out, idx, ws,
                                   wsb, None)


def test_forward_argument_errors(lib):
    assert fwd(lib, dtype=3) == DTYPE
    assert fwd(lib, Dv=48) == SHAPE
    assert fwd(lib, C=48) == SHAPE
    assert fwd(lib, M=512) == SHAPE
    assert fwd(lib, T=-5) == SHAPE
    assert fwd(lib, K=0) == KERR
    assert fwd(lib, q=None) == NULL
    assert fwd(lib, o=None) == NULL
    assert fwd(lib, ws=None) == WS
    assert fwd(lib, wsb=16) == WS
    assert fwd(lib, o=A) == ALIAS                      # o on top of q
    assert fwd(lib, H0=P(0x700000), H_out=P(0x700000 + 4)) == ALIAS  # partial overlap
    assert fwd(lib, B=0) == OK


def test_workspace_size(lib):
    f = lib.rsm_forward_workspace_bytes
    assert f(1, 8, 2048, 8, 64, 128, 64, 16) > 0
    assert f(1, 8, 0, 8, 64, 128, 64, 16) == 0
    assert f(1, 8, 2048, 8, 48, 128, 64, 16) == 0      # unsupported M
    assert f(1, 8, 2048, 8, 64, 128, 64, 65) == 0      # K > M
    # the route: a 64-bit selection mask per 64 slots and K decay factors (4 bytes) per
    # padded token-head
    assert f(1, 8, 2048, 8, 64, 128, 64, 16) >= 8 * 2048 * 8 * (8 + 16 * 4)
    assert f(1, 1, 100, 2, 64, 128, 64, 16) >= 1 * 128 * 2 * (8 + 16 * 4)   # T padded to whole chunks
    assert f(1, 1, 100, 2, 128, 64, 32, 16) >= 1 * 128 * 2 * (16 + 16 * 4)  # two mask words
    assert f(1, 1, 4096, 8, 64, 128, 64, 16) > f(1, 1, 2048, 8, 64, 128, 64, 16)
    # few heads: the sequence is cut into segments whose fp32 end states (M x Dv per head
    # and segment) also live in the workspace; 8 heads of 32 chunks give 32 segments
    assert f(1, 1, 2048, 8, 64, 128, 64, 16) >= 1 * 2048 * 8 * (8 + 16 * 4) + 8 * 31 * 64 * 128 * 4
    # enough heads for the whole chip: one segment, the route only
    assert f(1, 64, 2048, 8, 64, 128, 64, 16) < 64 * 2048 * 8 * (8 + 16 * 4) + 4096
    assert f(0, 1, 2048, 8, 64, 128, 64, 16) >= 1 * 2048 * 8 * (8 + 16 * 4)
    # M = 256, recurrent form (fp32, a router variant, or K > 32): the router's K indices and
    # K weights per token-head, each part 256-byte aligned
    assert f(0, 16, 2048, 4, 256, 256, 64, 32) == 2 * 16 * 2048 * 4 * 32 * 4
    assert f(0, 1, 3, 1, 256, 64, 64, 5) == 2 * 256
    assert f(1, 1, 3, 1, 256, 64, 64, 40) == 2 * 512
    # bf16 with K <= 32: the larger of that and the chunked route (chunks of 32 tokens: four
    # mask words and K decay factors per padded token-head)
    assert f(1, 16, 2048, 4, 256, 256, 64, 32) == 2 * 16 * 2048 * 4 * 32 * 4
    assert f(1, 1, 3, 1, 256, 64, 64, 5) == 32 * 4 * 8 + 768      # 640 bytes of factors, aligned
    assert f(1, 1, 0, 1, 256, 64, 64, 5) == 0


def dec(lib, dtype=1, B=4, Hh=2, M=64, Dv=128, K=8, H=F_, o=G_, idx=None, q=A):
    return lib.rsm_decode_step(q, B_, C_, D_, dtype, E_, H, B, Hh, M, Dv, K, o, idx, None)


def test_decode_argument_errors(lib):
    assert dec(lib, dtype=2) == DTYPE
    assert dec(lib, M=100) == SHAPE
    assert dec(lib, M=512) == SHAPE
    assert dec(lib, M=256, Hh=0) == OK                 # the router and decode take M = 256
    assert route(lib, M=256, B=0) == OK and route(lib, M=512) == SHAPE
    assert fwd(lib, M=256, B=0) == OK                  # so does the forward (recurrent form)
    assert fwd(lib, M=256, ws=None) == WS and fwd(lib, M=256, K=257) == KERR
    assert dec(lib, Dv=96) == SHAPE
    assert dec(lib, K=65) == KERR
    assert dec(lib, H=None) == NULL
    assert dec(lib, o=F_) == ALIAS                     # o on top of H
    assert dec(lib, Hh=0) == OK


class RouterOpts(ctypes.Structure):
    _fields_ = [("score", ctypes.c_int), ("normalize", ctypes.c_int), ("f_per_slot", ctypes.c_int),
                ("noise", P)]


def test_variant_argument_errors(lib):
    """Router variants: fields outside {0, 1}, a misaligned noise buffer and noise that
    overlaps an output are refused before any launch; a NULL struct is the default router."""
    O = ctypes.POINTER(RouterOpts)
    lib.rsm_route_topk_ex.argtypes = [P, ctypes.c_int, O, I64, I64, I64, I64, I64, P, P, P]
    lib.rsm_forward_chunked_ex.argtypes = [P, P, P, P, ctypes.c_int, P, P, I64, I64, I64, I64, I64, I64, I64,
                                           P, P, P, P, ctypes.c_size_t, O, P]
    lib.rsm_decode_step_ex.argtypes = [P, P, P, P, ctypes.c_int, P, P, I64, I64, I64, I64, I64, P, P, O, P]

    def r(opts, idx=B_):
        return lib.rsm_route_topk_ex(A, 1, opts, 1, 4, 2, 64, 4, idx, None, None)

    def fw(opts, o=F_):
        return lib.rsm_forward_chunked_ex(A, B_, C_, D_, 1, E_, None, 1, 100, 2, 64, 128, 8, 64, o, None, None,
                                          P(0x900000), 1 << 30, opts, None)

    def de(opts, o=G_):
        return lib.rsm_decode_step_ex(A, B_, C_, D_, 1, E_, F_, 4, 2, 64, 128, 8, o, None, opts, None)

    for bad in (RouterOpts(2, 0, 0, None), RouterOpts(0, 2, 0, None), RouterOpts(0, 0, -1, None),
                RouterOpts(1, 0, 0, P(0x800004))):
        assert r(ctypes.byref(bad)) == UNSUP
        assert fw(ctypes.byref(bad)) == UNSUP
        assert de(ctypes.byref(bad)) == UNSUP
    ok = RouterOpts(1, 1, 1, P(0x800000))
    assert r(ctypes.byref(ok), idx=P(0x800000)) == ALIAS          # idx on top of the noise
    assert fw(ctypes.byref(ok), o=P(0x800000)) == ALIAS           # o on top of the noise
    assert de(ctypes.byref(ok), o=P(0x800000)) == ALIAS
    # per-slot f is M times longer: o right after a per-token f overlaps a per-slot one
    per_slot = RouterOpts(0, 0, 1, None)
    assert fw(ctypes.byref(per_slot), o=P(0x50000 + 100 * 2 * 4)) == ALIAS
    assert lib.rsm_route_topk_ex(A, 1, None, 0, 4, 2, 64, 4, B_, None, None) == OK
    assert lib.rsm_abi_version() == 10300
