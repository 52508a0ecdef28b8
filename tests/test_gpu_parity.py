"""GPU parity of librsm (router, chunked forward, decode step) against the float64 oracle.

Every comparison is on the same seeded inputs: top-K indices bit-exact, outputs and states
within max|delta| <= 1e-5 * max|o| (fp32 inputs) or 2e-3 * max|o| (bf16 inputs, fp32
state), plus the bitwise invariants of untouched slots.  All calls go through the C ABI
(sparse_routed_slot_amd.rsm is ctypes marshalling only).
"""
import sys
import zlib

import numpy as np
import pytest

from oracle import oracle
from sparse_routed_slot_amd import inputs as gen
from tests._util import TOL, check_close, dev_inputs, f64_inputs, to_torch

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rsm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_routed_slot_amd import rsm as r
    r.load()
    return r


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def poison_pool(nbytes=1 << 28):
    """Fill freed device memory with NaN so that any read of a buffer the library did not
    write (workspace, outputs) shows up as a non-finite result."""
    junk = torch.full((nbytes // 4,), float("nan"), device="cuda")
    del junk


def run_forward(rsm, d, K, C, want_idx=True):
    poison_pool()
    t = dev_inputs(d, "cuda")
    B, T, Hh, _ = d["q"].shape
    out = torch.full((B, T, Hh, d["v"].shape[-1]), float("nan"), device="cuda")
    o, H, idx = rsm.forward_chunked(t["q"], t["k"], t["z"], t["v"], t["f"], K, C=C, H0=t["H0"],
                                    want_idx=want_idx, out=out)
    torch.cuda.synchronize()
    return o.cpu().numpy(), H.cpu().numpy(), (idx.cpu().numpy() if want_idx else None)


def compare_forward(d, K, o, H, idx, sl=slice(None), what=""):
    r = f64_inputs(d, sl)
    ro, rH, ridx = oracle.forward(r["q"], r["k"], r["z"], r["v"], r["f"], K, H0=r["H0"])
    tol = TOL[d["dtype"]]
    assert np.array_equal(idx[sl], ridx), f"{what}: top-K indices differ"
    scale = float(np.max(np.abs(ro)))
    eo = check_close(o[sl], ro, scale, tol, f"{what} o")
    eh = check_close(H[sl], rH, scale, tol, f"{what} H_final")
    log(f"{what}: max|o|={scale:.3e} err_o={eo:.3e} ({eo / scale:.2e} rel) err_H={eh:.3e} "
        f"(vs max|H| {eh / max(1e-30, float(np.max(np.abs(rH)))):.2e})")


# ------------------------------------------------------------------------------- router
ROUTE_CASES = ["tiny_f32", "fwd_b8_t2048", "long_t32768", "sweep_dense", "sweep_swa", "sweep_topk"]


@pytest.mark.parametrize("name", ROUTE_CASES)
def test_route_workloads(rsm, name):
    log(f"route {name}")
    d = gen.make_workload(name)
    K = d["K"]
    z = to_torch(d["z"], d["dtype"], "cuda")
    idx, score = rsm.route_topk(z, K)
    torch.cuda.synchronize()
    ridx, rscore = oracle.route_topk(gen.as_f64(d["z"], d["dtype"]), K)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    np.testing.assert_allclose(score.cpu().numpy(), rscore, rtol=2e-6, atol=1e-30)


@pytest.mark.parametrize("M", [16, 32, 64, 128, 256])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_route_ties_and_signed_zeros(rsm, M, dtype):
    log(f"route ties M={M} {dtype}")
    rng = np.random.default_rng(M)
    z = (rng.integers(-4, 5, size=(3, 50, 4, M)) * 0.25).astype(np.float32)
    z[rng.random(z.shape) < 0.15] = -0.0
    z[0, 0, 0, :] = 1.0                                 # all equal
    enc = gen.bf16_bits(z) if dtype == "bf16" else z
    for K in sorted({1, 3, M // 2, M - 1, M}):
        idx, _ = rsm.route_topk(to_torch(enc, dtype, "cuda"), K, want_score=False)
        ridx, _ = oracle.route_topk(gen.as_f64(enc, dtype), K)
        assert np.array_equal(idx.cpu().numpy(), ridx), f"K={K}"


@pytest.mark.parametrize("M", [16, 32, 64, 128])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_route_noisy_ties_and_signed_zeros(rsm, M, dtype):
    """Noisy logits z + g whose fp32 sums tie exactly (and are -0 or +0): the selection by
    value with ties to the lower slot, K <= 16 (value keys with the tie fix-up) and above."""
    log(f"noisy route ties M={M} {dtype}")
    rng = np.random.default_rng(100 + M)
    z = (rng.integers(-4, 5, size=(2, 40, 3, M)) * 0.25).astype(np.float32)
    z[rng.random(z.shape) < 0.2] = -0.0
    g = (rng.integers(-2, 3, size=z.shape) * 0.25).astype(np.float32)
    g[rng.random(g.shape) < 0.2] = -0.0
    z[0, 0, 0, :] = 0.5
    g[0, 0, 0, :] = 0.0                                 # all sums equal
    enc = gen.bf16_bits(z) if dtype == "bf16" else z
    for K in sorted({1, 3, 8, 16, M // 2, M - 1} - {0}):
        if K > M:
            continue
        idx, _ = rsm.route_topk(to_torch(enc, dtype, "cuda"), K, want_score=False, noise=torch.from_numpy(g).cuda())
        ridx, _ = oracle.route_topk(gen.as_f64(enc, dtype), K, noise=g.astype(np.float64))
        assert np.array_equal(idx.cpu().numpy(), ridx), f"K={K}"


# ------------------------------------------------------------------------------- forward
SMALL = [
    # dtype, B, T, Hh, M, Dv, K, C, H0
    ("f32", 1, 256, 2, 16, 16, 4, 16, False),
    ("f32", 2, 200, 3, 64, 128, 16, 64, True),
    ("bf16", 2, 200, 3, 64, 128, 16, 64, True),
    ("bf16", 1, 150, 4, 128, 64, 8, 64, True),
    ("bf16", 1, 100, 2, 32, 32, 5, 32, False),
    ("bf16", 2, 77, 2, 16, 16, 4, 16, True),
    ("f32", 1, 90, 2, 128, 64, 128, 32, True),
    ("bf16", 1, 70, 1, 64, 256, 16, 16, True),
    ("f32", 1, 130, 2, 32, 32, 32, 64, True),
    ("bf16", 3, 1, 2, 64, 128, 16, 64, True),
    # K = M = 128, bf16: the dense mode (alphas from z and f in the passes, no route):
    # 2 segments with the in-pass fold, 8 with the fold kernel, one segment, a ragged tail
    ("bf16", 1, 130, 4, 128, 64, 128, 64, True),
    ("bf16", 1, 1000, 1, 128, 64, 128, 64, True),
    ("bf16", 64, 40, 4, 128, 64, 128, 32, False),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "-".join(map(str, c)))
def test_forward_small(rsm, case):
    dtype, B, T, Hh, M, Dv, K, C, h0 = case
    log(f"forward small {case}")
    d = gen.make_inputs(B, T, Hh, M, Dv, dtype, seed=zlib.crc32(repr(case).encode()) % 1000, h0=h0)
    o, H, idx = run_forward(rsm, d, K, C)
    compare_forward(d, K, o, H, idx, what=str(case))


@pytest.mark.parametrize("C", [16, 32, 64])
def test_forward_chunk_size_invariance(rsm, C):
    log(f"chunk invariance C={C}")
    d = gen.make_inputs(2, 192, 2, 64, 128, "bf16", seed=5, h0=True)
    o, H, idx = run_forward(rsm, d, 16, C)
    compare_forward(d, 16, o, H, idx, what=f"C={C}")


def test_forward_cyclic_swa_limit(rsm):
    log("forward cyclic one-hot router, f = -inf")
    d = gen.make_inputs(1, 300, 2, 128, 64, "bf16", seed=6, router="cyclic", h0=True)
    o, H, idx = run_forward(rsm, d, 1, 64)
    compare_forward(d, 1, o, H, idx, what="cyclic")


def test_forward_unsafe_chunks_take_exact_path(rsm):
    """Dense routing with f = -inf on every token: the decay product of every slot in a
    chunk underflows, so every chunk is evaluated token by token with exact alphas."""
    log("forward unsafe chunks")
    d = gen.make_inputs(1, 160, 2, 16, 32, "f32", seed=7, h0=True)
    d["f"][:] = -np.inf
    d["f"][0, 40:70, 0] = -0.5                          # a mix of safe and unsafe chunks
    o, H, idx = run_forward(rsm, d, 16, 32)
    compare_forward(d, 16, o, H, idx, what="unsafe")


def test_forward_never_selected_slots_bitwise(rsm):
    log("never-selected slots keep H0 bits")
    d = gen.make_inputs(2, 333, 2, 64, 128, "bf16", seed=8, h0=True)
    z = gen.bf16_to_f32(d["z"]).copy()
    z[..., 40:] -= 50.0
    d["z"] = gen.bf16_bits(z)
    d["H0"][..., 41, :] = -0.0
    o, H, idx = run_forward(rsm, d, 16, 64)
    assert idx.max() < 40
    assert np.array_equal(H[..., 40:, :].view(np.uint32), d["H0"][..., 40:, :].view(np.uint32))
    compare_forward(d, 16, o, H, idx, what="never-selected")


def test_forward_deterministic(rsm):
    log("determinism")
    d = gen.make_inputs(2, 256, 4, 64, 128, "bf16", seed=9, h0=True)
    a = run_forward(rsm, d, 16, 64)
    b = run_forward(rsm, d, 16, 64)
    for x, y in zip(a, b):
        assert np.array_equal(x.view(np.uint32) if x.dtype != np.int32 else x,
                              y.view(np.uint32) if y.dtype != np.int32 else y)


def test_forward_split_sequence_resumes(rsm):
    log("forward(T1) -> forward(T2, H0=H) == forward(T1+T2)")
    d = gen.make_inputs(2, 256, 2, 64, 128, "bf16", seed=10)
    t = dev_inputs(d, "cuda")
    o, H, _ = rsm.forward_chunked(t["q"], t["k"], t["z"], t["v"], t["f"], 16, C=64)
    T1 = 100
    sl1 = (slice(None), slice(0, T1))
    sl2 = (slice(None), slice(T1, None))
    o1, H1, _ = rsm.forward_chunked(*(t[n][sl1] for n in "qkzvf"), 16, C=64)
    o2, H2, _ = rsm.forward_chunked(*(t[n][sl2] for n in "qkzvf"), 16, C=64, H0=H1)
    torch.cuda.synchronize()
    scale = float(o.abs().max())
    check_close(torch.cat([o1, o2], 1).cpu().numpy(), o.cpu().numpy().astype(np.float64), scale, TOL["bf16"],
                "split o")
    check_close(H2.cpu().numpy(), H.cpu().numpy().astype(np.float64), scale, TOL["bf16"], "split H")


@pytest.mark.parametrize("case", [("bf16", 1, 8192, 3, 64, 128, 16), ("bf16", 8, 1024, 8, 64, 128, 16),
                                  ("bf16", 2, 640, 2, 64, 128, 16), ("f32", 1, 2048, 2, 32, 64, 16),
                                  ("bf16", 1, 2048, 2, 128, 64, 128), ("bf16", 1, 1500, 2, 256, 128, 32)],
                         ids=lambda c: "-".join(map(str, c)))
def test_forward_inplace_state_with_segments(rsm, case):
    """H_out is the H0 buffer while the sequence is cut into segments: workgroups of early
    segments may start after the last segment's workgroup has written H_out, so the call
    must read the initial state from a copy (128 segments folded by the fold kernel; 4
    folded inside the second pass; 5; fp32; the dense mode at M = 128; chunked M = 256)."""
    dtype, B, T, Hh, M, Dv, K = case
    log(f"in-place state with segments {case}")
    d = gen.make_inputs(B, T, Hh, M, Dv, dtype, seed=zlib.crc32(repr(case).encode()) % 1000, h0=True)
    t = dev_inputs(d, "cuda")
    H = t["H0"].clone()
    o, H2, idx = rsm.forward_chunked(t["q"], t["k"], t["z"], t["v"], t["f"], K, C=64, H0=H, state_out=H,
                                     want_idx=True)
    torch.cuda.synchronize()
    assert H2.data_ptr() == H.data_ptr()
    compare_forward(d, K, o.cpu().numpy(), H.cpu().numpy(), idx.cpu().numpy(), what=f"in place {case}")


def test_forward_empty(rsm):
    log("empty sequence")
    H0 = torch.randn(2, 3, 64, 128, device="cuda")
    q = torch.empty(2, 0, 3, 64, device="cuda", dtype=torch.bfloat16)
    v = torch.empty(2, 0, 3, 128, device="cuda", dtype=torch.bfloat16)
    f = torch.empty(2, 0, 3, device="cuda")
    o, H, idx = rsm.forward_chunked(q, q, q, v, f, 16, C=64, H0=H0, want_idx=True)
    torch.cuda.synchronize()
    assert o.shape == (2, 0, 3, 128) and torch.equal(H, H0)
    o, H, _ = rsm.forward_chunked(q, q, q, v, f, 16, C=64)
    torch.cuda.synchronize()
    assert torch.count_nonzero(H) == 0


WORKLOADS = ["tiny_f32", "fwd_b8_t2048", "long_t32768", "sweep_dense", "sweep_swa", "sweep_topk"]


@pytest.mark.parametrize("name", WORKLOADS)
def test_forward_workloads(rsm, name):
    log(f"forward workload {name}")
    d = gen.make_workload(name)
    o, H, idx = run_forward(rsm, d, d["K"], d["C"])
    compare_forward(d, d["K"], o, H, idx, what=name)


# ------------------------------------------------------------------------------- decode
DEC = [
    # dtype, B, Hh, M, Dv, K
    ("f32", 3, 2, 16, 16, 4),
    ("bf16", 4, 3, 64, 128, 16),
    ("f32", 2, 2, 128, 64, 8),
    ("bf16", 2, 2, 32, 256, 32),
    ("bf16", 5, 1, 128, 32, 128),
    ("bf16", 3, 4, 128, 256, 16),
    ("bf16", 2, 4, 256, 256, 32),   # the pages' default layer: 4 heads, 256 slots, top-32, head dim 256
    ("f32", 2, 2, 256, 64, 16),
]


@pytest.mark.parametrize("case", DEC, ids=lambda c: "-".join(map(str, c)))
def test_decode_steps(rsm, case):
    dtype, B, Hh, M, Dv, K = case
    log(f"decode {case}")
    rng = np.random.default_rng(11)
    H = torch.from_numpy(rng.standard_normal((B, Hh, M, Dv), dtype=np.float32)).cuda()
    H[..., 0, :3] = -0.0
    tol = TOL[dtype]
    for step in range(12):
        s = gen.decode_step_inputs(rng, B, Hh, M, Dv, dtype)
        if step == 5:
            s["f"][:] = -np.inf
        Hprev = H.clone()
        t = {n: to_torch(s[n], dtype, "cuda") for n in "qkzv"}
        o, idx = rsm.decode_step(t["q"], t["k"], t["z"], t["v"], torch.from_numpy(s["f"]).cuda(), H, K,
                                 want_idx=True)
        torch.cuda.synchronize()
        Hr = Hprev.cpu().numpy().astype(np.float64)
        ro, ridx = oracle.decode_step(*(gen.as_f64(s[n], dtype) for n in "qkzv"), s["f"].astype(np.float64), Hr, K)
        idx_n = idx.cpu().numpy()
        assert np.array_equal(idx_n, ridx)
        scale = float(np.max(np.abs(ro)))
        check_close(o.cpu().numpy(), ro, scale, tol, f"decode o step {step}")
        check_close(H.cpu().numpy(), Hr, scale, tol, f"decode H step {step}")
        # rows not selected: bitwise unchanged
        keep = np.ones((B, Hh, M), dtype=bool)
        np.put_along_axis(keep, idx_n.astype(np.int64), False, axis=-1)
        hn, hp = H.cpu().numpy(), Hprev.cpu().numpy()
        assert np.array_equal(hn[keep].view(np.uint32), hp[keep].view(np.uint32))


def test_prefill_then_decode_matches_longer_forward(rsm):
    log("prefill + decode == forward")
    d = gen.make_inputs(2, 200, 4, 64, 128, "bf16", seed=12)
    t = dev_inputs(d, "cuda")
    K, T1 = 16, 150
    o, H, _ = rsm.forward_chunked(t["q"], t["k"], t["z"], t["v"], t["f"], K, C=64)
    _, Hs, _ = rsm.forward_chunked(*(t[n][:, :T1] for n in "qkzvf"), K, C=64)
    Hs = Hs.contiguous()
    outs = []
    for tt in range(T1, 200):
        od, _ = rsm.decode_step(*(t[n][:, tt] for n in "qkzvf"), Hs, K)
        outs.append(od)
    torch.cuda.synchronize()
    scale = float(o.abs().max())
    check_close(torch.stack(outs, 1).cpu().numpy(), o[:, T1:].cpu().numpy().astype(np.float64), scale,
                TOL["bf16"], "decode vs forward o")
    check_close(Hs.cpu().numpy(), H.cpu().numpy().astype(np.float64), scale, TOL["bf16"], "decode vs forward H")


def test_decode_workload_prefill_and_steps(rsm):
    """Batched decode: 256 sequences x 16 heads, M64 Dv128 K16; prefill T=512 by the
    chunked forward, then all 1024 single-token steps, the run bench.py times.  On four
    sampled sequences the oracle follows its own float64 prefill through every step (end to
    end: o checked at every step, the state at steps 256, 512 and 1024), and at those
    steps it also takes one step from the GPU's fp32 state (the decode kernel alone)."""
    log("decode workload: prefill")
    w = gen.WORKLOADS["decode_b256"]
    d = gen.make_workload("decode_b256")
    t = dev_inputs(d, "cuda")
    K = w.K
    o, H, idx = rsm.forward_chunked(t["q"], t["k"], t["z"], t["v"], t["f"], K, C=w.C, want_idx=True)
    torch.cuda.synchronize()
    samp = np.array([0, 37, 128, 255])
    samp_t = torch.from_numpy(samp).cuda()
    r = f64_inputs(d, samp)
    ro, rH, ridx = oracle.forward(r["q"], r["k"], r["z"], r["v"], r["f"], K)
    assert np.array_equal(idx.cpu().numpy()[samp], ridx)
    scale = float(np.max(np.abs(ro)))
    check_close(o.cpu().numpy()[samp], ro, scale, TOL["bf16"], "prefill o")
    check_close(H.cpu().numpy()[samp], rH, scale, TOL["bf16"], "prefill H")
    rng = np.random.default_rng(1000 + w.seed)
    steps = w.extra["steps"]
    checkpoints = {256, 512, steps}
    worst = 0.0
    for step in range(1, steps + 1):
        s = gen.decode_step_inputs(rng, w.B, w.Hh, w.M, w.Dv, "bf16")
        st = {n: to_torch(s[n], "bf16", "cuda") for n in "qkzv"}
        args = [gen.as_f64(s[n][samp], "bf16") for n in "qkzv"] + [s["f"][samp].astype(np.float64)]
        if step in checkpoints:  # the GPU state entering this step
            Hgpu = H.index_select(0, samp_t).cpu().numpy().astype(np.float64)
        od, idd = rsm.decode_step(st["q"], st["k"], st["z"], st["v"], torch.from_numpy(s["f"]).cuda(), H, K,
                                  want_idx=True)
        o_e2e, i_e2e = oracle.decode_step(*args, rH, K)
        od_s = od.index_select(0, samp_t).cpu().numpy()
        assert np.array_equal(idd.index_select(0, samp_t).cpu().numpy(), i_e2e), f"decode step {step}: top-K"
        sc = float(np.max(np.abs(o_e2e)))
        e = check_close(od_s, o_e2e, sc, TOL["bf16"], f"decode e2e step {step}")
        worst = max(worst, e / sc)
        if step in checkpoints:
            o_dec, _ = oracle.decode_step(*args, Hgpu, K)
            check_close(od_s, o_dec, sc, TOL["bf16"], f"decode-only step {step}")
            Hs = H.index_select(0, samp_t).cpu().numpy()
            check_close(Hs, Hgpu, sc, TOL["bf16"], f"decode-only state step {step}")
            eh = check_close(Hs, rH, sc, TOL["bf16"], f"decode e2e state step {step}")
            log(f"decode step {step}: worst e2e o error so far {worst:.2e} of max|o|, state {eh / sc:.2e}")


# ------------------------------------------------------------ router and decay variants
VARIANTS = [  # score, normalize, per-slot f, noise
    ("softmax", False, False, False),
    ("sigmoid", True, False, False),
    ("sigmoid", False, True, False),
    ("sigmoid", False, False, True),
    ("softmax", True, True, True),
]
VAR_SHAPES = [  # dtype, B, T, Hh, M, Dv, K, C
    ("bf16", 2, 200, 3, 64, 128, 16, 64),
    ("f32", 1, 130, 2, 32, 32, 8, 32),
    ("bf16", 1, 90, 2, 128, 64, 24, 32),
    ("bf16", 2, 77, 2, 16, 16, 16, 16),
    ("bf16", 1, 70, 2, 256, 64, 32, 64),   # M = 256: recurrent form
    ("f32", 1, 45, 2, 256, 32, 100, 64),   # M = 256, K > 64 (several route entries per lane)
]


def _vid(v):
    return "-".join(str(x) for x in v)


@pytest.mark.parametrize("shape", VAR_SHAPES, ids=_vid)
@pytest.mark.parametrize("var", VARIANTS, ids=_vid)
def test_variant_route_and_forward(rsm, var, shape):
    score, normalize, per_slot, noisy = var
    dtype, B, T, Hh, M, Dv, K, C = shape
    log(f"variant {var} forward {shape}")
    seed = zlib.crc32(repr((var, shape)).encode()) % 1000
    d = gen.make_inputs(B, T, Hh, M, Dv, dtype, seed=seed, h0=True)
    ex = gen.variant_inputs(np.random.default_rng(seed + 1), d["z"].shape)
    noise = ex["noise"] if noisy else None
    t = dev_inputs(d, "cuda")
    f = torch.from_numpy(ex["f_slot"]).cuda() if per_slot else t["f"]
    nz = torch.from_numpy(noise).cuda() if noisy else None
    # router alone: indices bit-exact, weights to fp32 rounding
    idx, sc = rsm.route_topk(t["z"], K, score=score, normalize=normalize, noise=nz)
    torch.cuda.synchronize()
    zr = gen.as_f64(d["z"], dtype)
    nr = None if noise is None else noise.astype(np.float64)
    ridx, rsc = oracle.route_topk(zr, K, noise=nr, score=score, normalize=normalize)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    np.testing.assert_allclose(sc.cpu().numpy(), rsc, rtol=2e-5, atol=1e-7)
    # forward
    poison_pool()
    out = torch.full((B, T, Hh, Dv), float("nan"), device="cuda")
    o, H, gidx = rsm.forward_chunked(t["q"], t["k"], t["z"], t["v"], f, K, C=C, H0=t["H0"], want_idx=True,
                                     out=out, score=score, normalize=normalize, noise=nz)
    torch.cuda.synchronize()
    r = f64_inputs(d)
    fr = ex["f_slot"].astype(np.float64) if per_slot else r["f"]
    ro, rH, ri = oracle.forward(r["q"], r["k"], r["z"], r["v"], fr, K, H0=r["H0"], noise=nr, score=score,
                                normalize=normalize)
    assert np.array_equal(gidx.cpu().numpy(), ri)
    scale = float(np.max(np.abs(ro)))
    eo = check_close(o.cpu().numpy(), ro, scale, TOL[dtype], f"variant {var} o")
    check_close(H.cpu().numpy(), rH, scale, TOL[dtype], f"variant {var} H")
    log(f"  err_o {eo / scale:.2e} rel")


@pytest.mark.parametrize("var", VARIANTS, ids=_vid)
@pytest.mark.parametrize("case", [("bf16", 3, 4, 64, 128, 16), ("f32", 2, 2, 128, 64, 40), ("bf16", 4, 2, 16, 32, 3),
                                  ("bf16", 2, 4, 256, 256, 32)], ids=_vid)
def test_variant_decode(rsm, var, case):
    score, normalize, per_slot, noisy = var
    dtype, B, Hh, M, Dv, K = case
    log(f"variant {var} decode {case}")
    rng = np.random.default_rng(zlib.crc32(repr((var, case)).encode()) % 1000)
    H = torch.from_numpy(rng.standard_normal((B, Hh, M, Dv), dtype=np.float32)).cuda()
    for step in range(6):
        s = gen.decode_step_inputs(rng, B, Hh, M, Dv, dtype)
        ex = gen.variant_inputs(rng, (B, Hh, M))
        f = ex["f_slot"] if per_slot else s["f"]
        if step == 3:
            f = np.full_like(f, -np.inf)
        noise = ex["noise"] if noisy else None
        Hprev = H.clone()
        t = {n: to_torch(s[n], dtype, "cuda") for n in "qkzv"}
        o, idx = rsm.decode_step(t["q"], t["k"], t["z"], t["v"], torch.from_numpy(np.ascontiguousarray(f)).cuda(),
                                 H, K, want_idx=True, score=score, normalize=normalize,
                                 noise=None if noise is None else torch.from_numpy(noise).cuda())
        torch.cuda.synchronize()
        Hr = Hprev.cpu().numpy().astype(np.float64)
        ro, ridx = oracle.decode_step(*(gen.as_f64(s[n], dtype) for n in "qkzv"), f.astype(np.float64), Hr, K,
                                      noise=None if noise is None else noise.astype(np.float64), score=score,
                                      normalize=normalize)
        assert np.array_equal(idx.cpu().numpy(), ridx)
        scale = float(np.max(np.abs(ro)))
        check_close(o.cpu().numpy(), ro, scale, TOL[dtype], f"variant decode o step {step}")
        check_close(H.cpu().numpy(), Hr, scale, TOL[dtype], f"variant decode H step {step}")


@pytest.mark.parametrize("name", ["fwd_b8_t2048", "long_t32768"])
@pytest.mark.parametrize("noisy", [False, True])
def test_variant_forward_workloads(rsm, name, noisy):
    """The benchmarked variant configurations at full size: softmax scores renormalised over
    the selected slots with per-slot decay rates, with and without logit noise."""
    log(f"variant forward workload {name} noise={noisy}")
    d = gen.make_workload(name)
    K, C, dtype = d["K"], d["C"], d["dtype"]
    ex = gen.variant_inputs(np.random.default_rng(77), d["z"].shape)
    t = dev_inputs(d, "cuda")
    nz = torch.from_numpy(ex["noise"]).cuda() if noisy else None
    poison_pool()
    o, H, idx = rsm.forward_chunked(t["q"], t["k"], t["z"], t["v"], torch.from_numpy(ex["f_slot"]).cuda(), K, C=C,
                                    H0=t["H0"], want_idx=True, score="softmax", normalize=True, noise=nz)
    torch.cuda.synchronize()
    r = f64_inputs(d)
    ro, rH, ri = oracle.forward(r["q"], r["k"], r["z"], r["v"], ex["f_slot"].astype(np.float64), K, H0=r["H0"],
                                noise=ex["noise"].astype(np.float64) if noisy else None, score="softmax",
                                normalize=True)
    assert np.array_equal(idx.cpu().numpy(), ri)
    scale = float(np.max(np.abs(ro)))
    eo = check_close(o.cpu().numpy(), ro, scale, TOL[dtype], f"{name} variant o")
    check_close(H.cpu().numpy(), rH, scale, TOL[dtype], f"{name} variant H")
    log(f"  err_o {eo / scale:.2e} rel")


@pytest.mark.parametrize("var", VARIANTS, ids=_vid)
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_variant_route_wide_rows(rsm, var, dtype):
    """The router at the pages' default slot count (M = 256, K = 32), every variant."""
    score, normalize, _, noisy = var
    log(f"variant route M=256 {var} {dtype}")
    rng = np.random.default_rng(zlib.crc32(repr((var, dtype)).encode()) % 1000)
    z = (rng.standard_normal((2, 37, 4, 256), dtype=np.float32) * 1.5).astype(np.float32)
    z[0, :3] = np.round(z[0, :3] * 2) / 2     # ties
    enc = gen.bf16_bits(z) if dtype == "bf16" else z
    noise = gen.variant_inputs(rng, z.shape)["noise"] if noisy else None
    idx, sc = rsm.route_topk(to_torch(enc, dtype, "cuda"), 32, score=score, normalize=normalize,
                             noise=None if noise is None else torch.from_numpy(noise).cuda())
    torch.cuda.synchronize()
    ridx, rsc = oracle.route_topk(gen.as_f64(enc, dtype), 32, noise=None if noise is None else noise.astype(np.float64),
                                  score=score, normalize=normalize)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    np.testing.assert_allclose(sc.cpu().numpy(), rsc, rtol=2e-5, atol=1e-7)


# ------------------------------------------------ forward at M = 256
# bf16 with K <= 32 runs chunked (chunks of 32, 64-column tiles); fp32 and K > 32 run in the
# recurrent form.
M256_CASES = [  # dtype, B, T, Hh, Dv, K, h0, f = -inf tokens
    ("bf16", 2, 70, 2, 64, 32, False, False),
    ("bf16", 1, 150, 2, 256, 32, True, True),    # four column tiles, segments, exact chunks
    ("f32", 1, 33, 1, 16, 100, True, False),     # recurrent: K > 64, several route entries per lane
    ("f32", 1, 5, 3, 32, 256, False, False),     # recurrent: K = M, every slot every token
    ("bf16", 3, 1, 2, 128, 8, True, False),      # one token
    ("bf16", 2, 130, 2, 32, 16, True, True),     # 32-column tile (two state waves per column tile)
    ("bf16", 1, 64, 3, 16, 1, False, False),     # 16-column tile, top-1
    ("bf16", 4, 96, 4, 128, 32, True, False),    # two column tiles, two segments
    ("bf16", 16, 100, 4, 256, 32, False, False), # 256 tiles: one segment
    ("bf16", 1, 97, 1, 64, 40, True, False),     # recurrent: K > 32
]


@pytest.mark.parametrize("case", M256_CASES, ids=_vid)
def test_forward_m256(rsm, case):
    dtype, B, T, Hh, Dv, K, h0, neg_inf = case
    log(f"forward M256 {case}")
    d = gen.make_inputs(B, T, Hh, 256, Dv, dtype, seed=zlib.crc32(repr(case).encode()) % 1000, h0=h0)
    if neg_inf:
        d["f"][:, T // 3: T // 3 + 7] = -np.inf
    o, H, idx = run_forward(rsm, d, K, 64)
    compare_forward(d, K, o, H, idx, what=f"M256 {case}")
    if h0:  # slots never selected keep their initial rows bit for bit
        never = np.ones((B, Hh, 256), dtype=bool)
        for b in range(B):
            for h in range(Hh):
                never[b, h, np.unique(idx[b, :, h, :])] = False
        assert np.array_equal(H[never], d["H0"][never])


def test_forward_default_layer_sampled(rsm):
    """The pages' default layer at its bench size (B16 T2048 Hh4 M256 d_v256 K32, chunked):
    indices, outputs and final states of sequences 0 and 15 against the oracle."""
    B, T, Hh, M, Dv, K = 16, 2048, 4, 256, 256, 32
    log(f"forward default layer B{B} T{T} Hh{Hh} M{M} Dv{Dv} K{K}")
    d = gen.make_inputs(B, T, Hh, M, Dv, "bf16", 11)
    o, H, idx = run_forward(rsm, d, K, 64)
    for b in (0, B - 1):
        compare_forward(d, K, o, H, idx, sl=slice(b, b + 1), what=f"default layer b={b}")


def test_forward_m256_inplace_and_empty(rsm):
    log("forward M256: H_out = H0 in place, and T = 0")
    d = gen.make_inputs(2, 40, 2, 256, 64, "bf16", seed=5, h0=True)
    t = dev_inputs(d, "cuda")
    H = t["H0"].clone()
    o, H2, idx = rsm.forward_chunked(t["q"], t["k"], t["z"], t["v"], t["f"], 32, H0=H, state_out=H,
                                     want_idx=True)
    torch.cuda.synchronize()
    assert H2.data_ptr() == H.data_ptr()
    compare_forward(d, 32, o.cpu().numpy(), H.cpu().numpy(), idx.cpu().numpy(), what="M256 in place")
    o_ns, H_ns, _ = rsm.forward_chunked(t["q"], t["k"], t["z"], t["v"], t["f"], 32, H0=t["H0"], want_state=False)
    torch.cuda.synchronize()
    assert H_ns is None
    ro, _, _ = oracle.forward(*(gen.as_f64(d[n], "bf16") for n in "qkzv"), d["f"], 32, H0=d["H0"])
    check_close(o_ns.cpu().numpy(), ro, float(np.max(np.abs(ro))), TOL["bf16"], "M256 without state output")
    e = gen.make_inputs(2, 0, 2, 256, 64, "bf16", seed=6, h0=True)
    te = dev_inputs(e, "cuda")
    o0, H0o, _ = rsm.forward_chunked(te["q"], te["k"], te["z"], te["v"], te["f"], 32, H0=te["H0"])
    torch.cuda.synchronize()
    assert o0.numel() == 0 and np.array_equal(H0o.cpu().numpy(), e["H0"])
