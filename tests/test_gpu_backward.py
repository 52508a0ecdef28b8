"""GPU backward pass (rsm_backward) against the float64 oracle gradients (oracle.backward),
through the C ABI.  Gradients are computed in fp32 throughout; the tolerance is relative to
the largest magnitude of each gradient tensor (see the tolerance note below)."""
import sys
import zlib

import numpy as np
import pytest

from oracle import oracle
from sparse_routed_slot_amd import inputs as gen
from tests._util import dev_inputs, f64_inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

# Tolerance on every gradient: max|delta| <= BWD_TOL * max|ref| of that gradient, the fp32
# bound the outputs are held to.  The inputs are exact on both sides (bf16 values are exact
# in fp32 and fp64) and the GPU computes in fp32 throughout (no bf16 operands), so the error
# is fp32 rounding (2^-24 per operation) grown over the T steps of the state and its
# gradient, plus the cancellation in dg = D - k u; measured up to 2e-6 at T = 2048.
BWD_TOL = 1e-5


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


def _upstream(shape_o, shape_h, seed, with_dht):
    rng = np.random.default_rng(seed)
    dO = rng.standard_normal(shape_o).astype(np.float32)
    dHT = rng.standard_normal(shape_h).astype(np.float32) if with_dht else None
    return dO, dHT


def run_and_compare(rsm, d, K, dO, dHT, what, sl=None):
    t = dev_inputs(d, "cuda")
    dO_t = torch.from_numpy(dO).cuda()
    dHT_t = torch.from_numpy(dHT).cuda() if dHT is not None else None
    got = rsm.backward(t["q"], t["k"], t["z"], t["v"], t["f"], K, dO_t, H0=t["H0"], dHT=dHT_t)
    torch.cuda.synchronize()
    got = [x.cpu().numpy() for x in got]
    r = f64_inputs(d, sl if sl is not None else slice(None))
    dOs = dO[sl] if sl is not None else dO
    dHs = (dHT[sl] if sl is not None else dHT) if dHT is not None else None
    ref = oracle.backward(r["q"], r["k"], r["z"], r["v"], r["f"], K, dOs.astype(np.float64), H0=r["H0"],
                          dHT=None if dHs is None else dHs.astype(np.float64))
    names = ("dq", "dk", "dz", "dv", "df", "dH0")
    msg = []
    for n, g, rr in zip(names, got, ref):
        g = g[sl] if sl is not None else g
        assert np.all(np.isfinite(g)), f"{what} {n}: non-finite"
        scale = max(float(np.max(np.abs(rr))), 1e-30)
        err = float(np.max(np.abs(g.astype(np.float64) - rr))) if g.size else 0.0
        msg.append(f"{n} {err / scale:.1e}")
        assert err <= BWD_TOL * scale, f"{what} {n}: max|delta| {err:.3e} > {BWD_TOL} * {scale:.3e}"
    log(f"{what}: " + ", ".join(msg))


# The passes cut each head's tokens into up to S segments (T / S >= 64, about 2048 workgroups):
# T = 256 at M = 16 runs 4, T = 130 runs 2, T <= 100 runs one.
SMALL = [  # dtype, B, T, Hh, M, Dv, K, H0, dHT, f=-inf tokens
    ("f32", 1, 256, 2, 16, 16, 4, False, False, False),
    ("f32", 2, 100, 3, 64, 128, 16, True, True, False),
    ("bf16", 2, 130, 2, 64, 128, 16, True, True, True),
    ("bf16", 1, 77, 2, 32, 64, 5, False, True, False),
    ("bf16", 1, 90, 2, 128, 64, 24, True, True, True),
    ("f32", 1, 60, 2, 128, 32, 128, True, False, False),
    ("bf16", 1, 40, 2, 256, 256, 32, True, True, False),
    ("bf16", 3, 1, 2, 64, 128, 16, True, True, False),
    # sequence segments walked in parallel (4 of 76, 76, 76, 73 tokens; 2 of 100 at M = 256)
    ("bf16", 1, 301, 3, 32, 32, 8, True, True, True),
    ("bf16", 1, 200, 1, 256, 64, 32, True, True, False),
    ("f32", 2, 512, 1, 16, 64, 16, False, True, False),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "-".join(map(str, c)))
def test_backward_small(rsm, case):
    dtype, B, T, Hh, M, Dv, K, h0, dht, neginf = case
    log(f"backward {case}")
    seed = zlib.crc32(repr(case).encode()) % 1000
    d = gen.make_inputs(B, T, Hh, M, Dv, dtype, seed=seed, h0=h0)
    if neginf:
        d["f"][0, T // 3, 0] = -np.inf
        d["f"][0, T // 2, 1] = -np.inf
    dO, dHT = _upstream((B, T, Hh, Dv), (B, Hh, M, Dv), seed + 1, dht)
    run_and_compare(rsm, d, K, dO, dHT, str(case))


def test_backward_tiny_workload(rsm):
    log("backward tiny_f32 workload")
    d = gen.make_workload("tiny_f32")
    w = d["workload"]
    dO, dHT = _upstream((w.B, w.T, w.Hh, w.Dv), (w.B, w.Hh, w.M, w.Dv), 7, True)
    run_and_compare(rsm, d, w.K, dO, dHT, "tiny_f32")


def test_backward_fwd_b8_t2048_sampled(rsm):
    """The training-shape layer (B8 T2048 Hh8 M64 Dv128 K16, bf16): GPU gradients of the whole
    batch, compared with the oracle on two sampled sequences (all heads)."""
    log("backward fwd_b8_t2048 (sampled sequences)")
    d = gen.make_workload("fwd_b8_t2048")
    w = d["workload"]
    dO, dHT = _upstream((w.B, w.T, w.Hh, w.Dv), (w.B, w.Hh, w.M, w.Dv), 8, True)
    run_and_compare(rsm, d, w.K, dO, dHT, "fwd_b8_t2048", sl=np.array([0, 5]))
