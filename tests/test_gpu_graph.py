"""HIP graph capture of the entry points.

A call launches kernels only (no memset, allocation or synchronisation inside the library),
so a caller may capture it in a HIP graph.  Each graph is replayed several times, with eager
work of the test's own (fills, copies) and synchronisations between the replays, and every
replay must equal the eager call bit for bit: the kernels and inputs are the same.
"""
import sys

import numpy as np
import pytest

from sparse_routed_slot_amd import inputs as gen
from tests._util import dev_inputs, to_torch

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

REPLAYS = 3


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


@pytest.mark.parametrize("variant,M,Dv,K", [(False, 64, 128, 16), (True, 64, 128, 16), (False, 128, 64, 128),
                                             (False, 256, 256, 32)],
                         ids=["default_router", "softmax_norm_noise_fslot", "dense_m128", "chunked_m256"])
def test_forward_graph_replays(rsm, variant, M, Dv, K):
    B, T, Hh, C = 2, 300, 2, 64
    log(f"graph forward B{B} T{T} Hh{Hh} M{M} Dv{Dv} K{K} C{C} variant={variant}")
    d = gen.make_inputs(B, T, Hh, M, Dv, "bf16", seed=21, h0=True)
    t = dev_inputs(d, "cuda")
    kw = {}
    f = t["f"]
    if variant:
        x = gen.variant_inputs(np.random.default_rng(22), d["z"].shape)
        f = torch.from_numpy(x["f_slot"]).cuda()
        kw = dict(score="softmax", normalize=True, noise=torch.from_numpy(x["noise"]).cuda())
    args = (t["q"], t["k"], t["z"], t["v"], f, K)
    o_e, H_e, i_e = rsm.forward_chunked(*args, C=C, H0=t["H0"], want_idx=True, **kw)
    torch.cuda.synchronize()

    ws = torch.empty(rsm.forward_workspace_bytes(torch.bfloat16, B, T, Hh, M, Dv, C, K), dtype=torch.uint8,
                     device="cuda")
    o = torch.empty((B, T, Hh, Dv), dtype=torch.float32, device="cuda")
    H = torch.empty((B, Hh, M, Dv), dtype=torch.float32, device="cuda")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        o_g, H_g, i_g = rsm.forward_chunked(*args, C=C, H0=t["H0"], want_idx=True, workspace=ws, out=o,
                                            state_out=H, **kw)
    for rep in range(REPLAYS):
        o.fill_(float("nan"))
        H.fill_(float("nan"))
        i_g.fill_(-1)
        ws.fill_(0xFF)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o_g, o_e), f"replay {rep}: o differs from the eager call"
        assert torch.equal(H_g, H_e), f"replay {rep}: H_final differs from the eager call"
        assert torch.equal(i_g, i_e), f"replay {rep}: idx differs from the eager call"
        log(f"  replay {rep}: equal")


@pytest.mark.parametrize("M,Dv,K", [(64, 128, 16), (256, 256, 32)])
def test_decode_graph_replays(rsm, M, Dv, K):
    B, Hh = 8, 4
    log(f"graph decode B{B} Hh{Hh} M{M} Dv{Dv} K{K}")
    rng = np.random.default_rng(31 + M)
    s = gen.decode_step_inputs(rng, B, Hh, M, Dv, "bf16")
    t = {n: to_torch(s[n], "bf16", "cuda") for n in ("q", "k", "z", "v")}
    f = torch.from_numpy(s["f"]).cuda()
    H0 = torch.from_numpy(rng.standard_normal((B, Hh, M, Dv), dtype=np.float32)).cuda()
    H_e = H0.clone()
    o_e, i_e = rsm.decode_step(t["q"], t["k"], t["z"], t["v"], f, H_e, K, want_idx=True)
    torch.cuda.synchronize()

    H = torch.empty_like(H0)
    o = torch.empty((B, Hh, Dv), dtype=torch.float32, device="cuda")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        o_g, i_g = rsm.decode_step(t["q"], t["k"], t["z"], t["v"], f, H, K, want_idx=True, out=o)
    for rep in range(REPLAYS):
        H.copy_(H0)
        o.fill_(float("nan"))
        i_g.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(H, H_e), f"replay {rep}: state differs from the eager step"
        assert torch.equal(o_g, o_e), f"replay {rep}: o differs from the eager step"
        assert torch.equal(i_g, i_e), f"replay {rep}: idx differs from the eager step"
        log(f"  replay {rep}: equal")
