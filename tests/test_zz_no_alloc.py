"""The no-allocation entry point (rsm_forward_chunked_noalloc) against the workspace entry
point (rsm_forward_chunked) it shares its kernels with: bit-identical outputs, final state
and indices on two calls in a row on one device, the second with a smaller input (the
fixed scratch array keeps the first call's contents), plus the size limit."""
import numpy as np
import pytest

from sparse_routed_slot_amd import inputs as gen
from tests._util import dev_inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rsm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_routed_slot_amd import rsm as r
    r.load()
    return r


def _bits(x):
    a = x.cpu().numpy()
    return a.view(np.uint32) if a.dtype == np.float32 else a


def test_noalloc_matches_workspace_entry_twice(rsm):
    # first call: the bench workload's shape (segments, folded in the second pass); second
    # call: a smaller, ragged one (128 segments folded by the fold kernel, tail chunk)
    for case in [("bf16", 8, 2048, 8, 64, 128, 16, 64), ("bf16", 1, 3001, 3, 64, 128, 16, 64)]:
        dtype, B, T, Hh, M, Dv, K, C = case
        print(f"no-alloc vs workspace entry {case}", flush=True)
        d = gen.make_inputs(B, T, Hh, M, Dv, dtype, seed=77 + T, h0=True)
        t = dev_inputs(d, "cuda")
        need = rsm.forward_workspace_bytes(t["q"].dtype, B, T, Hh, M, Dv, C, K)
        assert 0 < need <= rsm.noalloc_scratch_bytes()
        o1, H1, i1 = rsm.forward_chunked(t["q"], t["k"], t["z"], t["v"], t["f"], K, C=C, H0=t["H0"], want_idx=True)
        o2, H2, i2 = rsm.forward_chunked_noalloc(t["q"], t["k"], t["z"], t["v"], t["f"], K, C=C, H0=t["H0"],
                                                 want_idx=True)
        torch.cuda.synchronize()
        assert np.array_equal(_bits(o1), _bits(o2)), f"{case}: o differs"
        assert np.array_equal(_bits(H1), _bits(H2)), f"{case}: final state differs"
        assert np.array_equal(_bits(i1), _bits(i2)), f"{case}: indices differ"


def test_noalloc_rejects_oversized_problem(rsm):
    # refused on the host before any device call: the decode prefill shape needs ~150 MB
    q = torch.empty(256, 512, 16, 64, dtype=torch.bfloat16, device="cuda")
    v = torch.empty(256, 512, 16, 128, dtype=torch.bfloat16, device="cuda")
    f = torch.empty(256, 512, 16, device="cuda")
    assert rsm.forward_workspace_bytes(q.dtype, 256, 512, 16, 64, 128, 64, 16) > rsm.noalloc_scratch_bytes()
    with pytest.raises(rsm.RSMError, match="-9"):
        rsm.forward_chunked_noalloc(q, q, q, v, f, 16, C=64)
