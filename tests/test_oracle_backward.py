"""Pins of the float64 oracle's gradients (oracle.backward) against what does not depend on
its hand-written chain rule:

- central finite differences of the oracle's own forward loss, element by element;
- reverse-mode automatic differentiation (torch, float64, CPU) of the recurrence written
  out independently here, token by token, with the selection taken from a full sort;
- closed forms: a slot that is never selected keeps H0, so its row of dH0 is the sum of
  q_i dO over the tokens plus dH_T; f = -inf gives no decay-rate or logit gradient.

The loss is L = sum(dO * o) + sum(dH_T * H_final) (the vector-Jacobian product with
upstream gradients dO and dH_T).  The update and read are those of the Raven README page
("How Raven Works"): the chunked kernels the pages describe exist for training (README
kernel notes), and these gradients are what such a backward pass returns.
"""
import math

import numpy as np
import pytest

from oracle import oracle

torch = pytest.importorskip("torch")


def _topk_by_sort(z, K):
    order = sorted(range(len(z)), key=lambda i: (-z[i], i))
    return sorted(order[:K])


def _inputs(seed, B=1, T=20, Hh=2, M=8, Dv=4, spaced_z=True):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, T, Hh, M)) / math.sqrt(M)
    k = rng.standard_normal((B, T, Hh, M)) / math.sqrt(M)
    if spaced_z:  # logits at least 0.25 apart within a row: small perturbations keep the selection
        z = np.stack([rng.permutation(M) * 0.25 + rng.uniform(-0.05, 0.05, M)
                      for _ in range(B * T * Hh)]).reshape(B, T, Hh, M) - M * 0.125
    else:
        z = rng.standard_normal((B, T, Hh, M))
    v = rng.standard_normal((B, T, Hh, Dv))
    f = -np.log1p(np.exp(rng.standard_normal((B, T, Hh))))
    H0 = rng.standard_normal((B, Hh, M, Dv))
    dO = rng.standard_normal((B, T, Hh, Dv))
    dHT = rng.standard_normal((B, Hh, M, Dv))
    return dict(q=q, k=k, z=z, v=v, f=f, H0=H0, dO=dO, dHT=dHT)


def _loss(d, K):
    o, H, _ = oracle.forward(d["q"], d["k"], d["z"], d["v"], d["f"], K, H0=d["H0"])
    return float(np.sum(d["dO"] * o) + np.sum(d["dHT"] * H))


def _grads(d, K):
    dq, dk, dz, dv, df, dH0 = oracle.backward(d["q"], d["k"], d["z"], d["v"], d["f"], K, d["dO"], H0=d["H0"],
                                              dHT=d["dHT"])
    return {"q": dq, "k": dk, "z": dz, "v": dv, "f": df, "H0": dH0}


@pytest.mark.parametrize("K", [1, 3, 8])
def test_central_finite_differences(K):
    d = _inputs(1 + K)
    g = _grads(d, K)
    eps = 1e-6
    for name in ("q", "k", "z", "v", "f", "H0"):
        x = d[name]
        fd = np.empty_like(x)
        for idx in np.ndindex(x.shape):
            keep = x[idx]
            x[idx] = keep + eps
            lp = _loss(d, K)
            x[idx] = keep - eps
            lm = _loss(d, K)
            x[idx] = keep
            fd[idx] = (lp - lm) / (2 * eps)
        scale = max(1.0, float(np.max(np.abs(g[name]))))
        np.testing.assert_allclose(g[name], fd, rtol=0, atol=2e-7 * scale, err_msg=f"d{name}")


def _torch_loss(d, K, tf):
    """The recurrence written out with torch tensors (float64); selection from a full sort of
    the logits (piecewise constant, so it carries no gradient)."""
    B, T, Hh, M = d["q"].shape
    total = torch.zeros((), dtype=torch.float64)
    for b in range(B):
        for h in range(Hh):
            H = tf["H0"][b, h]
            for t in range(T):
                sel = torch.tensor(_topk_by_sort(list(d["z"][b, t, h]), K))
                s = torch.sigmoid(tf["z"][b, t, h, sel])
                ft = tf["f"][b, t, h]
                inf = bool(torch.isinf(ft))
                a_sel = torch.zeros_like(s) if inf else torch.exp(s * ft)
                a = torch.index_put(torch.ones(M, dtype=torch.float64), (sel,), a_sel)
                H = a[:, None] * H + ((1.0 - a) * tf["k"][b, t, h])[:, None] * tf["v"][b, t, h][None, :]
                o = tf["q"][b, t, h] @ H
                total = total + torch.sum(tf["dO"][b, t, h] * o)
            total = total + torch.sum(tf["dHT"][b, h] * H)
    return total


@pytest.mark.parametrize("K,neginf", [(2, False), (8, False), (3, True)])
def test_autograd_of_independent_recurrence(K, neginf):
    d = _inputs(20 + K, B=2, T=24, Hh=2, M=8, Dv=5, spaced_z=False)
    if neginf:  # full overwrites: no decay-rate or logit gradient on these tokens
        d["f"][0, 3, 1] = -np.inf
        d["f"][1, 10, 0] = -np.inf
    tf = {n: torch.tensor(d[n], dtype=torch.float64, requires_grad=n in ("q", "k", "z", "v", "f", "H0"))
          for n in d}
    _torch_loss(d, K, tf).backward()
    g = _grads(d, K)
    for name in ("q", "k", "z", "v", "f", "H0"):
        ref = tf[name].grad.numpy()
        assert np.all(np.isfinite(g[name])), name
        np.testing.assert_allclose(g[name], ref, rtol=1e-10, atol=1e-12, err_msg=f"d{name}")
    if neginf:
        assert g["f"][0, 3, 1] == 0.0 and g["f"][1, 10, 0] == 0.0
        assert not g["z"][0, 3, 1].any() and not g["z"][1, 10, 0].any()


def test_never_selected_slot_closed_form():
    """A slot no token selects keeps H0 all along: dH0[i,:] = sum_t q_t[i] dO_t + dH_T[i,:],
    its dk and dz are zero, and dq_t[i] = dO_t . H0[i,:]."""
    d = _inputs(40, T=30, M=8, Dv=3, spaced_z=False)
    d["z"][..., 5] = -50.0  # slot 5 never in the top 3
    g = _grads(d, 3)
    want = np.einsum("bth,bthc->bhc", d["q"][..., 5], d["dO"]) + d["dHT"][:, :, 5, :]
    np.testing.assert_allclose(g["H0"][:, :, 5, :], want, rtol=1e-13, atol=1e-13)
    assert not g["k"][..., 5].any() and not g["z"][..., 5].any()
    np.testing.assert_allclose(g["q"][..., 5], np.einsum("bthc,bhc->bth", d["dO"], d["H0"][:, :, 5, :]),
                               rtol=1e-13, atol=1e-13)


def test_zero_upstream_gives_zero_gradients():
    d = _inputs(41)
    d["dO"][:] = 0.0
    d["dHT"][:] = 0.0
    for name, x in _grads(d, 3).items():
        assert not x.any(), name
