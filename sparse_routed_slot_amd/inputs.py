"""Seeded synthetic inputs for the RSM mixer (router + chunked forward + decode step).

This module holds no arithmetic of the method itself: it only draws the tensors the
mixer consumes (router logits z, keys k, queries q, values v and the scalar log-decay
f per token and head) with the shapes, distributions and structure of the five
workloads, and encodes them as bfloat16 bit patterns where the workload says bf16.
Both the HIP path (through torch tensors) and the CPU oracle (through float64 copies)
read the very same bits from here, so parity never depends on two generators agreeing.

Draw order per workload: z, q, k, v, u, each ``rng.standard_normal(dtype=float32)``;
q and k are divided by sqrt(M); f = -softplus(u) is evaluated in float64 and stored as
float32.  The decay parameterisation f = -softplus(u) is the recipe the workloads state
(Raven's Mamba-2 style scalar decay is produced upstream of the mixer, "Model Structure"
table of the Raven README page); it is input preparation, not part of the mixer.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "bf16_bits", "bf16_to_f32", "make_inputs",
    "make_workload", "decode_step_inputs", "as_f64", "variant_inputs",
]


# ----------------------------------------------------------------------------------
# bfloat16 encoding (round to nearest, ties to even), done on the raw fp32 bits.
# ----------------------------------------------------------------------------------
def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 array -> uint16 bf16 bit patterns, round-to-nearest-even (NaN kept quiet)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    r = (u >> 16) & np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u                    # no wrap-around: finite values and infinities stay below 2^32
    r >>= np.uint32(16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = (u[nan] >> 16) | np.uint32(0x40)
    return r.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """uint16 bf16 bit patterns -> exact fp32 values."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def as_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 copy of a stored input (bf16 bits or fp32 values)."""
    if dtype == "bf16":
        return bf16_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float32).astype(np.float64)


def _softplus64(u: np.ndarray) -> np.ndarray:
    u = u.astype(np.float64)
    return np.where(u > 0, u + np.log1p(np.exp(-np.abs(u))), np.log1p(np.exp(u)))


# ----------------------------------------------------------------------------------
# Workload table
# ----------------------------------------------------------------------------------
@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    T: int
    Hh: int
    M: int
    Dv: int
    K: int
    C: int
    dtype: str            # "f32" or "bf16" for q, k, z, v; f, state and outputs are fp32
    seed: int
    z_std: float = 1.0    # router logits ~ N(0, z_std^2)
    router: str = "random"  # "random" | "needle" | "cyclic"
    note: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def tokens(self) -> int:
        return self.B * self.T


WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", 1, 256, 2, 16, 16, 4, 16, "f32", 0,
                         note="tiny fp32 case, H0 = 0"),
    "fwd_b8_t2048": Workload("fwd_b8_t2048", 8, 2048, 8, 64, 128, 16, 64, "bf16", 1,
                             note="400M-scale layer, training-shape forward"),
    "long_t32768": Workload("long_t32768", 1, 32768, 8, 64, 128, 16, 64, "bf16", 2,
                            router="needle",
                            note="long context; slots 0-3 get z+3 for t<64, z-3 after"),
    "decode_b256": Workload("decode_b256", 256, 512, 16, 64, 128, 16, 64, "bf16", 3,
                            note="prefill T=512 then 1024 single-token decode steps",
                            extra={"steps": 1024}),
    "sweep_dense": Workload("sweep_dense", 4, 4096, 16, 128, 64, 128, 64, "bf16", 4,
                            note="router limit: dense k = M (SSM limit)"),
    "sweep_swa": Workload("sweep_swa", 4, 4096, 16, 128, 64, 1, 64, "bf16", 4,
                          router="cyclic",
                          note="router limit: one-hot cyclic e_(t mod M), f = -inf (SWA limit)"),
    "sweep_topk": Workload("sweep_topk", 4, 4096, 16, 128, 64, 8, 64, "bf16", 4,
                           z_std=math.sqrt(2.0),
                           note="router limit: top-8 with logits ~ N(0, 2) (variance 2)"),
}


def _draw(rng, shape, M, z_std):
    z = rng.standard_normal(shape + (M,), dtype=np.float32)
    if z_std != 1.0:
        z = (z * np.float32(z_std)).astype(np.float32)
    inv = np.float32(1.0 / math.sqrt(M))
    q = (rng.standard_normal(shape + (M,), dtype=np.float32) * inv).astype(np.float32)
    k = (rng.standard_normal(shape + (M,), dtype=np.float32) * inv).astype(np.float32)
    return z, q, k


def make_inputs(B: int, T: int, Hh: int, M: int, Dv: int, dtype: str, seed: int,
                z_std: float = 1.0, router: str = "random", h0: bool = False,
                h0_std: float = 1.0) -> dict:
    """Draw one forward call's inputs.

    Returns a dict with q, k, z, v stored as bf16 bits (uint16) or fp32, f [B,T,Hh] fp32
    and H0 [B,Hh,M,Dv] fp32 or None.  ``router`` selects the logit structure: "random",
    "needle" (slots 0..3 biased +3 for t < 64 and -3 after, in fp32 before the bf16
    cast) or "cyclic" (z = 1 at slot t mod M, 0 elsewhere, and f = -inf).
    """
    assert dtype in ("f32", "bf16")
    rng = np.random.default_rng(seed)
    shape = (B, T, Hh)
    z, q, k = _draw(rng, shape, M, z_std)
    v = rng.standard_normal(shape + (Dv,), dtype=np.float32)
    u = rng.standard_normal(shape, dtype=np.float32)
    f = (-_softplus64(u)).astype(np.float32)
    if router == "needle":
        nslot = min(4, M)
        z[:, :64, :, :nslot] += np.float32(3.0)
        z[:, 64:, :, :nslot] -= np.float32(3.0)
    elif router == "cyclic":
        z = np.zeros_like(z)
        t = np.arange(T)
        z[:, t, :, t % M] = np.float32(1.0)
        f = np.full(shape, -np.inf, dtype=np.float32)
    elif router != "random":
        raise ValueError(router)
    H0 = None
    if h0:
        H0 = (rng.standard_normal((B, Hh, M, Dv), dtype=np.float32)
              * np.float32(h0_std)).astype(np.float32)
    enc = bf16_bits if dtype == "bf16" else (lambda a: np.ascontiguousarray(a, np.float32))
    return {"q": enc(q), "k": enc(k), "z": enc(z), "v": enc(v), "f": f, "H0": H0,
            "B": B, "T": T, "Hh": Hh, "M": M, "Dv": Dv, "dtype": dtype}


def make_workload(name: str, T: Optional[int] = None, B: Optional[int] = None) -> dict:
    """Inputs of a named workload (optionally with a shorter T or smaller B)."""
    w = WORKLOADS[name]
    d = make_inputs(B or w.B, T or w.T, w.Hh, w.M, w.Dv, w.dtype, w.seed, w.z_std, w.router)
    d["K"] = w.K
    d["C"] = w.C
    d["workload"] = w
    return d


def decode_step_inputs(rng: np.random.Generator, B: int, Hh: int, M: int, Dv: int,
                       dtype: str = "bf16") -> dict:
    """One decode step's inputs: q, k, z [B,Hh,M], v [B,Hh,Dv], f [B,Hh] (same recipe)."""
    z, q, k = _draw(rng, (B, Hh), M, 1.0)
    v = rng.standard_normal((B, Hh, Dv), dtype=np.float32)
    u = rng.standard_normal((B, Hh), dtype=np.float32)
    f = (-_softplus64(u)).astype(np.float32)
    enc = bf16_bits if dtype == "bf16" else (lambda a: np.ascontiguousarray(a, np.float32))
    return {"q": enc(q), "k": enc(k), "z": enc(z), "v": enc(v), "f": f}


# ----------------------------------------------------------------------------------
# Extra inputs of the router / decay variants
# ----------------------------------------------------------------------------------
def variant_inputs(rng: np.random.Generator, zshape) -> dict:
    """Per-slot log-decay rates and router exploration noise for logits of shape zshape
    (..., M), both fp32: f_slot = -softplus(u) with u ~ N(0, 1) (the scalar recipe drawn
    per slot), noise = standard Gumbel draws -log(-log(U)), U ~ Uniform(0, 1) (the
    exploration noise the caller adds during training).  Draw order: u, then U."""
    u = rng.standard_normal(zshape, dtype=np.float32)
    f_slot = (-_softplus64(u)).astype(np.float32)
    U = rng.random(zshape, dtype=np.float64)
    U = np.clip(U, 1e-12, 1.0 - 1e-12)
    noise = (-np.log(-np.log(U))).astype(np.float32)
    return {"f_slot": f_slot, "noise": noise}
