"""Shared helpers of the GPU tests: move generator outputs to torch / float64 and compare."""
from __future__ import annotations

import numpy as np

from sparse_routed_slot_amd import inputs as gen

# spec tolerances: max|delta| <= tol * max|o| (fp32 inputs / bf16 inputs, fp32 state)
TOL = {"f32": 1e-5, "bf16": 2e-3}


def to_torch(a: np.ndarray, dtype: str, device):
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def dev_inputs(d: dict, device):
    import torch
    dt = d["dtype"]
    out = {n: to_torch(d[n], dt, device) for n in ("q", "k", "z", "v")}
    out["f"] = torch.from_numpy(np.ascontiguousarray(d["f"], dtype=np.float32)).to(device)
    out["H0"] = None if d.get("H0") is None else torch.from_numpy(d["H0"]).to(device)
    return out


def f64_inputs(d: dict, sl=slice(None)):
    dt = d["dtype"]
    r = {n: gen.as_f64(d[n][sl], dt) for n in ("q", "k", "z", "v")}
    r["f"] = d["f"][sl].astype(np.float64)
    r["H0"] = None if d.get("H0") is None else d["H0"][sl].astype(np.float64)
    return r


def check_close(got: np.ndarray, ref: np.ndarray, scale: float, tol: float, what: str):
    err = float(np.max(np.abs(got.astype(np.float64) - ref))) if got.size else 0.0
    bound = tol * scale
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    assert err <= bound, f"{what}: max|delta| = {err:.3e} > {tol:g} * {scale:.3e} = {bound:.3e}"
    return err
