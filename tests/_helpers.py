"""Shared test helpers: host arrays -> device tensors, oracle references, error metrics."""
from __future__ import annotations

import numpy as np
import torch

from gated_token_recurrence_amd import workloads as W

TORCH_DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}

# Parity bar: 16-bit I/O is compared with the fp64 oracle rounded to the I/O
# type (rel-L2 and max-abs); float32 I/O with the unrounded fp64 oracle.
TOL = {"f32": (1e-5, None), "f16": (1e-3, 2e-2), "bf16": (1e-3, 2e-2)}


def to_dev(arr: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    if dtype == "bf16" and arr.dtype == np.uint16:
        return torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(arr)).to(device)


def inputs_to_dev(x: dict, dtype: str, device="cuda") -> dict:
    out = {}
    for key in ("q", "k", "v", "z"):
        out[key] = to_dev(x[key], dtype, device)
    out["log_g"] = torch.from_numpy(x["log_g"]).to(device)
    out["rms_w"] = torch.from_numpy(x["rms_w"]).to(device)
    return out


def inputs_f64(x: dict, dtype: str) -> dict:
    out = {key: W.io_to_f64(x[key], dtype) for key in ("q", "k", "v", "z")}
    out["log_g"] = x["log_g"].astype(np.float64)
    out["rms_w"] = x["rms_w"].astype(np.float64)
    return out


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to(torch.float64).cpu().numpy()


def errors(got: np.ndarray, ref: np.ndarray, dtype: str, oracle_mod):
    """(rel-L2, max-abs) of got against the reference rounded as the I/O type demands."""
    r = ref if dtype == "f32" else oracle_mod.round_io(ref, dtype)
    d = got - r
    rel = np.linalg.norm(d.ravel()) / max(np.linalg.norm(r.ravel()), 1e-300)
    return float(rel), float(np.max(np.abs(d)))


def assert_parity(got, ref, dtype, oracle_mod, what=""):
    rel, mx = errors(got, ref, dtype, oracle_mod)
    rtol, atol = TOL[dtype]
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    assert rel <= rtol, f"{what}: rel-L2 {rel:.3e} > {rtol:.0e} (max-abs {mx:.3e})"
    if atol is not None:
        assert mx <= atol, f"{what}: max-abs {mx:.3e} > {atol:.0e} (rel-L2 {rel:.3e})"
    return rel, mx
