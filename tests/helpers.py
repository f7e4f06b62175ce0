"""Test-side plumbing: host<->device copies of stored-format arrays and the
error metrics.  Holds none of the block's arithmetic."""
from __future__ import annotations

import numpy as np

from transformer_ffn_block_amd import inputs as I


def dev(a: np.ndarray, dtype: str = "bf16"):
    """Copy a stored-format host array to cuda:0 (bf16 bits -> torch.bfloat16)."""
    import torch
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16))
        return t.view(torch.bfloat16).to("cuda")
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda")
    if dtype == "i8":
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int8)).to("cuda")
    if dtype == "u8":
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to("cuda")
    if dtype == "u16":
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).to("cuda")
    raise ValueError(dtype)


def host_f64(t) -> np.ndarray:
    """Device tensor (bf16 or fp32) -> float64 numpy, exact."""
    import torch
    t = t.detach().to("cpu")
    if t.dtype == torch.bfloat16:
        return I.bf16_bits_to_f32(t.view(torch.int16).numpy().view(np.uint16)).astype(np.float64)
    return t.numpy().astype(np.float64)


def host_bits(t) -> np.ndarray:
    import torch
    t = t.detach().to("cpu")
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    return t.numpy().view(np.uint32).copy()


def max_norm_err(a: np.ndarray, r: np.ndarray) -> float:
    """max_i |a_i - r_i| / max_i |r_i|: the block's error metric (a per-element
    relative error is undefined where y = x + delta cancels)."""
    den = float(np.max(np.abs(r)))
    return float(np.max(np.abs(a - r))) / (den if den > 0 else 1.0)


def elementwise_rel_err(a: np.ndarray, r: np.ndarray) -> float:
    """max over r != 0 of |a - r| / |r|; entries with r == 0 must have a == 0
    (reported as inf otherwise)."""
    nz = r != 0
    if np.any(a[~nz] != 0):
        return float("inf")
    if not np.any(nz):
        return 0.0
    return float(np.max(np.abs(a[nz] - r[nz]) / np.abs(r[nz])))


def rel_l2(a: np.ndarray, r: np.ndarray) -> float:
    return float(np.linalg.norm(a - r) / max(np.linalg.norm(r), 1e-300))


# achieved error per parity case: (case, metric, error, tolerance), written
# out at the end of the session when FFN_PARITY_LOG names a file
PARITY = []


def record(case: str, err: float, tol: float, metric: str = "max_norm") -> float:
    """Log one parity figure (printed, and kept for the session's summary)."""
    PARITY.append({"case": case, "metric": metric, "err": float(err), "tol": float(tol)})
    print(f"[parity] {case}: {metric} {err:.3e} (tol {tol:g})", flush=True)
    return err
