"""Shared helpers of the GPU parity tests: tensor transfer and error metrics."""
from __future__ import annotations

import numpy as np

TOL = {"f32": 1e-5, "bf16": 1e-2}  # rel-L2 bars: float32 inputs, bf16 inputs with float32 accumulation


def rel_l2(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), "non-finite values in the GPU result"
    den = np.linalg.norm(ref.ravel())
    num = np.linalg.norm((got - ref).ravel())
    return float(num / den) if den > 0 else float(num)


def dev(x, dtype: str, device="cuda:0"):
    """float32 numpy array (values exact in `dtype`) -> contiguous torch tensor on the GPU."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    t = t.to(torch.bfloat16) if dtype == "bf16" else t
    return t.to(device).contiguous()


def host(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)
