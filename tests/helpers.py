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


#: per-row bar, as a multiple of the rel-L2 bar: the largest error of a single row
#: (a token of Y, a latent of Z or Q), relative to that row's norm floored at the
#: root-mean-square row norm of the reference.  A row that is wholly wrong has a
#: row error of order one and fails it however many rows are right.
ROW_FACTOR = 5.0


def row_err(got, ref) -> float:
    """Largest relative error of one row (the last axis) of got against ref."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), "non-finite values in the GPU result"
    g = got.reshape(-1, got.shape[-1])
    r = ref.reshape(-1, ref.shape[-1])
    if r.size == 0:
        return 0.0
    rn = np.linalg.norm(r, axis=1)
    floor = np.sqrt(np.mean(rn ** 2))
    if floor == 0:
        return float(np.max(np.linalg.norm(g - r, axis=1)))
    return float(np.max(np.linalg.norm(g - r, axis=1) / np.maximum(rn, floor)))


def lse_err(got, ref) -> float:
    """Error of a log-normaliser L = log l, measured on the normaliser l = e^L it encodes.

    The bars of TOL are relative errors of values; for L that is the relative error of l,
    e^(L - L_ref) - 1 at each entry, aggregated as a root mean square like the rel-L2 of the
    other outputs.  A rel-L2 of L itself would not measure precision: L is near zero
    whenever l is near one, and large L hides large errors.  Entries whose reference is
    -inf (a latent that saw no token) must be -inf too.
    """
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    empty = np.isneginf(ref)
    assert np.array_equal(np.isneginf(got), empty), "empty rows must have L = -inf, and only they"
    g, r = got[~empty], ref[~empty]
    assert np.all(np.isfinite(g)), "non-finite values in the GPU result"
    return float(np.sqrt(np.mean(np.expm1(g - r) ** 2))) if g.size else 0.0


def dev(x, dtype: str, device="cuda:0"):
    """float32 numpy array (values exact in `dtype`) -> contiguous torch tensor on the GPU."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    t = t.to(torch.bfloat16) if dtype == "bf16" else t
    return t.to(device).contiguous()


def host(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)
