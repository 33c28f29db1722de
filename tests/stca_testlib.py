"""Shared helpers for the GPU parity tests (no STCA arithmetic: that lives in oracle/)."""
from __future__ import annotations

import numpy as np

BF16_TOL = 2e-2   # max row-relative error, bf16 storage path
F32_TOL = 1e-4    # max row-relative error, fp32 debug path


def tol_for(cfg) -> float:
    return BF16_TOL if cfg.dtype == "bf16" else F32_TOL


def row_rel(g, o) -> float:
    """max over output rows of max_k |g - o| / max_k |o| (rows = last axis)."""
    g = np.asarray(g, np.float64)
    o = np.asarray(o, np.float64)
    assert g.shape == o.shape, (g.shape, o.shape)
    if g.size == 0:
        return 0.0
    g = g.reshape(-1, g.shape[-1])
    o = o.reshape(-1, o.shape[-1])
    num = np.max(np.abs(g - o), axis=1)
    den = np.maximum(np.max(np.abs(o), axis=1), 1e-30)
    r = num / den
    if np.any(np.isnan(r)):
        return float("inf")
    return float(np.max(r))


def announce(*parts):
    print("[case]", *parts, flush=True)
