"""Tolerance check of a layer output against the fp64 oracle.

TEST INFRASTRUCTURE ONLY: nothing in the product path may import this module.

Rule (the workload's acceptance bar): row r passes iff all its elements are
finite and either the largest error in bfloat16 ULPs of the reference is at
most 3, or the row's relative L2 error is at most 4e-3 -- whichever is looser.
ulp_bf16(v) = 2^(max(floor(log2|v|), -126) - 7).  A reference row that is
exactly zero must be reproduced exactly.
"""
from __future__ import annotations

import numpy as np

from .formats import ulp_bf16

ULP_BOUND = 3.0
REL_L2_BOUND = 4e-3


def rel_l2(out: np.ndarray, ref: np.ndarray) -> float:
    o = np.asarray(out, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    d = np.linalg.norm(r)
    return float(np.linalg.norm(o - r) / d) if d > 0 else float(np.linalg.norm(o))


def check_rows(out: np.ndarray, ref: np.ndarray, ulps: float = ULP_BOUND,
               rel: float = REL_L2_BOUND) -> dict:
    """Apply the rule row by row."""
    o = np.asarray(out, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    if o.shape != r.shape:
        raise ValueError(f"shape mismatch: out {o.shape} vs ref {r.shape}")
    o2 = o.reshape(-1, o.shape[-1]) if o.ndim else o.reshape(1, 1)
    r2 = r.reshape(-1, r.shape[-1]) if r.ndim else r.reshape(1, 1)
    rows = o2.shape[0]
    finite = np.isfinite(o2).all(axis=1)
    with np.errstate(invalid="ignore"):
        ulp_err = (np.abs(o2 - r2) / ulp_bf16(r2)).max(axis=1) if o2.shape[1] else np.zeros(rows)
    rnorm = np.linalg.norm(r2, axis=1)
    dnorm = np.linalg.norm(o2 - r2, axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        rl2 = np.where(rnorm > 0, dnorm / np.where(rnorm > 0, rnorm, 1.0), np.where(dnorm > 0, np.inf, 0.0))
    zero_ref = rnorm == 0
    ok = finite & np.where(zero_ref, dnorm == 0, (ulp_err <= ulps) | (rl2 <= rel))
    bad = np.nonzero(~ok)[0]
    return {
        "pass": bool(ok.all()),
        "rows": rows,
        "failing_rows": [int(i) for i in bad[:16]],
        "max_ulp": float(np.nanmax(ulp_err)) if rows else 0.0,
        "max_rel_l2": float(np.nanmax(np.where(np.isfinite(rl2), rl2, np.nan))) if rows and np.isfinite(rl2).any() else 0.0,
        "all_finite": bool(finite.all()),
    }
