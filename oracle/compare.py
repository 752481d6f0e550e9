"""Parity gate between a computed output and the oracle's fp64 reference.

TEST INFRASTRUCTURE ONLY (used by tests/, smoke() and nothing in the library).

Tolerances (the bar the fast path is held to):

* bf16 outputs: relative L2 error over the compared elements <= 2e-3, AND the
  largest per-element error is at most 4 bf16 ulps, where the ulp of element e
  is taken at max(|yref_e|, m) with the floor m = 2**-8 * max|yref| over the
  tensor.  The floor keeps near-zero elements (whose own ulp is tiny and which
  a correctly rounded fp32-accumulated result still misses by many of their own
  ulps) from deciding the gate; the looser whole-tensor figure
  (error / ulp(max|yref|)) is reported alongside.
* fp32 outputs: relative L2 error <= 1e-5 (max ulp reported, not gated).
"""
from __future__ import annotations

import numpy as np

BF16_REL_L2 = 2e-3
BF16_MAX_ULP = 4.0
F32_REL_L2 = 1e-5
ULP_FLOOR_FRACTION = 2.0 ** -8


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def to_f64(values, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_bits_to_f64(values)
    return np.asarray(values, dtype=np.float32).astype(np.float64)


def ulp_of(mag: np.ndarray, dtype: str) -> np.ndarray:
    """Spacing of the dtype's numbers at magnitude ``mag`` (mag > 0).

    For |a| in [2**e, 2**(e+1)) the spacing is 2**(e - p + 1) with p the
    significand precision: p = 8 for bf16, p = 24 for fp32.
    """
    p = 8 if dtype == "bf16" else 24
    mag = np.maximum(np.asarray(mag, dtype=np.float64), np.finfo(np.float32).tiny)
    _, e = np.frexp(mag)  # mag = m * 2**e with m in [0.5, 1)
    return np.ldexp(1.0, e - p)


def metrics(y, yref, dtype: str) -> dict:
    """Error figures of ``y`` (raw dtype values) against ``yref`` (float64)."""
    y64 = to_f64(y, dtype).reshape(-1)
    r64 = np.asarray(yref, dtype=np.float64).reshape(-1)
    if r64.size == 0:
        return dict(n=0, rel_l2=0.0, max_ulp=0.0, max_ulp_tensor=0.0, max_abs=0.0,
                    finite=True)
    err = np.abs(y64 - r64)
    denom = np.linalg.norm(r64)
    rel_l2 = float(np.linalg.norm(y64 - r64) / denom) if denom > 0 else float(np.linalg.norm(y64 - r64))
    amax = float(np.max(np.abs(r64)))
    floor = ULP_FLOOR_FRACTION * amax
    ulps = err / ulp_of(np.maximum(np.abs(r64), floor), dtype)
    return dict(n=int(r64.size), rel_l2=rel_l2, max_ulp=float(np.max(ulps)),
                max_ulp_tensor=float(np.max(err) / ulp_of(np.array([amax]), dtype)[0]) if amax > 0 else 0.0,
                max_abs=float(np.max(err)), finite=bool(np.all(np.isfinite(y64))))


def passes(m: dict, dtype: str) -> bool:
    if not m["finite"]:
        return False
    if dtype == "bf16":
        return m["rel_l2"] <= BF16_REL_L2 and m["max_ulp"] <= BF16_MAX_ULP
    return m["rel_l2"] <= F32_REL_L2


def check(y, yref, dtype: str, what: str = "") -> dict:
    """Raise AssertionError with the figures when the gate fails."""
    m = metrics(y, yref, dtype)
    if not passes(m, dtype):
        raise AssertionError(f"parity gate failed {what}: {m}")
    return m
