"""Exact conversions from stored scalar bits to binary64.

Test infrastructure only (see ``oracle/__init__.py``).

The pool stores K/V scalars as raw bits: ``uint16`` for bfloat16 and ``uint32``
for IEEE binary32.  Both widen to binary64 without rounding, so the oracle reads
exactly the values the cache holds (not the fp32 draws they were rounded from).
"""
from __future__ import annotations

import numpy as np

BITS_DTYPE = {"bf16": np.uint16, "f32": np.uint32}
SCALAR_BYTES = {"bf16": 2, "f32": 4}


def bf16_bits_to_f64(bits) -> np.ndarray:
    """bfloat16 is the upper half of a binary32: shift into place, widen.
    Signalling-NaN payloads (poisoned pool rows) widen to NaN; numpy's
    warning about them is silenced."""
    wide = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return wide.view(np.float32).astype(np.float64)


def f32_bits_to_f64(bits) -> np.ndarray:
    with np.errstate(invalid="ignore"):
        return np.asarray(bits, dtype=np.uint32).view(np.float32).astype(np.float64)


def bits_to_f64(bits, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_bits_to_f64(bits)
    if dtype == "f32":
        return f32_bits_to_f64(bits)
    raise ValueError(f"unknown dtype {dtype!r}")
