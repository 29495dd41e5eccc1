"""Storage formats of the synthetic inputs (numpy only).

Element types are named "f32", "f16" and "bf16". In numpy they are stored as float32, float16
and uint16 (the bit pattern of a bfloat16, the upper half of a binary32). Random inputs are
drawn in float32 and rounded to the storage type to nearest, ties to even. This module holds
input plumbing only, none of the attention arithmetic.
"""
from __future__ import annotations

import numpy as np

DTYPES = ("f32", "f16", "bf16")
# Codes of the C ABI's pa_dtype and of the oracle.
DTYPE_CODE = {"f32": 0, "f16": 1, "bf16": 2}
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2}
STORAGE = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}


def check_dtype(dtype: str) -> str:
    if dtype not in DTYPES:
        raise ValueError(f"unknown element type {dtype!r}; expected one of {DTYPES}")
    return dtype


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    rounded = ((u + (0x7FFF + ((u >> 16) & 1))) >> 16).astype(np.uint16)
    return np.where(nan, np.uint16(0x7FC0), rounded).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 (or float64) data to the storage representation of `dtype`."""
    check_dtype(dtype)
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f16":
        return np.ascontiguousarray(np.asarray(x, dtype=np.float32).astype(np.float16))
    return f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def to_float64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of stored values to float64 (for building expected values in tests)."""
    check_dtype(dtype)
    if dtype == "bf16":
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a).astype(np.float64)


def nan_value(dtype: str):
    """A quiet-NaN element of the storage type (used as poison in unused slots)."""
    check_dtype(dtype)
    if dtype == "f32":
        return np.float32(np.nan)
    if dtype == "f16":
        return np.float16(np.nan)
    return np.uint16(0x7FC0)


def inf_value(dtype: str):
    check_dtype(dtype)
    if dtype == "f32":
        return np.float32(np.inf)
    if dtype == "f16":
        return np.float16(np.inf)
    return np.uint16(0x7F80)


def full(shape, value, dtype: str) -> np.ndarray:
    return np.full(shape, value, dtype=STORAGE[check_dtype(dtype)])
