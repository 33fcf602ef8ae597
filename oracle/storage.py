"""Exact conversion of stored K/V/q values to fp64.

Storage representations on the host: fp32 as float32, fp16 as float16, bf16 as
the uint16 bit pattern (the upper half of an IEEE fp32).  All three widen to
fp64 without rounding.
"""
import numpy as np


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype in ("f32", "f16"):
        return np.asarray(a).astype(np.float64)
    if dtype == "bf16":
        bits = np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    raise ValueError(dtype)


def host_dtype(dtype: str):
    return {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}[dtype]
