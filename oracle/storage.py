"""Exact conversion of stored K/V/q values to fp64, and the FP8 KV format.

Storage representations on the host: fp32 as float32, fp16 as float16, bf16 as
the uint16 bit pattern (the upper half of an IEEE fp32), fp8 as the uint8
code.  All widen to fp64 without rounding.

FP8 KV cache (lshu.cn/news/11644, "性能关键路径与瓶颈": quantising the KV cache
to FP8/INT8 halves the bytes decode reads).  The pages give no format or
scaling; the reading here is the OCP 8-bit E4M3 format without infinities
(sign, 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 is
subnormal; S.1111.111 is NaN; largest finite 448) with one scale per tensor:
a stored code is the nearest E4M3 value to x * (1 / scale), both factors and
the product in fp32, ties to the even code, magnitudes past 448 saturating;
its value is code * scale.
"""
import numpy as np


def _e4m3_values() -> np.ndarray:
    """Value of every E4M3 code, from the bit fields."""
    vals = np.empty(256, dtype=np.float64)
    for c in range(256):
        sign = -1.0 if c & 0x80 else 1.0
        e, m = (c >> 3) & 0xF, c & 0x7
        if e == 0xF and m == 0x7:
            vals[c] = np.nan
        elif e == 0:
            vals[c] = sign * (m / 8.0) * 2.0 ** (1 - 7)
        else:
            vals[c] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


E4M3 = _e4m3_values()
E4M3_MAX = 448.0


def quantize_e4m3(y) -> np.ndarray:
    """fp32 values -> E4M3 codes: nearest value, ties to the even code (the
    one with an even mantissa), |y| > 448 saturates to the largest finite
    code, NaN -> S.1111.111; the sign of zero is kept."""
    y = np.asarray(y, dtype=np.float32)
    a = np.minimum(np.abs(y.astype(np.float64)), E4M3_MAX)
    pos = E4M3[:127]  # codes 0..126: the non-negative finite values, ascending
    hi = np.clip(np.searchsorted(pos, a), 0, 126)
    lo = np.clip(hi - 1, 0, 126)
    dlo, dhi = a - pos[lo], pos[hi] - a
    code = np.where(dhi < dlo, hi, np.where(dlo < dhi, lo, np.where(lo % 2 == 0, lo, hi)))
    code = np.where(a == pos[hi], hi, code).astype(np.uint8)
    code = np.where(np.isnan(y), np.uint8(0x7F), code)
    return (code | np.where(np.signbit(y), np.uint8(0x80), np.uint8(0))).astype(np.uint8)


def kv_encode(x: np.ndarray, act_dtype: str, scale: float) -> np.ndarray:
    """Activation values (storage representation of act_dtype) -> E4M3 codes
    of x * (1 / scale), computed in fp32."""
    inv = np.float32(1.0) / np.float32(scale)
    y = to_f64(x, act_dtype).astype(np.float32) * inv
    return quantize_e4m3(y)


def kv_values(codes: np.ndarray, scale: float) -> np.ndarray:
    """E4M3 codes -> fp64 values code * scale (exact: the product of a 4-bit
    significand and an fp32 scale fits fp64)."""
    return E4M3[np.asarray(codes, dtype=np.uint8)] * np.float64(np.float32(scale))


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype in ("f32", "f16"):
        return np.asarray(a).astype(np.float64)
    if dtype == "bf16":
        bits = np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    if dtype == "fp8":
        return E4M3[np.asarray(a, dtype=np.uint8)]
    raise ValueError(dtype)


def host_dtype(dtype: str):
    return {"f32": np.float32, "f16": np.float16, "bf16": np.uint16, "fp8": np.uint8}[dtype]
