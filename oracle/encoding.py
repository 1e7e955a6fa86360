"""Element encodings of the pool, the queries and the outputs.

The pages never name a precision.  The pool holds fp32, bf16 or fp16 values
(the per-element size ``s`` of the KV-bytes-per-token formula in [icarus]
"KV Cache 为什么难管理").  The oracle keeps every tensor as raw bit patterns
and widens them to float64 only to compute.

bf16 is the upper half of an IEEE binary32; rounding fp32 -> bf16 is
round-to-nearest, ties-to-even on the dropped 16 bits, written out here from
that definition.  fp16 uses NumPy's IEEE binary16 conversion (also
round-to-nearest-even).
"""

import numpy as np

DTYPES = ("f32", "bf16", "f16")
ITEMSIZE = {"f32": 4, "bf16": 2, "f16": 2}
BITS_DTYPE = {"f32": np.uint32, "bf16": np.uint16, "f16": np.uint16}

BF16_QNAN = 0x7FC0


def f32_to_bf16_bits(x):
    """Round float32 values to bf16, nearest-even; returns uint16 bit patterns."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    hi = u >> 16
    lo = u & 0xFFFF
    # above the halfway point, or exactly halfway with an odd kept part: round up
    up = (lo > 0x8000) | ((lo == 0x8000) & ((hi & 1) == 1))
    r = hi + up.astype(np.uint64)  # a carry out of the mantissa bumps the exponent (to inf at the top)
    exp_all_ones = (u & 0x7F800000) == 0x7F800000
    is_nan = exp_all_ones & ((u & 0x007FFFFF) != 0)
    r = np.where(is_nan, np.uint64(BF16_QNAN), r)
    return r.astype(np.uint16)


def bf16_bits_to_f64(b):
    u = np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):  # signalling-NaN patterns widen to NaN
        return u.view(np.float32).astype(np.float64)


def encode(x, dtype):
    """float32 array -> bit patterns of ``dtype``."""
    x = np.asarray(x, dtype=np.float32)
    if dtype == "f32":
        return x.view(np.uint32).copy()
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    if dtype == "f16":
        with np.errstate(over="ignore"):  # past the largest half, round-to-nearest gives infinity
            return x.astype(np.float16).view(np.uint16)
    raise ValueError(dtype)


def decode(bits, dtype):
    """bit patterns of ``dtype`` -> float64 array."""
    bits = np.asarray(bits)
    if dtype == "f32":
        return bits.astype(np.uint32).view(np.float32).astype(np.float64)
    if dtype == "bf16":
        return bf16_bits_to_f64(bits)
    if dtype == "f16":
        return bits.astype(np.uint16).view(np.float16).astype(np.float64)
    raise ValueError(dtype)


def nan_bits(dtype):
    """A quiet NaN of ``dtype``: the poison written into unused pool slots."""
    return {"f32": 0x7FC00000, "bf16": BF16_QNAN, "f16": 0x7E00}[dtype]
