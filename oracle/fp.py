"""Number formats of the oracle: exact bf16 decoding and round-to-nearest-even encoding.

The pages fix no precision for the head.  The reading used throughout: bf16 weights and
hidden states are decoded exactly; every dot product is accumulated in float64; the
intermediate low-rank vector (SlimSpec section 三, the r-dim summary W_down h) and the
SpecVocab reduced state h' (section 2.2.1) are rounded ONCE to the configuration's storage
dtype with round-to-nearest-even, as two stacked bf16 linear layers would store them.
"""
import numpy as np

BF16 = "bf16"
F32 = "f32"


def bf16_bits_to_f64(bits):
    """Decode bf16 bit patterns (uint16) exactly to float64."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x):
    """Round float64 values to bf16 bit patterns, nearest-even, in ONE rounding step.

    Rounding goes straight from float64 (not through float32), so no double rounding.
    bf16 has an 8-bit significand (7 stored bits) and float32's exponent range.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.float64)
    ax = np.abs(x)
    # quantum (spacing) of bf16 at |x|: 2^(e-8) for x = f*2^e, f in [0.5,1); floor at subnormal 2^-133
    _, e = np.frexp(ax)
    q_exp = np.maximum(e.astype(np.int64) - 8, -133)
    q = np.ldexp(np.ones_like(ax), q_exp)
    out = np.rint(ax / q) * q          # np.rint rounds halves to even; ax/q is exact (power-of-two scaling)
    out = np.where(out >= 2.0 ** 128, np.inf, out)
    out = np.copysign(out, x)
    return (out.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def round_to_dtype(x, dtype):
    """Round float64 -> storage dtype (bf16 or f32) with RNE, return as float64 again."""
    if dtype == BF16:
        return bf16_bits_to_f64(f64_to_bf16_bits(x))
    if dtype == F32:
        return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
    raise ValueError(dtype)


def decode(arr, dtype):
    """Input array (uint16 bf16 bits, or float32) -> float64."""
    if dtype == BF16:
        return bf16_bits_to_f64(arr)
    if dtype == F32:
        return np.asarray(arr, dtype=np.float32).astype(np.float64)
    raise ValueError(dtype)
