"""bf16 / f32 bit helpers for the tests (no seam arithmetic)."""
import numpy as np


def bf16_to_f32(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def f32_bits(a):
    return np.asarray(a, np.float32).view(np.uint32)


def bf16_ordered(bits):
    """Map bf16 bit patterns to integers ordered like the values (so the
    difference of two mapped patterns counts ulps); -0 and +0 coincide."""
    b = np.asarray(bits, np.uint16).astype(np.int32)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def ulp_diff(a_bits, b_bits):
    return np.abs(bf16_ordered(a_bits) - bf16_ordered(b_bits))


def exact_bf16(values):
    """bf16 bits of values that are exactly representable (asserted)."""
    f = np.asarray(values, np.float32)
    bits = (f.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(bf16_to_f32(bits), f), "value not exact in bf16"
    return bits
