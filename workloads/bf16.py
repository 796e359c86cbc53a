"""bfloat16 storage format: float32 -> bf16 bits (round to nearest, ties to even) and back.

bf16 is the upper 16 bits of an IEEE-754 binary32.  Inputs are drawn in float32
and rounded once to bf16; every consumer then reads those exact bf16 values
(the oracle widens them to float64 exactly), so input quantisation is never
counted as an error of the path under test.
"""
import numpy as np

_CHUNK = 1 << 24


def f32_to_bf16_bits(a):
    """Round a float32 array to bf16 (RNE); returns uint16 bit patterns."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    flat = a.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint16)
    for s in range(0, flat.size, _CHUNK):
        u = flat[s:s + _CHUNK].view(np.uint32)
        lsb = (u >> np.uint32(16)) & np.uint32(1)
        r = (u + (np.uint32(0x7FFF) + lsb)) >> np.uint32(16)
        o = r.astype(np.uint16)
        nan = np.isnan(flat[s:s + _CHUNK])
        if nan.any():
            o[nan] = 0x7FC0
        out[s:s + _CHUNK] = o
    return out.reshape(a.shape)


def bf16_bits_to_f32(b):
    b = np.asarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_bits_to_f64(b):
    """Exact widening of bf16 bit patterns to float64."""
    return bf16_bits_to_f32(b).astype(np.float64)
