"""Comparison helpers shared by the tests (no arithmetic of the method itself)."""
import numpy as np


def f32(bits):
    """Widen bfloat16 bit patterns to float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def bf16_ordered(bits):
    """Map bf16 bit patterns to integers that are ordered like the values (+0 == -0)."""
    v = np.asarray(bits, dtype=np.uint16).astype(np.int32)
    mag = v & 0x7FFF
    return np.where(v & 0x8000, -mag, mag)


def bf16_ulp_diff(a, b):
    """Distance in bf16 units in the last place between two arrays of bf16 bit patterns."""
    return np.abs(bf16_ordered(a) - bf16_ordered(b))


def torch_bf16_bits(x):
    """float64/float32 array -> bf16 bit patterns through torch's cast (via float32)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
