"""Q8_1 activation quantizer, emulated in IEEE float32 (oracle side).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Per block of 32 activations ([8e] §2 for the rule, §3.2 for the arithmetic
the kernel performs; [MMQ] "What they do right" for the one-byte-per-element
Q8_1 activation):

1. ``am = max |x_e|``                               (float32, exact)
2. ``d  = fl32(am / 127)``                          (IEEE division)
3. ``di = fl32(1 / d)`` if ``d >= 2^-126`` else 0   (IEEE division)
4. ``q_e = clamp(rint(fl32(x_e * di)), -128, 127)`` (round half to even)
5. store ``f16(d)`` (round to nearest even), two zero pad bytes, the 32 int8
   values and their int32 sum.

Step 3 treats a subnormal float32 ``d`` (a block maximum below 127 * 2^-126)
like ``d == 0``, as a GPU that flushes float32 subnormals would: the pages
take the reciprocal only of a nonzero scale and do not say what a subnormal
one does; its reciprocal can overflow to infinity, and its f16 rounding is 0,
so the block dequantizes to 0 whatever its values.  Such a block is stored as
all zeros.
Step 4 quantizes with the float32 ``d``, not the f16 value that is stored.
numpy float32 arithmetic performs each step with a single IEEE rounding and
``np.rint`` rounds half to even; the float32 -> float16 cast rounds to nearest
even.  The tests pin each of these facts.
"""
from __future__ import annotations

import numpy as np

from .formats import Q8_1_BYTES


def quantize_q8_1(x: np.ndarray) -> np.ndarray:
    """fp32 ``x[T, K]`` (K a multiple of 32) -> Q8_1 bytes ``uint8[T, K/32, 40]``."""
    x = np.asarray(x)
    if x.dtype != np.float32:
        raise TypeError("activations must be float32")
    T, K = x.shape
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    xb = x.reshape(T, K // 32, 32)
    am = np.abs(xb).max(axis=-1)                                   # step 1
    d = (am / np.float32(127.0)).astype(np.float32)                # step 2
    with np.errstate(divide="ignore", over="ignore"):
        recip = (np.float32(1.0) / d).astype(np.float32)
    di = np.where(d >= np.float32(2.0**-126), recip, np.float32(0.0)).astype(np.float32)  # step 3
    v = (xb * di[..., None]).astype(np.float32)                    # step 4: fl32(x * di)
    q = np.clip(np.rint(v), -128, 127).astype(np.int8)
    out = np.zeros((T, K // 32, Q8_1_BYTES), dtype=np.uint8)       # step 5
    out[..., 0:2] = d.astype(np.float16).view(np.uint8).reshape(T, K // 32, 2)
    out[..., 4:36] = q.view(np.uint8)
    qsum = q.astype(np.int32).sum(axis=-1, dtype=np.int32)
    out[..., 36:40] = qsum.astype("<i4").view(np.uint8).reshape(T, K // 32, 4)
    return out
