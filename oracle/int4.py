"""Group-128 symmetric INT4 weights of the oracle.

"Rebuilding Kshipra Around Memory", §2: weights are quantised to INT4 per
group of 128 with two nibbles per byte and one fp16 scale per group, i.e.
4 + 16/128 = 4.125 bits per weight; rounding to the nearest step bounds the
reconstruction error by half a step, and that bound only holds when the same
(fp16-rounded) scale is used to encode and to decode.

Readings fixed here: groups run along the input (K) dimension of each output
row; s = fp16(max|w| / 7) with the division in fp32; q = clamp(round-half-even
(w / s), -8, 7) with the division in fp32 by the fp16 scale widened to fp32;
s = 0 gives q = 0; even k sits in the low nibble; w_hat = q * s exactly.
"""
from __future__ import annotations

import numpy as np

GROUP = 128


def quantize_g128(w: np.ndarray):
    """w [N][K] (fp32) -> (packed uint8 [N][K/2], scales fp16 [N][K/128], w_hat fp32 [N][K])."""
    w = np.asarray(w, dtype=np.float32)
    n, k = w.shape
    if k % GROUP:
        raise ValueError("K must be a multiple of 128")
    g = w.reshape(n, k // GROUP, GROUP)
    amax = np.abs(g).max(axis=-1)
    s16 = (amax / np.float32(7.0)).astype(np.float16)
    s32 = s16.astype(np.float32)[..., None]
    safe = np.where(s32 == 0, np.float32(1.0), s32)
    # fp32 throughout (integer values: the clamp and the zero case are exact)
    q = np.clip(np.rint(g / safe), np.float32(-8.0), np.float32(7.0))
    q = np.where(s32 == 0, np.float32(0.0), q).astype(np.int8)
    w_hat = (q.astype(np.float32) * s32).reshape(n, k)
    qn = (q.reshape(n, k).astype(np.int16) & 0xF).astype(np.uint8)
    packed = (qn[:, 0::2] | (qn[:, 1::2] << 4)).astype(np.uint8)
    return packed, s16, w_hat


def dequantize_g128(packed: np.ndarray, s16: np.ndarray) -> np.ndarray:
    """Inverse of the packing: w_hat = q * s (fp32)."""
    n, kh = packed.shape
    lo = (packed & 0xF).astype(np.int16)
    hi = (packed >> 4).astype(np.int16)
    q = np.empty((n, kh * 2), dtype=np.int16)
    q[:, 0::2] = np.where(lo > 7, lo - 16, lo)
    q[:, 1::2] = np.where(hi > 7, hi - 16, hi)
    s32 = s16.astype(np.float32)
    return (q.reshape(n, -1, GROUP).astype(np.float32) * s32[..., None]).reshape(n, -1)


def bits_per_weight(k: int) -> float:
    """Storage bits per weight for one row of length k: 4-bit codes plus one fp16 per 128."""
    return (4 * k + 16 * (k // GROUP)) / k
