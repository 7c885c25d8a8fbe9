"""Forward-only quantisation-aware weights: STE fake quantisation and
Noisy-QAT noise injection.  Test infrastructure: only tests/,
__graft_entry__.smoke() and bench.py's CPU baseline use this package.

Sources (page, section):
  * pwwt.cn "parameter-golf 16MB 极限压缩实战 …", 训练时的模拟量化: in the
    training forward each row's scale is its absolute maximum / 127, codes
    are round(w / scale) (int6: round(code / 4) * 4 clamped to [-128, 124]),
    and the straight-through estimator makes the forward use the quantised
    weight: w + (w_q - w) with the difference detached.
  * kwkr.cn PR #363 write-up, Noisy QAT: instead of fake quantisation the
    forward adds uniform noise of one quantisation step: step = amax / 127
    per row (amax floored at 1e-12), noise = (U[0, 1) - 0.5) * step; the
    write-up's closing notes name amax / 15 as the int5-matched step.

Readings of the pages:
  * fake quantisation uses the quantiser's codes at the given clip quantile
    (1.0 = the plain absolute maximum of the training-time simulation) and
    the fp32 scale, not its binary16 rounding (the training forward never
    rounds the scale); w_q = code * scale in fp32;
  * the STE sum w + (w_q - w) equals w_q exactly (pinned by a test), so the
    forward value is w_q; a zero code gives +0 (the sum x + (-x) is +0);
  * the uniform numbers come from Philox4x32-10 (Salmon, Moraes, Dror, Shaw,
    "Parallel random numbers: as easy as 1, 2, 3", SC 2011), key = the 64-bit
    seed, counter = (i // 4 as 64 bits, 0, 0) for element i of the row-major
    matrix, output word i % 4; U = (word >> 8) * 2^-24;
  * noise and sum in fp32, each operation rounded once:
    w_noisy = w + (U - 0.5) * step, step = max(amax, 1e-12) / levels.
"""
from __future__ import annotations

import numpy as np

from oracle import quant as oq

F32 = np.float32
M0, M1 = 0xD2511F53, 0xCD9E8D57          # Philox4x32 multipliers
W0, W1 = 0x9E3779B9, 0xBB67AE85          # Weyl key increments
MASK = 0xFFFFFFFF


def philox4x32_10(counter, key):
    """One Philox4x32-10 block: counter (4 uint32), key (2 uint32) -> 4 uint32.
    Works elementwise on numpy uint64 arrays holding 32-bit values."""
    c0, c1, c2, c3 = (np.asarray(c, dtype=np.uint64) for c in counter)
    k0, k1 = (np.asarray(k, dtype=np.uint64) for k in key)
    for r in range(10):
        if r:
            k0 = (k0 + W0) & MASK
            k1 = (k1 + W1) & MASK
        p0 = c0 * M0                      # < 2^64: exact in uint64
        p1 = c2 * M1
        hi0, lo0 = p0 >> 32, p0 & MASK
        hi1, lo1 = p1 >> 32, p1 & MASK
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return c0, c1, c2, c3


def uniforms(n: int, seed: int) -> np.ndarray:
    """U[0, 1) fp32 for elements 0 .. n-1 (counter i // 4, word i % 4)."""
    q = np.arange((n + 3) // 4, dtype=np.uint64)
    words = philox4x32_10((q & MASK, q >> 32, np.zeros_like(q), np.zeros_like(q)),
                          (np.uint64(seed & MASK), np.uint64((seed >> 32) & MASK)))
    w = np.stack(words, axis=1).ravel()[:n]
    return ((w >> 8).astype(np.float64) * 2.0 ** -24).astype(F32)


def fake_quantize_rows(w: np.ndarray, bits: int, q: float = 1.0) -> np.ndarray:
    """The straight-through forward value of each row: code * scale (fp32)."""
    w = np.ascontiguousarray(w, dtype=F32)
    codes, _ = oq.quantize_rows(w, bits, q)
    c = oq.clip_values(w, q)
    scale32 = (c / F32(oq.LEVELS[bits])).astype(F32)
    return (codes.astype(F32) * scale32[:, None]).astype(F32)


def noisy_weights(w: np.ndarray, levels: float, seed: int) -> np.ndarray:
    """w + (U - 0.5) * step per row, step = max(amax, 1e-12) / levels (fp32)."""
    w = np.ascontiguousarray(w, dtype=F32)
    amax = np.maximum(np.abs(w).max(axis=1), oq.CLIP_FLOOR).astype(F32)
    step = (amax / F32(levels)).astype(F32)
    u = uniforms(w.size, seed).reshape(w.shape)
    noise = ((u - F32(0.5)).astype(F32) * step[:, None]).astype(F32)
    return (w + noise).astype(F32)
