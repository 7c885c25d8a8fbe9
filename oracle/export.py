"""Export side of the int6 format: bit packing, code statistics, artifact
size, dequantisation.  Test infrastructure: only tests/,
__graft_entry__.smoke() and bench.py's CPU baseline use this package.

Sources (page, section):
  * kwkr.cn PR #363 write-up, timeline (Day 0): an entropy analysis puts
    int6 codes at about 2.94 bits per value; bit packing was tried as a
    compressor.
  * the same write-up, run notes: the artifact must fit 16,000,000 bytes
    (decimal), the script prints the headroom, then dequantises the codes
    and evaluates again (roundtrip).
  * pwwt.cn "parameter-golf 16MB 极限压缩实战 …", 后训练量化导出: one fp16
    scale per row; tensors below the passthrough size stay fp16.

Readings (listed in the design doc): an int6 code c (a multiple of 4 in
[-128, 124]) packs as the 6-bit value u = c/4 + 32; four values u0..u3 form
the 24-bit word u0 | u1 << 6 | u2 << 12 | u3 << 18 stored as 3 bytes, least
significant first; a tail of fewer than four codes is padded with code 0;
entropy is the Shannon entropy of the code histogram in bits per value;
the artifact's byte count is the packed codes plus 2 bytes per row scale
plus every passthrough tensor at 2 bytes per element (no general-purpose
compressor).
"""
from __future__ import annotations

import numpy as np

ARTIFACT_LIMIT = 16_000_000


def is_int6_code(c: np.ndarray) -> np.ndarray:
    """True where c is a multiple of 4 in [-128, 124]."""
    c = np.asarray(c, dtype=np.int64)
    return (c % 4 == 0) & (c >= -128) & (c <= 124)


def pack_int6(codes: np.ndarray) -> np.ndarray:
    """int6 codes (int8, any shape, flattened) -> uint8 bytes, 3 per 4 codes."""
    c = np.asarray(codes, dtype=np.int64).ravel()
    if not np.all(is_int6_code(c)):
        raise ValueError("not an int6 code")
    n = len(c)
    pad = (-n) % 4
    u = np.concatenate([c // 4 + 32, np.full(pad, 32, dtype=np.int64)]).reshape(-1, 4)
    word = u[:, 0] | (u[:, 1] << 6) | (u[:, 2] << 12) | (u[:, 3] << 18)
    out = np.empty((len(word), 3), dtype=np.uint8)
    out[:, 0] = word & 0xFF
    out[:, 1] = (word >> 8) & 0xFF
    out[:, 2] = (word >> 16) & 0xFF
    return out.ravel()


def unpack_int6(packed: np.ndarray, n: int) -> np.ndarray:
    """The first n int6 codes (int8) held in packed bytes."""
    b = np.asarray(packed, dtype=np.int64).reshape(-1, 3)
    word = b[:, 0] | (b[:, 1] << 8) | (b[:, 2] << 16)
    u = np.stack([(word >> s) & 63 for s in (0, 6, 12, 18)], axis=1).ravel()
    return ((u[:n] - 32) * 4).astype(np.int8)


def code_histogram(codes: np.ndarray) -> np.ndarray:
    """Counts of every int8 value, index v + 128 (int64 [256])."""
    c = np.asarray(codes, dtype=np.int64).ravel()
    return np.bincount(c + 128, minlength=256).astype(np.int64)


def entropy_bits(hist: np.ndarray) -> float:
    """Shannon entropy in bits per value of a histogram."""
    h = np.asarray(hist, dtype=np.float64)
    n = h.sum()
    p = h[h > 0] / n
    return float(-(p * np.log2(p)).sum())


def artifact_bytes(matrices, passthrough_elements: int) -> int:
    """Bytes of the packed artifact: for each (rows, cols) int6 matrix,
    3 bytes per 4 codes (rounded up per matrix) + 2 bytes per row scale;
    plus 2 bytes per passthrough (fp16) element."""
    total = 0
    for rows, cols in matrices:
        total += 3 * ((rows * cols + 3) // 4) + 2 * rows
    return total + 2 * passthrough_elements


def dequantize_f32(codes: np.ndarray, scale16: np.ndarray) -> np.ndarray:
    """code * scale per row (fp32).  The product of an int8 code and a
    binary16 scale has at most 19 significant bits, so the fp32 result is
    the exact product (computed in fp64, then converted)."""
    c = np.asarray(codes, dtype=np.float64)
    s = np.asarray(scale16, dtype=np.float16).astype(np.float64)
    return (c * s[:, None]).astype(np.float32)


def dequantize_bf16(codes: np.ndarray, scale16: np.ndarray) -> np.ndarray:
    """code * scale rounded to bfloat16 (round to nearest, ties to even);
    returns the bfloat16 bit patterns as uint16.  torch's CPU float32 to
    bfloat16 conversion is the rounding step."""
    import torch
    exact = torch.from_numpy(dequantize_f32(codes, scale16))
    return exact.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
