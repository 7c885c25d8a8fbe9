"""Export side of the int6 / int5 formats: bit packing, code statistics,
artifact size, dequantisation.  Test infrastructure: only tests/,
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

Readings of the pages: an int6 code c (a multiple of 4 in
[-128, 124]) packs as the 6-bit value u = c/4 + 32; four values u0..u3 form
the 24-bit word u0 | u1 << 6 | u2 << 12 | u3 << 18 stored as 3 bytes, least
significant first; a tail of fewer than four codes is padded with code 0;
entropy is the Shannon entropy of the code histogram in bits per value;
the artifact's byte count is the packed codes (int8 matrices at one byte
per code) plus 2 bytes per row scale plus every passthrough tensor at 2
bytes per element (no general-purpose compressor).
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


def is_int5_code(c: np.ndarray) -> np.ndarray:
    """True where c is in [-16, 15]."""
    c = np.asarray(c, dtype=np.int64)
    return (c >= -16) & (c <= 15)


def pack_int5(codes: np.ndarray) -> np.ndarray:
    """int5 codes (int8, flattened) -> uint8 bytes, 5 per 8 codes."""
    c = np.asarray(codes, dtype=np.int64).ravel()
    if not np.all(is_int5_code(c)):
        raise ValueError("not an int5 code")
    pad = (-len(c)) % 8
    u = np.concatenate([c + 16, np.full(pad, 16, dtype=np.int64)]).reshape(-1, 8)
    word = np.zeros(len(u), dtype=np.int64)
    for i in range(8):
        word |= u[:, i] << (5 * i)
    out = np.stack([(word >> (8 * k)) & 0xFF for k in range(5)], axis=1).astype(np.uint8)
    return out.ravel()


def unpack_int5(packed: np.ndarray, n: int) -> np.ndarray:
    """The first n int5 codes (int8) held in packed bytes."""
    b = np.asarray(packed, dtype=np.int64).reshape(-1, 5)
    word = np.zeros(len(b), dtype=np.int64)
    for k in range(5):
        word |= b[:, k] << (8 * k)
    u = np.stack([(word >> (5 * i)) & 31 for i in range(8)], axis=1).ravel()
    return (u[:n] - 16).astype(np.int8)


def packed_bytes(n: int, bits: int) -> int:
    """Bytes of n packed codes: 3 per 4 int6 codes, 5 per 8 int5 codes, 1 per
    int8 code (unpacked), each rounded up to whole words."""
    if bits == 6:
        return 3 * ((n + 3) // 4)
    if bits == 5:
        return 5 * ((n + 7) // 8)
    if bits == 8:
        return n
    raise ValueError("bits must be 5, 6 or 8")


def pack_codes(codes: np.ndarray, bits: int) -> np.ndarray:
    return {6: pack_int6, 5: pack_int5}[bits](codes)


def unpack_codes(packed: np.ndarray, n: int, bits: int) -> np.ndarray:
    return {6: unpack_int6, 5: unpack_int5}[bits](packed, n)


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


def artifact_bytes(matrices, passthrough_elements: int, bits=None) -> int:
    """Bytes of the packed artifact: for each (rows, cols) matrix its packed
    codes (bits[i], default 6; rounded up per matrix) + 2 bytes per row
    scale; plus 2 bytes per passthrough (fp16) element."""
    total = 0
    for i, (rows, cols) in enumerate(matrices):
        b = 6 if bits is None else bits[i]
        total += packed_bytes(rows * cols, b) + 2 * rows
    return total + 2 * passthrough_elements


def dequantize_f32(codes: np.ndarray, scale16: np.ndarray) -> np.ndarray:
    """code * scale per row (fp32).  The product of an int8 code and a
    binary16 scale has at most 19 significant bits, so the fp32 result is
    the exact product (computed in fp64, then converted).  A zero code times
    an infinite scale is NaN, as IEEE multiplication defines it."""
    c = np.asarray(codes, dtype=np.float64)
    s = np.asarray(scale16, dtype=np.float16).astype(np.float64)
    with np.errstate(invalid="ignore"):
        return (c * s[:, None]).astype(np.float32)


def dequantize_bf16(codes: np.ndarray, scale16: np.ndarray) -> np.ndarray:
    """code * scale rounded to bfloat16 (round to nearest, ties to even);
    returns the bfloat16 bit patterns as uint16.  torch's CPU float32 to
    bfloat16 conversion is the rounding step."""
    import torch
    exact = torch.from_numpy(dequantize_f32(codes, scale16))
    return exact.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
