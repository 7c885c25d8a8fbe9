"""Per-row int8 / int6 / int5 quantiser, one IEEE binary32 operation at a time.

Source: pwwt.cn "parameter-golf 16MB 极限压缩实战 …", section 训练时的模拟量化
(scale = amax/127 per row; q_raw = round(w/scale); in int6 mode additionally
q = round(q_raw/4)*4 clamped to [-128, 124], i.e. 64 levels in an int8
container) and section 后训练量化导出 (rows of 2-D matrices, one fp16 scale per
row, clipping at the 99.99984th percentile before quantising; export uses the
same rounding as the training-time simulation).  The 1e-12 floor on the clip
value follows the Noisy-QAT code block of the kwkr.cn PR #363 write-up
(``amax(...).clamp_min(1e-12)``).  int5 follows the same write-up: the flat
11-layer runs export MLP and attention matrices as int5 (MLP_INT5 /
ATTN_INT5 in its run commands), and its closing notes give the int5 step as
amax / 15 against int8's amax / 127.

Readings where the pages are silent:
  * the percentile is of |w| over the row, linear interpolation between order
    statistics (pos = q*(n-1) in binary64, lo = floor(pos), hi = min(lo+1, n-1),
    f = fp32(pos - lo));
  * codes are computed with the fp32 scale; the stored scale is its fp16 RNE
    rounding, which is what dequantisation uses;
  * ``round`` is round-half-to-even (torch ``.round()``), applied twice in
    int6 mode;
  * int8 codes are clamped to [-127, 127];
  * int5: scale = c / 15 and code = clamp(round(w / scale), -16, 15), the
    5-bit two's complement range, stored in an int8 container (inside the
    clip |w / scale| <= 15, so -16 is never produced: 31 levels are used);
  * values are clipped to [-c, c] before the division.

numpy scalar/array float32 arithmetic rounds every operation separately (no
fused multiply-add), which is exactly the binary32 sequence written below.
"""
from __future__ import annotations

import math
import numpy as np

F32 = np.float32
INT6_MIN, INT6_MAX = -128, 124
INT8_MIN, INT8_MAX = -127, 127
INT5_MIN, INT5_MAX = -16, 15
LEVELS = {8: 127.0, 6: 127.0, 5: 15.0}     # c / LEVELS[bits] is the fp32 scale
CLIP_FLOOR = F32(1e-12)


def clip_position(n: int, q: float):
    """Order-statistic indices and fp32 weight of the linear-interpolation
    quantile of n sorted values (binary64 position, then fp32 fraction)."""
    if not (0.0 < q <= 1.0):
        raise ValueError("quantile must be in (0, 1]")
    pos = float(q) * float(n - 1)
    lo = int(math.floor(pos))
    hi = min(lo + 1, n - 1)
    f = F32(pos - lo)
    return lo, hi, f


def clip_values(w: np.ndarray, q: float) -> np.ndarray:
    """Per-row clip value c (fp32) = quantile of |w| (rows along axis 1)."""
    w = np.asarray(w, dtype=F32)
    n = w.shape[1]
    s = np.sort(np.abs(w), axis=1)
    lo, hi, f = clip_position(n, q)
    s_lo = s[:, lo]
    s_hi = s[:, hi]
    diff = (s_hi - s_lo).astype(F32)          # fp32 subtract
    step = (f * diff).astype(F32)             # fp32 multiply
    c = (s_lo + step).astype(F32)             # fp32 add
    return np.maximum(c, CLIP_FLOOR).astype(F32)


def quantize_rows(w: np.ndarray, bits: int, q: float):
    """Quantise each row of fp32 ``w`` [rows, cols].

    Returns ``(codes int8 [rows, cols], scale16 float16 [rows])``.
    Raises ValueError on non-finite input.
    """
    if bits not in (5, 6, 8):
        raise ValueError("bits must be 5, 6 or 8")
    w = np.ascontiguousarray(w, dtype=F32)
    if w.ndim != 2 or w.shape[0] < 1 or w.shape[1] < 1:
        raise ValueError("w must be a non-empty 2-D array")
    if not np.all(np.isfinite(w)):
        raise ValueError("non-finite weight")
    c = clip_values(w, q)                                  # [rows]
    scale32 = (c / F32(LEVELS[bits])).astype(F32)          # correctly rounded fp32 division
    cc = c[:, None]
    v = np.minimum(np.maximum(w, -cc), cc)                 # clip to [-c, c]
    r = (v / scale32[:, None]).astype(F32)                 # fp32 division per element
    k = np.rint(r)                                         # round half to even
    if bits == 8:
        code = np.clip(k, INT8_MIN, INT8_MAX)
    elif bits == 5:
        code = np.clip(k, INT5_MIN, INT5_MAX)
    else:
        k4 = np.rint(k / F32(4.0))                          # exact /4, then round half to even
        code = np.clip(k4 * F32(4.0), INT6_MIN, INT6_MAX)
    scale16 = scale32.astype(np.float16)                   # binary16 RNE, subnormals kept
    return code.astype(np.int8), scale16


def dequantize(codes: np.ndarray, scale16: np.ndarray) -> np.ndarray:
    """W_hat[o, i] = code[o, i] * scale16[o], in float64."""
    return codes.astype(np.float64) * scale16.astype(np.float64)[:, None]


ATTN_MATRICES = ("q", "k", "v", "o")
MLP_MATRICES = ("fc", "proj")


def matrix_bits(arch: dict, name: str) -> int:
    """Bits of one block matrix: arch['bits_attn'] for q, k, v, o and
    arch['bits_mlp'] for fc, proj when given (mixed int5 / int6 export),
    else arch['bits']."""
    key = "bits_attn" if name in ATTN_MATRICES else "bits_mlp"
    return int(arch.get(key) or arch["bits"])


def quantize_model(model: dict) -> dict:
    """Quantise the six matrices of every unique block of a synthetic model
    (matrix_bits, arch['clip_q']); every other tensor passes through."""
    arch = model["arch"]
    qblocks = []
    for blk in model["blocks"]:
        qb = {}
        for name, w in blk.items():
            qb[name] = quantize_rows(w, matrix_bits(arch, name), arch["clip_q"])
        qblocks.append(qb)
    out = dict(model)
    out["qblocks"] = qblocks
    return out
