"""Pins for the oracle's row quantiser (CPU only).

Each test fixes the quantiser to something other than itself:
  * a replay of every step in exact rational arithmetic with explicit IEEE
    binary32 / binary16 round-to-nearest-even after each operation;
  * the code set printed on the pages (multiples of 4 in [-128, 124]: 64
    levels) and hand-worked double-rounding vectors;
  * closed forms: quantile position, amax when q = 1, idempotence of int8,
    and the RMS error ratio int6/int8 = 4 (the PR #363 write-up reports int6
    per-row error about 4x int8).
"""
import math
from fractions import Fraction as Fr

import numpy as np
import pytest

import synth
from oracle import quant

GOLDEN = __import__("os").path.join(__import__("os").path.dirname(__file__), "golden")


# ---------------------------------------------------------------- exact replay
def _round_binary(x: Fr, mant: int, emin: int) -> Fr:
    """IEEE round-to-nearest-even of a rational to a binary format with
    ``mant`` fraction bits and minimum normal exponent ``emin``."""
    if x == 0:
        return Fr(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fr(2) ** e > a:
        e -= 1
    if Fr(2) ** (e + 1) <= a:
        e += 1
    e = max(e, emin)
    ulp = Fr(2) ** (e - mant)
    qq = a / ulp
    n = qq.numerator // qq.denominator
    rem = qq - n
    if rem > Fr(1, 2) or (rem == Fr(1, 2) and n % 2 == 1):
        n += 1
    return sign * n * ulp


def r32(x):
    return _round_binary(Fr(x), 23, -126)


def r16(x):
    return _round_binary(Fr(x), 10, -14)


def _rne_int(x: Fr) -> int:
    n = x.numerator // x.denominator
    rem = x - n
    if rem > Fr(1, 2) or (rem == Fr(1, 2) and n % 2 == 1):
        n += 1
    return n


def replay_row(w, bits, q):
    ws = [Fr(float(v)) for v in np.asarray(w, np.float32)]
    n = len(ws)
    srt = sorted(abs(v) for v in ws)
    pos = float(q) * float(n - 1)            # binary64 product, as specified
    lo = math.floor(pos)
    hi = min(lo + 1, n - 1)
    f = r32(Fr(pos) - lo)
    c = r32(srt[lo] + r32(f * r32(srt[hi] - srt[lo])))
    c = max(c, r32(Fr(1e-12)))
    scale = r32(c / (15 if bits == 5 else 127))
    codes = []
    for v in ws:
        v = min(max(v, -c), c)
        k = _rne_int(r32(v / scale))
        if bits == 8:
            code = min(max(k, -127), 127)
        elif bits == 5:
            code = min(max(k, -16), 15)
        else:
            code = min(max(_rne_int(Fr(k, 4)) * 4, -128), 124)
        codes.append(code)
    return codes, r16(scale)


def _check_rows(w, bits, q):
    codes, s16 = quant.quantize_rows(w, bits, q)
    for i in range(w.shape[0]):
        ref_codes, ref_s = replay_row(w[i], bits, q)
        assert codes[i].tolist() == ref_codes, f"row {i}"
        assert Fr(float(s16[i])) == ref_s, f"row {i} scale"


@pytest.mark.parametrize("bits,q", [(8, 1.0), (8, 0.9999984), (6, 0.9999984), (6, 1.0), (6, 0.9),
                                    (5, 0.9999984), (5, 1.0), (5, 0.9)])
def test_exact_replay_random(bits, q):
    rng = np.random.default_rng(7)
    for cols in (1, 2, 3, 17, 64, 130):
        w = rng.normal(0, 0.02, size=(6, cols)).astype(np.float32)
        w[0, 0] *= 40.0                      # an outlier so the clip matters
        _check_rows(w, bits, q)


@pytest.mark.parametrize("bits,q", [(8, 1.0), (6, 0.9999984), (6, 0.5), (5, 0.9999984), (5, 1.0)])
def test_exact_replay_adversarial(bits, q):
    rng = np.random.default_rng(11)
    w = synth.adversarial_rows(rng, 48)
    _check_rows(w, bits, q)


# ---------------------------------------------------------------- code set
def _golden_int_list(name):
    vals = []
    with open(f"{GOLDEN}/{name}") as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if line:
                vals.extend(int(t) for t in line.split())
    return vals


def test_int6_code_set_is_64_levels():
    levels = _golden_int_list("int6_levels.txt")
    assert len(levels) == 64
    rng = np.random.default_rng(3)
    w = rng.uniform(-1, 1, size=(64, 4096)).astype(np.float32)
    codes, _ = quant.quantize_rows(w, 6, 1.0)
    assert sorted(set(codes.ravel().tolist())) == levels


def test_int8_code_range():
    rng = np.random.default_rng(4)
    w = rng.normal(0, 1, size=(32, 999)).astype(np.float32)
    codes, _ = quant.quantize_rows(w, 8, 0.9999984)
    assert codes.min() >= -127 and codes.max() <= 127
    codes1, _ = quant.quantize_rows(w, 8, 1.0)
    # with q = 1 the largest |w| of each row lands exactly on +-127
    assert np.all(np.abs(codes1).max(axis=1) == 127)


def test_double_rounding_hand_vectors():
    """Hand-worked int6 cases: r = 2.4 -> 0, 5.5 -> 8, -125.9 -> -128 (a single
    rounding of r/4 would give 4, 4, -124)."""
    rows = []
    with open(f"{GOLDEN}/int6_double_rounding.txt") as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if line:
                r, want = line.split()
                rows.append((float(r), int(want)))
    # a row whose max |w| is 127 has fp32 scale exactly 1, so w/scale = w
    w = np.array([[127.0] + [r for r, _ in rows]], dtype=np.float32)
    codes, s16 = quant.quantize_rows(w, 6, 1.0)
    assert float(s16[0]) == 1.0
    assert codes[0, 1:].tolist() == [want for _, want in rows]


# ---------------------------------------------------------------- closed forms
def test_quantile_position_closed_form():
    for n in (2, 128, 512, 640, 1536, 2048, 625_000):
        lo, hi, f = quant.clip_position(n, 0.9999984)
        assert lo == n - 2 and hi == n - 1
        assert 0 < f < 1
    lo, hi, f = quant.clip_position(512, 0.9999984)
    assert abs(float(f) - (0.9999984 * 511 - 510)) < 1e-7
    for n in (1, 2, 77):
        lo, hi, f = quant.clip_position(n, 1.0)
        assert lo == hi == n - 1 and f == 0


def test_q1_clip_is_amax():
    rng = np.random.default_rng(5)
    w = rng.normal(0, 0.02, size=(20, 300)).astype(np.float32)
    c = quant.clip_values(w, 1.0)
    assert np.array_equal(c, np.abs(w).max(axis=1))


def test_zero_row_and_underflow():
    w = np.zeros((2, 16), np.float32)
    w[1, 3] = 1e-9
    codes, s16 = quant.quantize_rows(w, 6, 1.0)
    assert np.all(codes[0] == 0) and float(s16[0]) == 0.0
    # 1e-9/127 underflows binary16: scale 0, dequantised row 0
    assert float(s16[1]) == 0.0


def test_int8_idempotent():
    rng = np.random.default_rng(6)
    w = rng.normal(0, 0.02, size=(40, 257)).astype(np.float32)
    codes, s16 = quant.quantize_rows(w, 8, 1.0)
    w_hat = (codes.astype(np.float32) * s16.astype(np.float32)[:, None]).astype(np.float32)
    codes2, s16b = quant.quantize_rows(w_hat, 8, 1.0)
    assert np.array_equal(codes, codes2)
    assert np.array_equal(s16.view(np.uint16), s16b.view(np.uint16))


def test_rms_error_ratio_int6_vs_int8():
    """RMS rounding error in units of the fp32 scale, closed forms for a
    smooth input: int8 rounds once to step 1 -> 1/sqrt(12).  int6 rounds to
    an integer k and then k/4 to an integer: k = 0, 1, 3 (mod 4) leave an
    error uniform on (-1.5, 1.5), k = 2 (mod 4) a half-even tie with error
    in +-(1.5, 2.5); E[e^2] = 9/16 + 49/48 = 19/12.  The ratio
    sqrt(19) = 4.36 is the "about 4x int8" of the PR #363 write-up (a single
    rounding to step 4 would give exactly 4/sqrt(12))."""
    rng = np.random.default_rng(8)
    w = rng.normal(0, 0.02, size=(256, 1536)).astype(np.float32)
    errs = {}
    for bits in (8, 6):
        codes, s16 = quant.quantize_rows(w, bits, 0.9999984)
        s32 = quant.clip_values(w, 0.9999984) / np.float32(127.0)
        e = (w.astype(np.float64) / s32[:, None].astype(np.float64) - codes)
        errs[bits] = float(np.sqrt(np.mean(e * e)))
    assert abs(errs[8] - 1 / math.sqrt(12)) < 0.005
    assert abs(errs[6] - math.sqrt(19 / 12)) < 0.01
    assert abs(errs[6] / errs[8] - math.sqrt(19)) < 0.05


def test_nonfinite_rejected():
    w = np.zeros((1, 8), np.float32)
    w[0, 2] = np.nan
    with pytest.raises(ValueError):
        quant.quantize_rows(w, 6, 1.0)


def test_config_matrix_counts():
    """11-layer model: 66 matrices, 39,424 rows, 25,952,256 weights."""
    arch = synth.CONFIGS["11l"]["arch"]
    rows, weights = synth.gemm_rows(arch)
    assert (rows, weights) == (39_424, 25_952_256)


# ---------------------------------------------------------------- int5
def test_int5_hand_row():
    # c = 0.9375 (q = 1), scale = c / 15 = 0.0625 exactly; ratios w / scale
    # 15, -8, 0.5 (tie -> 0), 1.5 (tie -> 2), -2.5 (tie -> -2), 3.2, -15, 7.5 (tie -> 8)
    w = np.array([[0.9375, -0.5, 0.03125, 0.09375, -0.15625, 0.2, -0.9375, 0.46875]], np.float32)
    codes, s16 = quant.quantize_rows(w, 5, 1.0)
    assert codes[0].tolist() == [15, -8, 0, 2, -2, 3, -15, 8]
    assert float(s16[0]) == 0.0625


def test_int5_code_set_and_step():
    rng = np.random.default_rng(5)
    w = rng.normal(0, 0.02, size=(8, 4096)).astype(np.float32)
    codes, s16 = quant.quantize_rows(w, 5, 1.0)
    # inside the clip |w / scale| <= 15: at most 31 levels; Gaussian rows
    # of 4096 reach every level of the bulk on both signs
    assert codes.min() >= -15 and codes.max() <= 15
    for row in codes:
        assert set(range(-10, 11)) <= set(row.tolist())
    # the step is amax / 15 (the largest |w| of each row maps to +-15)
    amax = np.abs(w).max(axis=1)
    assert np.allclose(s16.astype(np.float64), amax / 15.0, rtol=2 ** -11)
    assert np.all(np.abs(codes[np.arange(8), np.abs(w).argmax(axis=1)]) == 15)


def test_rms_error_ratio_int5_vs_int8():
    # uniform rounding error: RMS = step / sqrt(12); the steps are amax/15
    # and amax/127, so the ratio is 127 / 15 for rows whose values fill the range
    rng = np.random.default_rng(9)
    w = rng.uniform(-1, 1, size=(64, 2048)).astype(np.float32)
    e5 = quant.dequantize(*quant.quantize_rows(w, 5, 1.0)) - w
    e8 = quant.dequantize(*quant.quantize_rows(w, 8, 1.0)) - w
    ratio = math.sqrt(np.mean(e5 ** 2) / np.mean(e8 ** 2))
    assert abs(ratio - 127 / 15) < 0.25


def test_mixed_bits_per_matrix():
    arch = dict(bits=6, bits_mlp=5)
    assert [quant.matrix_bits(arch, n) for n in ("q", "k", "v", "o", "fc", "proj")] == [6, 6, 6, 6, 5, 5]
    arch = dict(bits=6, bits_attn=5, bits_mlp=5)
    assert {quant.matrix_bits(arch, n) for n in ("q", "k", "v", "o", "fc", "proj")} == {5}
    assert quant.matrix_bits(dict(bits=8), "fc") == 8
    with pytest.raises(ValueError):
        quant.quantize_rows(np.ones((1, 4), np.float32), 4, 1.0)
