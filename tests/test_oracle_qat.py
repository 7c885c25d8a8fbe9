"""Pins for the forward-only QAT oracle (STE fake quantisation, Noisy-QAT
noise, the Philox4x32-10 generator behind the noise)."""
import os
from fractions import Fraction as Fr

import numpy as np
import pytest

from oracle import qat
from oracle import quant as oq

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _kat():
    rows = []
    with open(os.path.join(GOLDEN, "philox4x32_10_kat.txt")) as fh:
        for line in fh:
            line = line.split("#", 1)[0].split()
            if line:
                v = [int(t, 16) for t in line]
                rows.append((v[:4], v[4:6], v[6:]))
    return rows


def test_philox_known_answers():
    rows = _kat()
    assert len(rows) == 3
    for ctr, key, out in rows:
        got = qat.philox4x32_10([np.uint64(c) for c in ctr], [np.uint64(k) for k in key])
        assert [int(x) for x in got] == out


def test_uniform_mapping_and_range():
    seed = 0x0123456789ABCDEF
    u = qat.uniforms(10, seed)
    # element i is word i % 4 of the block with counter i // 4
    for q in range(3):
        words = qat.philox4x32_10([np.uint64(q), np.uint64(0), np.uint64(0), np.uint64(0)],
                                  [np.uint64(seed & 0xFFFFFFFF), np.uint64(seed >> 32)])
        for j in range(4):
            if 4 * q + j < 10:
                assert Fr(float(u[4 * q + j])) == Fr(int(words[j]) >> 8, 1 << 24)
    big = qat.uniforms(1 << 20, 7)
    assert big.min() >= 0.0 and big.max() < 1.0
    assert np.all(big * 2.0 ** 24 == np.floor(big * 2.0 ** 24))
    assert abs(big.mean() - 0.5) < 2e-3 and abs(big.var() - 1 / 12) < 1e-3
    assert not np.array_equal(qat.uniforms(64, 7), qat.uniforms(64, 8))


def test_ste_sum_is_the_quantised_weight():
    # w + (w_q - w), each operation rounded to fp32, equals w_q: the
    # difference is exact (w_q is 0 or within a factor 2 of w, same sign)
    rng = np.random.default_rng(1)
    w = (rng.standard_normal((64, 512)) * 0.02).astype(np.float32)
    w[0, :5] = [1e-30, -3e-8, 0.0, 5.0, -5.0]
    for bits in (8, 6, 5):
        wq = qat.fake_quantize_rows(w, bits)
        ste = (w + (wq - w).astype(np.float32)).astype(np.float32)
        assert np.array_equal(ste.view(np.int32), wq.view(np.int32))   # zeros are +0 on both


def test_fake_quant_hand_row_int8():
    # amax 0.5, scale = fp32(0.5 / 127); codes 127, -64 (-63.5 ties to even), 25
    w = np.array([[0.5, -0.25, 0.1]], np.float32)
    s = np.float32(0.5) / np.float32(127.0)
    got = qat.fake_quantize_rows(w, 8)
    assert list(got[0]) == [np.float32(127) * s, np.float32(-64) * s, np.float32(25) * s]


@pytest.mark.parametrize("bits,levels,bound", [(8, 127, 0.5), (6, 127, 2.5), (5, 15, 0.5)])
def test_fake_quant_error_bounds(bits, levels, bound):
    rng = np.random.default_rng(bits)
    w = rng.uniform(-1, 1, (32, 1024)).astype(np.float32)
    wq = qat.fake_quantize_rows(w, bits)
    step = np.abs(w).max(axis=1, keepdims=True) / levels
    inside = np.abs(w) <= (levels - 3) * step          # away from the int6 top clamp
    err = np.abs(wq.astype(np.float64) - w)
    assert np.all(err[inside] <= bound * np.broadcast_to(step, w.shape)[inside] * (1 + 1e-6))
    # the forward value sits on the code grid of the fp32 scale
    assert np.allclose(wq / step, np.rint(wq / step), atol=1e-3)


def test_fake_quant_matches_export_codes_with_fp32_scale():
    rng = np.random.default_rng(4)
    w = (rng.standard_normal((16, 300)) * 0.02).astype(np.float32)
    for bits in (8, 6, 5):
        codes, s16 = oq.quantize_rows(w, bits, 1.0)
        wq = qat.fake_quantize_rows(w, bits)
        # same codes; the scale differs from the exported one only by its
        # binary16 rounding
        s = wq.astype(np.float64) / np.where(codes == 0, 1, codes)
        nz = codes != 0
        rel = np.abs(s - s16.astype(np.float64)[:, None]) / s16.astype(np.float64)[:, None]
        assert np.all(rel[nz] <= 2.0 ** -11 * 1.001)
        assert np.all(wq[~nz] == 0)


@pytest.mark.parametrize("levels", [127, 15])
def test_noise_bounded_by_half_a_step(levels):
    rng = np.random.default_rng(levels)
    w = (rng.standard_normal((64, 1536)) * 0.02).astype(np.float32)
    out = qat.noisy_weights(w, levels, seed=99)
    step = np.maximum(np.abs(w).max(axis=1), 1e-12) / levels
    d = (out.astype(np.float64) - w) / step[:, None]
    ulp = np.spacing(np.abs(w).astype(np.float32)).astype(np.float64) / step[:, None]
    assert np.all(np.abs(d) <= 0.5 + ulp)
    assert abs(d.mean()) < 0.01 and abs(d.var() - 1 / 12) < 0.005
    assert np.array_equal(out, qat.noisy_weights(w, levels, seed=99))
    assert not np.array_equal(out, qat.noisy_weights(w, levels, seed=100))


def test_noise_on_a_zero_row_uses_the_floor():
    w = np.zeros((2, 8), np.float32)
    out = qat.noisy_weights(w, 127, seed=1)
    assert np.all(np.abs(out) <= np.float32(1e-12) / 127 / 2 * (1 + 1e-6))
