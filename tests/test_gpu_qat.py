"""Parity of the forward-only QAT weights (STE fake quantisation, Noisy-QAT
noise) between the HIP kernels and the oracle: fp32 outputs bit-exact,
bfloat16 outputs bit-exact up to NaN payloads."""
import numpy as np
import pytest

from oracle import qat as oqat
from gpu_common import need_gpu, print_case

pytestmark = pytest.mark.gpu

SHAPES = [(1, 1), (3, 5), (7, 64), (16, 300), (33, 512), (1536, 512), (512, 1536), (9, 2044), (5, 4099)]


def _dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _w(shape, seed):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal(shape) * 0.02).astype(np.float32)
    if shape[1] > 4:
        w[0, 1] = 0.5                      # an outlier row maximum
    if shape[0] > 2:
        w[2] = 0.0                         # a zero row: the 1e-12 floor
    return w


def _to_bf16_bits(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy()


def _bf16_equal(got, ref):
    got, ref = np.asarray(got).view(np.uint16), np.asarray(ref).view(np.uint16)
    nan = lambda b: ((b & 0x7F80) == 0x7F80) & ((b & 0x7F) != 0)
    assert np.array_equal(nan(got), nan(ref))
    assert np.array_equal(got[~nan(ref)], ref[~nan(ref)])


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("bits,q", [(8, 1.0), (6, 1.0), (5, 1.0), (6, 0.9999984), (5, 0.999)])
def test_fake_quantize_bit_exact(shape, bits, q):
    g = need_gpu()
    import torch
    if q < 1.0 and shape[1] - int(np.floor(q * (shape[1] - 1))) > 8:
        pytest.skip("quantile needs more than the 8 largest values")
    print_case("fake_quantize", shape, bits, q)
    w = _w(shape, shape[0] * 31 + shape[1])
    ref = oqat.fake_quantize_rows(w, bits, q)
    wd = _dev(w)
    got = g.fake_quantize_rows(wd, bits, q, torch.float32).cpu().numpy()
    assert np.array_equal(got.view(np.int32), ref.view(np.int32))
    got16 = g.fake_quantize_rows(wd, bits, q, torch.bfloat16).view(torch.int16).cpu().numpy()
    _bf16_equal(got16, _to_bf16_bits(ref))


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("levels,seed", [(127, 0), (15, 12345), (127, 0xFEDCBA9876543210)])
def test_noisy_weights_bit_exact(shape, levels, seed):
    g = need_gpu()
    import torch
    print_case("noisy_weights", shape, levels, seed)
    w = _w(shape, shape[0] * 7 + shape[1])
    ref = oqat.noisy_weights(w, levels, seed)
    wd = _dev(w)
    got = g.noisy_weights(wd, levels, seed, torch.float32).cpu().numpy()
    assert np.array_equal(got.view(np.int32), ref.view(np.int32))
    got16 = g.noisy_weights(wd, levels, seed, torch.bfloat16).view(torch.int16).cpu().numpy()
    _bf16_equal(got16, _to_bf16_bits(ref))


def test_nonfinite_rows_give_nan_and_flag():
    g = need_gpu()
    import torch
    w = _w((6, 64), 3)
    w[1, 5] = np.nan
    w[4, 0] = np.inf
    for fn in (lambda wd, f: g.fake_quantize_rows(wd, 6, 1.0, torch.float32, f),
               lambda wd, f: g.noisy_weights(wd, 127, 9, torch.float32, f)):
        flags = torch.zeros(1, dtype=torch.int32, device="cuda")
        out = fn(_dev(w), flags).cpu().numpy()
        assert int(flags.item()) & 1
        assert np.all(np.isnan(out[[1, 4]]))
        assert np.all(np.isfinite(out[[0, 2, 3, 5]]))
    good = np.delete(w, [1, 4], axis=0)
    # without a flag tensor the binding reports the rows as I6G_ENONFINITE
    with pytest.raises(g.I6GError) as ei:
        g.noisy_weights(_dev(w), 127, 9)
    assert ei.value.code == -4
    flags = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = g.noisy_weights(_dev(w), 127, 9, torch.float32, flags).cpu().numpy()
    # finite rows are unaffected by the bad rows (counters are by element index)
    ref = oqat.noisy_weights(np.where(np.isfinite(w), w, 0), 127, 9)
    assert np.array_equal(out[[0, 2, 3, 5]].view(np.int32), ref[[0, 2, 3, 5]].view(np.int32))
    assert good.shape[0] == 4
