"""The no-allocation code histogram (i6g_code_histogram_noalloc) against
i6g_code_histogram, called through the C ABI: two calls in a row, the
second on a smaller input, so that the shared device scratch must be
cleared between calls; plain and accumulating modes."""
import ctypes

import numpy as np
import pytest

from gpu_common import need_gpu, print_case

pytestmark = pytest.mark.gpu


def _hist(L, fn, codes, n, acc, hist, stream):
    rc = getattr(L, fn)(ctypes.c_void_p(codes.data_ptr()), n, acc, ctypes.c_void_p(hist.data_ptr()), stream)
    assert rc == 0, L.i6g_last_error().decode()


def test_noalloc_histogram_matches_allocating_one():
    import torch
    g = need_gpu()
    L = g.lib()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rng = np.random.default_rng(2024)
    big = (rng.integers(-32, 31, size=3_000_017) * 4).astype(np.int8)       # int6 codes, ragged length
    small = rng.integers(-128, 128, size=70_001).astype(np.int8)            # every int8 value
    for label, arr in (("3,000,017 int6 codes", big), ("70,001 int8 codes (second, smaller call)", small)):
        print_case("code_histogram_noalloc", label)
        codes = torch.from_numpy(arr).cuda()
        want = torch.empty(256, dtype=torch.int64, device="cuda")
        got = torch.full((256,), -7, dtype=torch.int64, device="cuda")
        _hist(L, "i6g_code_histogram", codes, arr.size, 0, want, stream)
        _hist(L, "i6g_code_histogram_noalloc", codes, arr.size, 0, got, stream)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(got.cpu().numpy(), want.cpu().numpy())
        ref = np.bincount(arr.astype(np.int64) + 128, minlength=256)
        np.testing.assert_array_equal(got.cpu().numpy(), ref)
        # accumulating into an existing histogram adds the same counts again
        _hist(L, "i6g_code_histogram_noalloc", codes, arr.size, 1, got, stream)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(got.cpu().numpy(), 2 * ref)
    # an empty input clears (or, accumulating, keeps) the histogram
    empty = torch.empty(16, dtype=torch.int8, device="cuda")
    _hist(L, "i6g_code_histogram_noalloc", empty, 0, 0, got, stream)
    torch.cuda.synchronize()
    assert int(got.abs().sum().item()) == 0
