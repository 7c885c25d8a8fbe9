"""GPU parity of the row quantiser: codes and binary16 scales bit-exact
against the oracle on every configuration's matrices and on adversarial
rows."""
import numpy as np
import pytest

import synth
from oracle import quant as oq
from gpu_common import need_gpu, print_case

pytestmark = pytest.mark.gpu


def _gpu_quant(g, w, bits, q):
    import torch
    codes, scales = g.quantize_rows(torch.from_numpy(w).cuda(), bits, q)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scales.cpu().numpy().view(np.uint16)


def _assert_same(g, w, bits, q, label):
    print_case("quantize", label, w.shape, bits, q)
    codes, scales = _gpu_quant(g, w, bits, q)
    rc, rs = oq.quantize_rows(w, bits, q)
    bad = np.argwhere(codes != rc)
    assert bad.size == 0, f"{label}: {len(bad)} code mismatches, first {bad[:3].tolist()}"
    sb = np.argwhere(scales != rs.view(np.uint16))
    assert sb.size == 0, f"{label}: {len(sb)} scale mismatches, first {sb[:3].tolist()}"


@pytest.mark.parametrize("name", ["tiny", "baseline", "11l", "midcycle", "largevocab", "11l_int5", "10l_int5mlp"])
def test_config_matrices_bit_exact(name):
    g = need_gpu()
    cfg = synth.config(name)
    model = synth.make_model(cfg["arch"], seed=1337)
    a = cfg["arch"]
    for b, blk in enumerate(model["blocks"]):
        if b > 1 and name != "tiny" and b % 3:
            continue                     # every third block beyond the first two
        for mname, w in blk.items():
            _assert_same(g, w, oq.matrix_bits(a, mname), a["clip_q"], f"{name}/block{b}/{mname}")


@pytest.mark.parametrize("cols", [48, 512, 1536, 2048])
@pytest.mark.parametrize("bits,q", [(6, 0.9999984), (8, 0.9999984), (6, 1.0), (8, 1.0), (6, 0.999),
                                    (5, 0.9999984), (5, 1.0)])
def test_adversarial_rows_bit_exact(cols, bits, q):
    g = need_gpu()
    if cols - int(np.floor(q * (cols - 1))) > 8:
        pytest.skip("quantile outside the kernel's top-8 window")
    rng = np.random.default_rng(cols + bits)
    w = synth.adversarial_rows(rng, cols)
    _assert_same(g, w, bits, q, f"adversarial/{cols}")


def test_ragged_rows_and_many_rows():
    g = need_gpu()
    rng = np.random.default_rng(5)
    # widths around the register-resident limit (2048 columns, in chunks of
    # 512) and past it, where rows are read twice
    for rows, cols in [(1, 1), (3, 7), (5, 65), (4097, 130), (6, 4), (5, 516), (3, 1028),
                       (4, 2044), (3, 2052), (2, 4096)]:
        w = rng.normal(0, 0.02, size=(rows, cols)).astype(np.float32)
        _assert_same(g, w, 6, 0.9999984 if cols > 1 else 1.0, f"ragged/{rows}x{cols}")


def _half_integer_rows(rng, cols, bits):
    """Rows whose weights sit a few ulps around (n + 1/2) * scale for every
    half-integer n of the code range, with the row maximum fixing the clip
    value at q = 1: the quotients the kernel settles by division."""
    top = {5: 15.0, 6: 127.0, 8: 127.0}[bits]
    rows = []
    for _ in range(6):
        c = np.float32(rng.uniform(1e-4, 1.0))
        scale = np.float32(c / np.float32(top))
        h = (np.arange(-int(top) - 1, int(top) + 1) + 0.5).astype(np.float32)
        v = (h * scale).astype(np.float32)
        k = rng.integers(-4, 5, size=v.shape)
        for i in range(v.size):
            for _ in range(abs(int(k[i]))):
                v[i] = np.nextafter(v[i], np.float32(np.inf if k[i] > 0 else -np.inf))
        row = np.resize(v, cols)
        rng.shuffle(row)
        row[cols // 2] = c
        rows.append(np.clip(row, -c, c))
    return np.stack(rows).astype(np.float32)


@pytest.mark.parametrize("cols", [100, 512, 1024, 1536, 4096])
@pytest.mark.parametrize("bits", [5, 6, 8])
def test_half_integer_quotients_bit_exact(cols, bits):
    g = need_gpu()
    rng = np.random.default_rng(1000 * bits + cols)
    w = _half_integer_rows(rng, cols, bits)
    _assert_same(g, w, bits, 1.0, f"half-integers/{cols}/int{bits}")


def test_nonfinite_row_flagged():
    import torch
    g = need_gpu()
    w = np.random.default_rng(6).normal(0, 0.02, size=(4, 1540)).astype(np.float32)
    w[2, 1537] = np.inf
    flags = torch.zeros(1, dtype=torch.int32, device="cuda")
    codes, scales = g.quantize_rows(torch.from_numpy(w).cuda(), 6, 1.0, flags)
    torch.cuda.synchronize()
    assert int(flags.item()) & 1
    s = scales.cpu().numpy().view(np.uint16)
    assert s[2] == 0x7E00 and np.all(codes.cpu().numpy()[2] == 0)
    rc, rs = oq.quantize_rows(w[[0, 1, 3]], 6, 1.0)
    assert np.array_equal(codes.cpu().numpy()[[0, 1, 3]], rc)


def test_many_matrices_in_one_call_bit_exact():
    """i6g_quantize_rows_many on more than 160 matrices (three launches of at
    most 80) of ragged shapes gives the single-matrix results and the
    oracle's."""
    import torch
    g = need_gpu()
    rng = np.random.default_rng(11)
    shapes = [(int(rng.integers(1, 40)), int(c)) for c in rng.choice([7, 48, 64, 100, 512, 1536, 2048], 170)]
    ws = [torch.from_numpy((rng.standard_normal(s) * 0.02).astype(np.float32)).cuda() for s in shapes]
    ws[5][0, 3] = float("nan")          # one non-finite row
    for bits, q in [(6, 0.9999984), (8, 1.0), (5, 0.9999984)]:
        print_case("quantize_rows_many", "bits", bits, "q", q, "jobs", len(ws))
        jobs = [(w, torch.empty(w.shape, dtype=torch.int8, device="cuda"),
                 torch.empty(w.shape[0], dtype=torch.int16, device="cuda")) for w in ws]
        flags = torch.zeros(1, dtype=torch.int32, device="cuda")
        g.quantize_rows_many(jobs, bits, q, flags=flags)
        torch.cuda.synchronize()
        assert int(flags.item()) & 1
        for w, codes, scales in jobs:
            f1 = torch.zeros(1, dtype=torch.int32, device="cuda")
            c1, s1 = g.quantize_rows(w, bits, q, flags=f1)
            torch.cuda.synchronize()
            assert torch.equal(codes, c1) and torch.equal(scales, s1)
            wn = w.cpu().numpy()
            if np.all(np.isfinite(wn)):
                rc, rs = oq.quantize_rows(wn, bits, q)
                np.testing.assert_array_equal(codes.cpu().numpy(), rc)
                np.testing.assert_array_equal(scales.cpu().numpy().view(np.uint16), rs.view(np.uint16))


def test_default_binding_path_raises_on_nonfinite_weights():
    """Without a flag tensor the quantiser's NaN/Inf flag goes to the
    library's latch and the binding raises I6G_ENONFINITE; the latch is then
    clear, so the next finite model quantises without error."""
    import synth
    g = need_gpu()
    cfg = synth.config("tiny")
    model = synth.make_model(cfg["arch"], seed=5)
    model["blocks"][1]["fc"][7, 3] = np.nan
    print_case("quantize_model", "tiny with a NaN weight, default flags")
    with pytest.raises(g.I6GError) as ei:
        g.quantize_model(model)
    assert ei.value.code == -4
    model["blocks"][1]["fc"][7, 3] = 0.0
    q = g.quantize_model(model)
    g.weights_status()
    # a NaN scale on the device is refused by load_model
    bad = [dict(qb) for qb in q]
    s = bad[0]["o"][1].clone()
    s[5] = 0x7e00
    bad[0]["o"] = (bad[0]["o"][0], s)
    print_case("load", "tiny with a NaN scale on the device")
    with pytest.raises(g.I6GError) as ei:
        g.load(model, bad)
    assert ei.value.code == -4
    g.load(model, q)
