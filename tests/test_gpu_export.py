"""Parity of the export side (int6 / int5 bit packing, dequantisation, code
histogram and entropy, artifact size) between the HIP kernels and the
oracle: packed bytes, codes, histograms and dequantised values bit-exact,
entropy to 1e-12."""
import numpy as np
import pytest

from oracle import export as ox
from gpu_common import make_case, need_gpu, oracle_quantized

pytestmark = pytest.mark.gpu

LEVELS = np.arange(-128, 125, 4, dtype=np.int8)
INT5 = np.arange(-16, 16, dtype=np.int8)
CODESET = {6: LEVELS, 5: INT5}
# binary16 scales: ordinary, smallest subnormal, largest subnormal, largest
# finite, zero, -1, +Inf, NaN
EDGE_SCALES = np.array([0x2E66, 0x0001, 0x03FF, 0x7BFF, 0x0000, 0xBC00, 0x7C00, 0x7E00], dtype=np.uint16)


def _dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _bf16_bits_equal(got, ref):
    """bfloat16 bit patterns equal, except that any NaN matches any NaN (a
    NaN's sign and payload are not fixed by the rounding rule, and torch's
    CPU conversion has its own pattern)."""
    got, ref = np.asarray(got).view(np.uint16), np.asarray(ref).view(np.uint16)
    nan = lambda b: ((b & 0x7F80) == 0x7F80) & ((b & 0x7F) != 0)
    assert np.array_equal(nan(got), nan(ref))
    assert np.array_equal(got[~nan(ref)], ref[~nan(ref)])


def _f32_bits_equal(got, ref):
    got, ref = np.asarray(got, np.float32), np.asarray(ref, np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.int32), ref[~nan].view(np.int32))


@pytest.mark.parametrize("n", [1, 3, 4, 5, 7, 8, 9, 15, 16, 17, 31, 32, 33, 1000, 16 * 1024 + 7,
                               16 * 1024 * 4 + 12, 3_000_017])
@pytest.mark.parametrize("bits", [6, 5])
def test_pack_unpack_bit_exact(n, bits):
    g = need_gpu()
    import torch
    print(f"pack/unpack int{bits} n={n}", flush=True)
    codes = np.random.default_rng(n).choice(CODESET[bits], n)
    flags = torch.zeros(1, dtype=torch.int32, device="cuda")
    packed = g.pack_codes(_dev(codes), bits, flags)
    ref = ox.pack_codes(codes, bits)
    assert np.array_equal(packed.cpu().numpy(), ref)
    assert int(flags.item()) == 0
    back = g.unpack_codes(_dev(ref), n, bits)
    assert np.array_equal(back.cpu().numpy(), codes)


@pytest.mark.parametrize("bits", [6, 5])
def test_pack_every_level_in_every_slot_and_empty(bits):
    g = need_gpu()
    import torch
    lv = CODESET[bits]
    wc = 4 if bits == 6 else 8
    codes = np.zeros((len(lv), wc), dtype=np.int8)
    for pos in range(wc):
        codes[:, pos] = np.roll(lv, 17 * pos)
    packed = g.pack_codes(_dev(codes.ravel()), bits)
    assert np.array_equal(packed.cpu().numpy(), ox.pack_codes(codes, bits))
    empty = torch.empty(0, dtype=torch.int8, device="cuda")
    assert g.pack_codes(empty, bits).numel() == 0
    assert g.unpack_codes(torch.empty(0, dtype=torch.uint8, device="cuda"), 0, bits).numel() == 0


@pytest.mark.parametrize("bad_at", [0, 5, 16 * 300 + 3, 16 * 1024 + 2])
@pytest.mark.parametrize("bits,bad,fixed", [(6, 6, 4), (5, 16, -16), (5, -17, 15), (5, 100, 4)])
def test_pack_flags_codes_outside_the_format(bad_at, bits, bad, fixed):
    g = need_gpu()
    import torch
    n = 16 * 1024 + 5
    codes = np.random.default_rng(bad_at).choice(CODESET[bits], n)
    codes[bad_at] = bad
    flags = torch.zeros(1, dtype=torch.int32, device="cuda")
    packed = g.pack_codes(_dev(codes), bits, flags)
    assert int(flags.item()) & g.FLAG_CODE
    with pytest.raises(ValueError):
        ox.pack_codes(codes, bits)
    # the other codes are packed as usual; the bad byte is packed from its
    # low bits (int6: bits 2..7; int5: bits 0..4), i.e. as the code `fixed`
    ok = codes.copy()
    ok[bad_at] = fixed
    assert np.array_equal(packed.cpu().numpy(), ox.pack_codes(ok, bits))


def _scales(rows, seed):
    rng = np.random.default_rng(seed)
    s = rng.uniform(1e-4, 0.2, rows).astype(np.float16).view(np.uint16)
    s[: min(rows, len(EDGE_SCALES))] = EDGE_SCALES[: min(rows, len(EDGE_SCALES))]
    return s


@pytest.mark.parametrize("rows,cols", [(1, 1), (3, 5), (8, 16), (4, 32), (37, 45), (64, 512), (9, 1536),
                                       (1536, 512), (5, 4099)])
@pytest.mark.parametrize("bits", [6, 5, 8])
def test_dequantize_bit_exact(rows, cols, bits):
    g = need_gpu()
    import torch
    print(f"dequantize {rows}x{cols} bits={bits}", flush=True)
    rng = np.random.default_rng(rows * 7919 + cols)
    codes = (rng.choice(CODESET[bits], (rows, cols)) if bits in CODESET
             else rng.integers(-127, 128, (rows, cols)).astype(np.int8))
    s16 = _scales(rows, cols)
    ref32 = ox.dequantize_f32(codes, s16.view(np.float16))
    ref16 = ox.dequantize_bf16(codes, s16.view(np.float16))
    c_d, s_d = _dev(codes), _dev(s16.view(np.int16))
    _f32_bits_equal(g.dequantize(c_d, s_d, torch.float32).cpu().numpy(), ref32)
    _bf16_bits_equal(g.dequantize(c_d, s_d, torch.bfloat16).view(torch.int16).cpu().numpy(), ref16)
    if bits in CODESET:
        p = _dev(ox.pack_codes(codes, bits))
        _f32_bits_equal(g.dequantize_packed(p, s_d, rows, cols, torch.float32, bits).cpu().numpy(), ref32)
        _bf16_bits_equal(g.dequantize_packed(p, s_d, rows, cols, torch.bfloat16, bits).view(torch.int16)
                         .cpu().numpy(), ref16)


@pytest.mark.parametrize("n", [1, 15, 16, 17, 4097, 1_000_003])
def test_histogram_bit_exact_and_accumulates(n):
    g = need_gpu()
    import torch
    rng = np.random.default_rng(n)
    a = rng.integers(-128, 128, n).astype(np.int8)
    b = rng.choice(LEVELS, n // 2 + 1)
    h = g.code_histogram(_dev(a))
    assert np.array_equal(h.cpu().numpy(), ox.code_histogram(a))
    h = g.code_histogram(_dev(b), h, accumulate=True)
    assert np.array_equal(h.cpu().numpy(), ox.code_histogram(a) + ox.code_histogram(b))
    # a fresh (non-accumulating) call clears what was there
    h = g.code_histogram(_dev(b), h)
    assert np.array_equal(h.cpu().numpy(), ox.code_histogram(b))
    e = g.code_entropy(h).item()
    assert abs(e - ox.entropy_bits(ox.code_histogram(b))) <= 1e-12
    zero = g.code_histogram(torch.empty(0, dtype=torch.int8, device="cuda"))
    assert int(zero.sum().item()) == 0 and g.code_entropy(zero).item() == 0.0


def test_entropy_closed_forms():
    g = need_gpu()
    uni = g.code_histogram(_dev(np.tile(LEVELS, 1000)))
    assert abs(g.code_entropy(uni).item() - 6.0) <= 1e-12
    one = g.code_histogram(_dev(np.full(4099, -8, dtype=np.int8)))
    assert g.code_entropy(one).item() == 0.0


@pytest.mark.parametrize("name", ["11l", "10l_int5mlp"])
def test_model_export_roundtrip_full_size(name):
    """A full-size model (all int6; int5 MLP with int6 attention): pack every
    block matrix at its width, check bytes, histogram, entropy and artifact
    size against the oracle, decode the packed matrices to bfloat16
    bit-exactly, and score with the unpacked codes: identical nats to the
    codes that were packed."""
    g = need_gpu()
    import torch
    import synth
    from oracle import quant as oq
    cfg, model = make_case(name)
    arch = cfg["arch"]
    ref_q = oracle_quantized(model)
    qb = g.quantize_model(model)
    pt = model["embed"].size + (model["skip_w"].size if model["skip_w"] is not None else 0)
    print(f"export {name}", flush=True)
    ex = g.export_model(qb, arch, pt)
    shapes, widths, all_codes = [], [], []
    for pb, rb in zip(ex["packed"], ref_q["qblocks"]):
        for mname, (packed, scales, shape, bits) in pb.items():
            codes, s16 = rb[mname]
            assert bits == oq.matrix_bits(arch, mname)
            assert np.array_equal(packed.cpu().numpy(), ox.pack_codes(codes, bits)), mname
            got = g.dequantize_packed(packed, scales, shape[0], shape[1], torch.bfloat16, bits)
            _bf16_bits_equal(got.view(torch.int16).cpu().numpy(), ox.dequantize_bf16(codes, s16))
            shapes.append(shape)
            widths.append(bits)
            all_codes.append(codes.ravel())
    hist = ox.code_histogram(np.concatenate(all_codes))
    assert np.array_equal(ex["hist"].cpu().numpy(), hist)
    assert abs(ex["entropy_bits"].item() - ox.entropy_bits(hist)) <= 1e-12
    assert ex["bytes"] == ox.artifact_bytes(shapes, pt, widths)

    back = g.import_model(ex["packed"])
    tokens, nbytes = synth.make_stream(cfg, seed=7, n_tokens=2 * 2048 + 1)
    t, b = torch.from_numpy(tokens).cuda(), torch.from_numpy(nbytes).cuda()
    m0 = g.load(model, qb)
    n0, tot0 = m0.score(t, b, 2048, 1024)
    del m0
    m1 = g.load(model, back)
    n1, tot1 = m1.score(t, b, 2048, 1024)
    assert torch.equal(n0, n1) and torch.equal(tot0, tot1)
