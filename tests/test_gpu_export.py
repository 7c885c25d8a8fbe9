"""Parity of the export side (6-bit packing, dequantisation, code histogram
and entropy, artifact size) between the HIP kernels and the oracle: packed
bytes, codes, histograms and dequantised values bit-exact, entropy to 1e-12."""
import numpy as np
import pytest

from oracle import export as ox
from gpu_common import make_case, need_gpu, oracle_quantized

pytestmark = pytest.mark.gpu

LEVELS = np.arange(-128, 125, 4, dtype=np.int8)
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


@pytest.mark.parametrize("n", [1, 3, 4, 5, 15, 16, 17, 31, 33, 1000, 16 * 1024 + 7, 16 * 1024 * 4 + 12,
                               3_000_017])
def test_pack_unpack_bit_exact(n):
    g = need_gpu()
    import torch
    print(f"pack/unpack n={n}", flush=True)
    codes = np.random.default_rng(n).choice(LEVELS, n)
    flags = torch.zeros(1, dtype=torch.int32, device="cuda")
    packed = g.pack_int6(_dev(codes), flags)
    ref = ox.pack_int6(codes)
    assert np.array_equal(packed.cpu().numpy(), ref)
    assert int(flags.item()) == 0
    back = g.unpack_int6(_dev(ref), n)
    assert np.array_equal(back.cpu().numpy(), codes)


def test_pack_every_level_in_every_slot_and_empty():
    g = need_gpu()
    import torch
    codes = np.zeros((64, 4), dtype=np.int8)
    for pos in range(4):
        codes[:, pos] = np.roll(LEVELS, 17 * pos)
    packed = g.pack_int6(_dev(codes.ravel()))
    assert np.array_equal(packed.cpu().numpy(), ox.pack_int6(codes))
    empty = torch.empty(0, dtype=torch.int8, device="cuda")
    assert g.pack_int6(empty).numel() == 0
    assert g.unpack_int6(torch.empty(0, dtype=torch.uint8, device="cuda"), 0).numel() == 0


@pytest.mark.parametrize("bad_at", [0, 5, 16 * 300 + 3, 16 * 1024 + 2])
def test_pack_flags_non_int6_codes(bad_at):
    g = need_gpu()
    import torch
    n = 16 * 1024 + 5
    codes = np.random.default_rng(bad_at).choice(LEVELS, n)
    codes[bad_at] = 6            # not a multiple of 4
    flags = torch.zeros(1, dtype=torch.int32, device="cuda")
    packed = g.pack_int6(_dev(codes), flags)
    assert int(flags.item()) & g.FLAG_CODE
    with pytest.raises(ValueError):
        ox.pack_int6(codes)
    # the other codes are packed as usual: compare with the code cleared of its low bits
    fixed = codes.copy()
    fixed[bad_at] = 4
    assert np.array_equal(packed.cpu().numpy(), ox.pack_int6(fixed))


def _scales(rows, seed):
    rng = np.random.default_rng(seed)
    s = rng.uniform(1e-4, 0.2, rows).astype(np.float16).view(np.uint16)
    s[: min(rows, len(EDGE_SCALES))] = EDGE_SCALES[: min(rows, len(EDGE_SCALES))]
    return s


@pytest.mark.parametrize("rows,cols", [(1, 1), (3, 5), (8, 16), (37, 45), (64, 512), (9, 1536), (1536, 512),
                                       (5, 4099)])
@pytest.mark.parametrize("bits", [6, 8])
def test_dequantize_bit_exact(rows, cols, bits):
    g = need_gpu()
    import torch
    print(f"dequantize {rows}x{cols} bits={bits}", flush=True)
    rng = np.random.default_rng(rows * 7919 + cols)
    codes = (rng.choice(LEVELS, (rows, cols)) if bits == 6
             else rng.integers(-127, 128, (rows, cols)).astype(np.int8))
    s16 = _scales(rows, cols)
    ref32 = ox.dequantize_f32(codes, s16.view(np.float16))
    ref16 = ox.dequantize_bf16(codes, s16.view(np.float16))
    c_d, s_d = _dev(codes), _dev(s16.view(np.int16))
    _f32_bits_equal(g.dequantize(c_d, s_d, torch.float32).cpu().numpy(), ref32)
    _bf16_bits_equal(g.dequantize(c_d, s_d, torch.bfloat16).view(torch.int16).cpu().numpy(), ref16)
    if bits == 6:
        p = _dev(ox.pack_int6(codes))
        _f32_bits_equal(g.dequantize_packed(p, s_d, rows, cols, torch.float32).cpu().numpy(), ref32)
        _bf16_bits_equal(g.dequantize_packed(p, s_d, rows, cols, torch.bfloat16).view(torch.int16).cpu().numpy(),
                         ref16)


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


def test_model_export_roundtrip_full_size():
    """The 11-layer model at its real shapes: pack every block matrix, check
    bytes, histogram, entropy and artifact size against the oracle, decode
    the packed matrices to bfloat16 bit-exactly, and score with the unpacked
    codes: identical nats to the codes that were packed."""
    g = need_gpu()
    import torch
    import synth
    cfg, model = make_case("11l")
    ref_q = oracle_quantized(model)
    qb = g.quantize_model(model)
    pt = model["embed"].size + (model["skip_w"].size if model["skip_w"] is not None else 0)
    print("export 11l", flush=True)
    ex = g.export_model(qb, pt)
    shapes, all_codes = [], []
    for pb, rb in zip(ex["packed"], ref_q["qblocks"]):
        for name, (packed, scales, shape) in pb.items():
            codes, s16 = rb[name]
            assert np.array_equal(packed.cpu().numpy(), ox.pack_int6(codes)), name
            got = g.dequantize_packed(packed, scales, shape[0], shape[1], torch.bfloat16)
            _bf16_bits_equal(got.view(torch.int16).cpu().numpy(), ox.dequantize_bf16(codes, s16))
            shapes.append(shape)
            all_codes.append(codes.ravel())
    hist = ox.code_histogram(np.concatenate(all_codes))
    assert np.array_equal(ex["hist"].cpu().numpy(), hist)
    assert abs(ex["entropy_bits"].item() - ox.entropy_bits(hist)) <= 1e-12
    assert ex["bytes"] == ox.artifact_bytes(shapes, pt)
    print(f"11l artifact {ex['bytes']} bytes, code entropy {ex['entropy_bits'].item():.4f} bits", flush=True)

    back = g.import_model(ex["packed"])
    tokens, nbytes = synth.make_stream(cfg, seed=7, n_tokens=2 * 2048 + 1)
    t, b = torch.from_numpy(tokens).cuda(), torch.from_numpy(nbytes).cuda()
    m0 = g.load(model, qb)
    n0, tot0 = m0.score(t, b, 2048, 1024)
    del m0
    m1 = g.load(model, back)
    n1, tot1 = m1.score(t, b, 2048, 1024)
    assert torch.equal(n0, n1) and torch.equal(tot0, tot1)
