"""The C-ABI library on the CPU: it loads, exports every symbol its header
declares, plans windows exactly as the oracle does, and rejects invalid
arguments before touching a GPU."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib():
    import int6_row_gemm_amd as g
    if not os.path.exists(g.LIB_PATH):
        pytest.skip("libi6g.so not built (run __graft_entry__.build())")
    return g, g.lib()


def _header_functions():
    src = open(os.path.join(ROOT, "include", "i6g.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(i6g_[a-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    g, L = _lib()
    names = _header_functions()
    assert "i6g_score_tokens" in names and "i6g_quantize_rows" in names
    for n in names:
        assert hasattr(L, n), n
    assert sorted(g.EXPORTED) == names


@pytest.mark.parametrize("n,L,S", [(1025, 256, 256), (1000, 128, 64), (3000, 512, 100), (50, 128, 64),
                                   (2, 1, 1), (1_048_576, 2048, 64), (4_194_304, 2048, 64),
                                   (65_537, 2048, 2048), (400, 128, 128), (700, 200, 50)])
def test_window_plan_matches_oracle(n, L, S):
    g, _ = _lib()
    from oracle import windows
    st, en, sf = g.plan_windows(n, L, S)
    plan = windows.plan_windows(n, L, S)
    assert len(plan) == len(st)
    assert np.array_equal(st, [p[0] for p in plan])
    assert np.array_equal(en, [p[1] for p in plan])
    assert np.array_equal(sf, [p[2] for p in plan])


def test_argument_validation_without_gpu():
    g, L = _lib()
    fake = ctypes.c_void_p(0x1000)     # never dereferenced: validation fails first
    null = ctypes.c_void_p(0)
    # bits not in {6, 8}
    assert L.i6g_quantize_rows(fake, 4, 4, 7, 1.0, fake, fake, null, null) == -1
    # quantile outside (0, 1]
    assert L.i6g_quantize_rows(fake, 4, 4, 6, 1.5, fake, fake, null, null) == -1
    assert L.i6g_quantize_rows(fake, 4, 4, 6, 0.0, fake, fake, null, null) == -1
    # empty shapes and NULL arrays
    assert L.i6g_quantize_rows(fake, 0, 4, 6, 1.0, fake, fake, null, null) == -1
    assert L.i6g_quantize_rows(null, 4, 4, 6, 1.0, fake, fake, null, null) == -1
    # a quantile needing more than the 8 largest values of a row
    assert L.i6g_quantize_rows(fake, 4, 100, 6, 0.5, fake, fake, null, null) == -6
    assert "largest" in L.i6g_last_error().decode()
    # score_tokens / load_model on bad input
    assert L.i6g_score_tokens(null, fake, fake, 10, 4, 2, fake, fake, null) == -1
    out = ctypes.c_void_p(0)
    assert L.i6g_load_model(null, null, ctypes.byref(out)) == -1
    assert out.value is None
    n = ctypes.c_int64(0)
    assert L.i6g_plan_windows(10, 4, 5, ctypes.byref(n), None, None, None, 0) == -1
    assert L.i6g_plan_windows(1, 4, 2, ctypes.byref(n), None, None, None, 0) == -1


def test_load_model_rejects_bad_descriptors():
    g, L = _lib()
    d = g._Desc()
    d.vocab, d.d_model, d.n_heads, d.n_kv_heads, d.head_dim, d.d_ff = 1024, 512, 8, 4, 64, 1536
    d.n_unique, d.n_eff = 1, 1
    out = ctypes.c_void_p(0)
    # NULL schedule / blocks / embedding
    assert L.i6g_load_model(ctypes.byref(d), None, ctypes.byref(out)) == -1
    sched = (ctypes.c_int32 * 1)(0)
    blocks = (g._Block * 1)()
    emb = ctypes.c_void_p(0x1000)
    d.schedule = ctypes.cast(sched, ctypes.c_void_p)
    d.blocks = ctypes.cast(blocks, ctypes.c_void_p)
    d.embed = emb
    d.head_dim = 48
    d.n_heads = 10
    d.d_model = 480
    assert L.i6g_load_model(ctypes.byref(d), None, ctypes.byref(out)) in (-1, -6)
    d.d_model, d.n_heads, d.n_kv_heads, d.head_dim = 384, 6, 3, 64   # odd number of kv heads
    assert L.i6g_load_model(ctypes.byref(d), None, ctypes.byref(out)) == -6
    assert "kv heads" in L.i6g_last_error().decode()
    d.d_model, d.n_heads, d.n_kv_heads, d.head_dim = 512, 8, 4, 64
    # evaluation variants: partial RoPE granularity, XSA depth, temperature
    d.rope_dims = 24                     # not a multiple of head_dim / 4
    assert L.i6g_load_model(ctypes.byref(d), None, ctypes.byref(out)) == -6
    d.rope_dims = 80                     # more than head_dim
    assert L.i6g_load_model(ctypes.byref(d), None, ctypes.byref(out)) == -1
    d.rope_dims = 0
    d.xsa_last_n = 2                     # more than n_eff = 1
    assert L.i6g_load_model(ctypes.byref(d), None, ctypes.byref(out)) == -1
    d.xsa_last_n = 0
    d.logit_temperature = -0.5
    assert L.i6g_load_model(ctypes.byref(d), None, ctypes.byref(out)) == -1
    assert "temperature" in L.i6g_last_error().decode()
    d.logit_temperature = 0.0
    bad = (ctypes.c_int32 * 1)(3)      # schedule names a block that does not exist
    d.schedule = ctypes.cast(bad, ctypes.c_void_p)
    assert L.i6g_load_model(ctypes.byref(d), None, ctypes.byref(out)) == -1
    assert "schedule" in L.i6g_last_error().decode()


def test_binding_refuses_missing_library(monkeypatch, tmp_path):
    import int6_row_gemm_amd as g
    monkeypatch.setattr(g, "_lib", None)
    monkeypatch.setattr(g, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        g.lib()


def test_quantize_rows_many_validates_before_enqueueing():
    g, L = _lib()
    assert L.i6g_quantize_rows_many(None, 1, 6, 0.9999984, None, None) == -1
    jobs = (g._QuantJob * 2)()
    assert L.i6g_quantize_rows_many(ctypes.cast(jobs, ctypes.c_void_p), 0, 6, 0.9999984, None, None) == -1
    # job 1 has NULL arrays
    jobs[0] = g._QuantJob(0x1000, 0x2000, 0x3000, 4, 512)
    assert L.i6g_quantize_rows_many(ctypes.cast(jobs, ctypes.c_void_p), 2, 6, 0.9999984, None, None) == -1
    assert "job 1" in L.i6g_last_error().decode()
    jobs[1] = g._QuantJob(0x1000, 0x2000, 0x3000, 4, 512)
    assert L.i6g_quantize_rows_many(ctypes.cast(jobs, ctypes.c_void_p), 2, 7, 0.9999984, None, None) == -1
    assert L.i6g_quantize_rows_many(ctypes.cast(jobs, ctypes.c_void_p), 2, 6, 0.5, None, None) == -6


def test_export_entry_points_validate_without_gpu():
    g, L = _lib()
    fake = ctypes.c_void_p(0x1000)     # 4096-aligned, never dereferenced
    odd = ctypes.c_void_p(0x1001)
    null = ctypes.c_void_p(0)
    for bits in (5, 6):
        assert L.i6g_pack_codes(fake, -1, bits, fake, null, null) == -1
        assert L.i6g_pack_codes(null, 4, bits, fake, null, null) == -1
        assert L.i6g_pack_codes(null, 0, bits, null, null, null) == 0          # nothing to do
        assert L.i6g_pack_codes(odd, 16, bits, fake, null, null) == -6
        assert L.i6g_unpack_codes(fake, 16, bits, odd, null) == -6
        assert L.i6g_unpack_codes(fake, -3, bits, fake, null) == -1
        assert L.i6g_dequantize_packed(fake, bits, fake, 4, 4, 2, odd, null) == -6
    for bits in (4, 7, 8):
        assert L.i6g_pack_codes(fake, 16, bits, fake, null, null) == -1
        assert L.i6g_unpack_codes(fake, 16, bits, fake, null) == -1
        assert L.i6g_dequantize_packed(fake, bits, fake, 4, 4, 2, fake, null) == -1
    assert L.i6g_dequantize_rows(fake, fake, 4, 4, 0, fake, null) == -1   # fp16 output: not offered
    assert L.i6g_dequantize_rows(fake, fake, -1, 4, 1, fake, null) == -1
    assert L.i6g_dequantize_rows(null, fake, 4, 4, 1, fake, null) == -1
    assert L.i6g_dequantize_rows(fake, fake, 0, 4, 2, null, null) == 0
    assert L.i6g_code_histogram(fake, 16, 0, null, null) == -1
    assert L.i6g_code_histogram(odd, 16, 0, fake, null) == -6
    assert L.i6g_code_entropy(null, fake, null) == -1
    out = ctypes.c_int64(0)
    assert L.i6g_artifact_bytes(None, None, -1, 0, ctypes.byref(out)) == -1
    assert L.i6g_artifact_bytes(None, None, 0, -5, ctypes.byref(out)) == -1
    bad = (ctypes.c_int64 * 2)(3, -1)
    assert L.i6g_artifact_bytes(bad, None, 1, 0, ctypes.byref(out)) == -1
    ok = (ctypes.c_int64 * 2)(3, 5)
    assert L.i6g_artifact_bytes(ok, (ctypes.c_int32 * 1)(7), 1, 0, ctypes.byref(out)) == -1


def test_artifact_bytes_matches_oracle():
    g, _ = _lib()
    from oracle import export as ox
    from oracle import quant as oq
    import synth
    for shapes, pt in [([(3, 5)], 7), ([(1, 4), (2, 2), (7, 1)], 0), ([], 11), ([(0, 5), (5, 0)], 1)]:
        assert g.artifact_bytes(shapes, pt) == ox.artifact_bytes(shapes, pt)
        for b in (5, 8):
            assert g.artifact_bytes(shapes, pt, [b] * len(shapes)) == ox.artifact_bytes(shapes, pt, [b] * len(shapes))
    for name in ("11l", "11l_next", "midcycle", "tiny", "11l_int5", "10l_int5mlp"):
        arch = synth.config(name)["arch"]
        ms = synth.matrix_shapes(arch)
        shapes = list(ms.values()) * len(set(arch["schedule"]))
        bits = [oq.matrix_bits(arch, k) for k in ms] * len(set(arch["schedule"]))
        pt = arch["vocab"] * arch["d_model"]
        assert g.artifact_bytes(shapes, pt, bits) == ox.artifact_bytes(shapes, pt, bits)


def test_qat_entry_points_validate_without_gpu():
    g, L = _lib()
    fake = ctypes.c_void_p(0x1000)
    odd = ctypes.c_void_p(0x1004)
    null = ctypes.c_void_p(0)
    assert L.i6g_fake_quantize_rows(fake, 4, 4, 7, 1.0, 1, fake, null, null) == -1     # bits
    assert L.i6g_fake_quantize_rows(fake, 4, 4, 6, 1.5, 1, fake, null, null) == -1     # quantile
    assert L.i6g_fake_quantize_rows(fake, 4, 4, 6, 1.0, 0, fake, null, null) == -1     # fp16 output
    assert L.i6g_fake_quantize_rows(null, 4, 4, 6, 1.0, 1, fake, null, null) == -1
    assert L.i6g_fake_quantize_rows(fake, 4, 100, 5, 0.5, 1, fake, null, null) == -6   # > 8 largest
    for levels in (0.0, -1.0, float("inf"), float("nan"), 1e300):
        assert L.i6g_noisy_weights(fake, 4, 4, levels, 1, 1, fake, null, null) == -1
    assert L.i6g_noisy_weights(fake, 0, 4, 127.0, 1, 1, fake, null, null) == -1
    assert L.i6g_noisy_weights(fake, 4, 4, 127.0, 1, 3, fake, null, null) == -1
    assert L.i6g_noisy_weights(odd, 4, 4, 127.0, 1, 1, fake, null, null) == -6
    assert L.i6g_noisy_weights(fake, 4, 4, 127.0, 1, 1, odd, null, null) == -6


def _host_desc(g, nan_at=None):
    """A well-formed 512-wide, one-block descriptor whose tensors are all in
    host memory; ``nan_at`` puts one NaN into the named tensor."""
    V, d, Hq, Hkv, hd, F = 1024, 512, 8, 4, 64, 1536
    kvd = Hkv * hd
    keep = []
    blocks = (g._Block * 1)()
    for name, (rows, cols) in dict(q=(d, d), k=(kvd, d), v=(kvd, d), o=(d, d), fc=(F, d), proj=(d, F)).items():
        c = np.zeros((rows, cols), np.int8)
        s = np.full(rows, 0.01, np.float16)
        if nan_at == name:
            s[rows // 2] = np.nan
        keep += [c, s]
        setattr(blocks[0], name, g._Matrix(c.ctypes.data, s.ctypes.data))
    emb = np.full((V, d), 0.02, np.float16)
    if nan_at == "embed":
        emb[3, 7] = np.inf
    skip = np.ones((1, d), np.float16)
    if nan_at == "skip":
        skip[0, 0] = -np.inf
    sched = (ctypes.c_int32 * 2)(0, 0)
    keep += [emb, skip, sched]
    D = g._Desc()
    D.vocab, D.d_model, D.n_heads, D.n_kv_heads, D.head_dim, D.d_ff = V, d, Hq, Hkv, hd, F
    D.rope_base, D.norm_eps = 10000.0, 1e-6
    D.n_unique, D.n_eff = 1, 2
    D.schedule = ctypes.cast(sched, ctypes.c_void_p)
    D.blocks = ctypes.cast(blocks, ctypes.c_void_p)
    D.embed_dtype, D.embed = 0, emb.ctypes.data
    D.skip_kind, D.n_skip, D.skip_weights = 1, 1, skip.ctypes.data
    return D, (blocks, keep)


@pytest.mark.parametrize("where", ["q", "v", "fc", "proj", "embed", "skip"])
def test_load_model_rejects_nonfinite_host_tensors(where):
    """A NaN or Inf row scale, embedding value or skip weight in host memory
    is refused with I6G_ENONFINITE before anything is allocated (so this
    runs without a GPU): [11L] 后训练量化导出 gives every row one finite
    binary16 scale."""
    g, L = _lib()
    D, keep = _host_desc(g, nan_at=where)
    out = ctypes.c_void_p(0)
    assert L.i6g_load_model(ctypes.byref(D), None, ctypes.byref(out)) == -4
    assert out.value is None
    assert "NaN or Inf" in L.i6g_last_error().decode()


def test_load_model_temperature_floor():
    """Temperatures in (0, 0.01) are refused: the head keeps the normed row
    times log2(e) / temperature in binary16, which would overflow."""
    g, L = _lib()
    D, keep = _host_desc(g, nan_at="q")
    out = ctypes.c_void_p(0)
    for t in (0.005, 1e-4):
        D.logit_temperature = t
        assert L.i6g_load_model(ctypes.byref(D), None, ctypes.byref(out)) == -6
        assert "temperature" in L.i6g_last_error().decode()
    D.logit_temperature = 0.01          # accepted: the NaN scale is what fails next
    assert L.i6g_load_model(ctypes.byref(D), None, ctypes.byref(out)) == -4
