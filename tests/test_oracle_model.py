"""Pins for the oracle's forward pass, windows and bits-per-byte (CPU only).

Pins used (none re-types the oracle's own formula):
  * attention against a scalar brute-force loop and exact special cases
    (T = 1, identical keys, GQA = MHA with repeated KV heads);
  * RoPE: identity at position 0, norm preservation, relative-position
    invariance, an explicit angle;
  * MLP / norm: a hand-worked 2-d example, scale invariance;
  * LoRA: equals the merged weight W + B A; B = 0 is the base model;
  * BigramHash hand values; zero table is a no-op;
  * schedules: zero skip weights = plain stack, the loop equals a flat
    model with duplicated blocks, the pages' U-Net split;
  * loss: uniform logits give ln V per token and bpb = log2(V) P / bytes,
    log-softmax agrees with scipy's logsumexp;
  * windows: every prediction scored once, chunked eval = stride L, a
    context-free model is independent of L and S, stride 1 equals scoring
    each prediction with its own truncated context;
  * the pages' printed (loss, bpb) pairs share one bytes/token ratio.
"""
import math
import os

import numpy as np
import pytest
from scipy.special import logsumexp

import synth
from oracle import quant as oq
from oracle import quant, model as om, windows as ow

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _tiny(seed=1, **ov):
    cfg = synth.config("tiny", **ov)
    m = synth.make_model(cfg["arch"], seed=seed)
    return cfg, quant.quantize_model(m)


# ---------------------------------------------------------------- attention
def _brute_attention(q, k, v):
    T, Hq, hd = q.shape
    Hkv = k.shape[1]
    out = np.zeros_like(q)
    for h in range(Hq):
        g = h // (Hq // Hkv)
        for i in range(T):
            w = [math.exp(sum(q[i, h, c] * k[j, g, c] for c in range(hd)) / math.sqrt(hd))
                 for j in range(i + 1)]
            z = sum(w)
            for c in range(hd):
                out[i, h, c] = sum(w[j] * v[j, g, c] for j in range(i + 1)) / z
    return out


def test_attention_brute_force():
    rng = np.random.default_rng(0)
    for T, Hq, Hkv, hd in [(1, 2, 1, 4), (5, 4, 2, 8), (8, 6, 3, 4), (7, 2, 2, 6)]:
        q = rng.normal(size=(T, Hq, hd))
        k = rng.normal(size=(T, Hkv, hd))
        v = rng.normal(size=(T, Hkv, hd))
        np.testing.assert_allclose(om.causal_attention(q, k, v), _brute_attention(q, k, v),
                                   rtol=1e-12, atol=1e-12)


def test_attention_special_cases():
    rng = np.random.default_rng(1)
    T, hd = 6, 8
    q = rng.normal(size=(T, 4, hd))
    v = rng.normal(size=(T, 2, hd))
    k = np.repeat(rng.normal(size=(1, 2, hd)), T, axis=0)    # identical keys
    o = om.causal_attention(q, k, v)
    prefix_mean = np.cumsum(v, axis=0) / np.arange(1, T + 1)[:, None, None]
    for h in range(4):
        np.testing.assert_allclose(o[:, h], prefix_mean[:, h // 2], atol=1e-12)
    o1 = om.causal_attention(q[:1], rng.normal(size=(1, 2, hd)), v[:1])
    np.testing.assert_allclose(o1[0, 3], v[0, 1], atol=1e-15)
    # GQA == MHA with each KV head repeated for its consecutive query heads
    k = rng.normal(size=(T, 2, hd))
    np.testing.assert_allclose(om.causal_attention(q, k, v),
                               om.causal_attention(q, np.repeat(k, 2, axis=1), np.repeat(v, 2, axis=1)),
                               atol=1e-13)


# ---------------------------------------------------------------- RoPE
def test_rope_properties():
    rng = np.random.default_rng(2)
    T, H, hd = 9, 2, 16
    x = rng.normal(size=(T, H, hd))
    y = om.rope(x, 10000.0)
    np.testing.assert_allclose(y[0], x[0], atol=1e-15)
    half = hd // 2
    nx = x[..., :half] ** 2 + x[..., half:] ** 2
    ny = y[..., :half] ** 2 + y[..., half:] ** 2
    np.testing.assert_allclose(nx, ny, rtol=1e-12)
    q = rng.normal(size=(1, 1, hd))
    k = rng.normal(size=(1, 1, hd))
    def dot(pq, pk):
        return float(np.sum(om.rope(q, 500.0, [pq]) * om.rope(k, 500.0, [pk])))
    assert abs(dot(7, 3) - dot(107, 103)) < 1e-10
    assert abs(dot(7, 3) - dot(4, 0)) < 1e-10
    # hd = 2: the single pair rotates by exactly p radians (theta_0 = 1)
    e = np.zeros((1, 1, 2)); e[0, 0, 0] = 1.0
    r = om.rope(e, 10000.0, [1.0])
    np.testing.assert_allclose(r[0, 0], [math.cos(1.0), math.sin(1.0)], atol=1e-15)
    # second pair of hd = 4 uses theta_1 = base^(-1/2)
    e = np.zeros((1, 1, 4)); e[0, 0, 1] = 1.0
    r = om.rope(e, 100.0, [2.0])
    np.testing.assert_allclose(r[0, 0], [0, math.cos(0.2), 0, math.sin(0.2)], atol=1e-15)


# ---------------------------------------------------------------- MLP / norm
def test_block_mlp_hand_example():
    """d = 2, x = (3, 4), eps = 0: N(x) = (3, 4)/sqrt(12.5) = (0.8485.., 1.1314..);
    fc = diag(1, -1) -> relu -> (0.8485.., 0); squared -> (0.72, 0);
    proj = I -> x + (0.72, 0) = (3.72, 4).  Attention output weight 0."""
    arch = dict(n_heads=1, n_kv_heads=1, head_dim=2, norm_eps=0.0, rope_base=10000.0,
                parallel=False)
    W = {"q": np.eye(2), "k": np.eye(2), "v": np.eye(2), "o": np.zeros((2, 2)),
         "fc": np.diag([1.0, -1.0]), "proj": np.eye(2)}
    out = om.block_forward(np.array([[3.0, 4.0]]), W, arch)
    np.testing.assert_allclose(out, [[3.72, 4.0]], atol=1e-14)


def test_rms_norm_scale_invariance():
    rng = np.random.default_rng(3)
    x = rng.normal(size=(4, 64))
    np.testing.assert_allclose(om.rms_norm(7.5 * x, 0.0), om.rms_norm(x, 0.0), atol=1e-14)
    np.testing.assert_allclose(np.mean(om.rms_norm(x, 0.0) ** 2, axis=1), 1.0, atol=1e-14)


# ---------------------------------------------------------------- LoRA / bigram
def test_lora_equals_merged_weight():
    rng = np.random.default_rng(4)
    d, hd, T, r = 16, 4, 5, 2
    arch = dict(n_heads=4, n_kv_heads=2, head_dim=hd, norm_eps=1e-6, rope_base=10000.0,
                parallel=False)
    W = {n: rng.normal(0, 0.2, size=s) for n, s in
         dict(q=(d, d), k=(8, d), v=(8, d), o=(d, d), fc=(32, d), proj=(d, 32)).items()}
    aq, bq = rng.normal(size=(r, d)), rng.normal(size=(d, r))
    av, bv = rng.normal(size=(r, d)), rng.normal(size=(8, r))
    x = rng.normal(size=(T, d))
    merged = dict(W)
    merged["q"] = W["q"] + bq @ aq
    merged["v"] = W["v"] + bv @ av
    np.testing.assert_allclose(om.block_forward(x, W, arch, (aq, bq, av, bv)),
                               om.block_forward(x, merged, arch), atol=1e-12)
    zero = (aq, np.zeros_like(bq), av, np.zeros_like(bv))
    np.testing.assert_allclose(om.block_forward(x, W, arch, zero), om.block_forward(x, W, arch),
                               atol=1e-15)


def test_bigram_hash_values():
    u = np.array([5, 1, 2, 1023, 0])
    h = om.bigram_buckets(u, 4096)
    assert h[0] == 0
    assert h[2] == 581                          # (1*1000003 + 2) mod 4096 = 1000005 mod 4096
    assert h[1] == (5 * 1000003 + 1) % 4096
    assert h[3] == (2 * 1000003 + 1023) % 4096
    assert h[4] == (1023 * 1000003) % 4096


def test_zero_bigram_table_is_noop():
    cfg = synth.config("midcycle", schedule=[0, 1, 2, 3], n_skip=2, d_model=64, n_heads=4,
                       n_kv_heads=2, vocab=64)
    m = synth.make_model(cfg["arch"], seed=3)
    qm = quant.quantize_model(m)
    u = np.array([3, 9, 2, 7, 7, 1])
    base = om.window_logits(qm, u)
    qm0 = dict(qm); qm0["bigram"] = {"table": np.zeros_like(m["bigram"]["table"]),
                                     "proj": m["bigram"]["proj"]}
    qmN = dict(qm); qmN["bigram"] = None
    np.testing.assert_allclose(om.window_logits(qm0, u), om.window_logits(qmN, u), atol=1e-14)
    assert np.max(np.abs(base - om.window_logits(qmN, u))) > 0


# ---------------------------------------------------------------- schedules
def test_unet_split_matches_pages():
    """11 layers: 5 encoder layers push, 6 decoder layers, the first 5 pop in
    reverse order with skip_weights[i] (num_encoder_layers = num_layers // 2)."""
    push, pop = om.skip_plan(synth.CONFIGS["11l"]["arch"])
    assert push == [True] * 5 + [False] * 6
    assert pop == [-1] * 5 + [0, 1, 2, 3, 4, -1]
    push, pop = om.skip_plan(synth.CONFIGS["baseline"]["arch"])
    assert push == [True] * 4 + [False] * 5 and pop == [-1] * 4 + [0, 1, 2, 3, -1]
    push, pop = om.skip_plan(synth.CONFIGS["midcycle"]["arch"])
    assert push == [True] * 3 + [False] * 12 and pop == [-1] * 12 + [0, 1, 2]


def test_midcycle_and_loop_schedules():
    """Stem 3 -> core 3 x 3 -> tail 3 = 15 effective over 9 unique blocks;
    layers 4-5 looped twice over 11 blocks = 13 effective."""
    a = synth.CONFIGS["midcycle"]["arch"]
    assert a["n_eff"] == 15 and a["n_unique"] == 9
    assert a["schedule"][3:12] == [3, 4, 5] * 3
    b = synth.CONFIGS["largevocab"]["arch"]
    assert b["n_eff"] == 13 and b["n_unique"] == 11


def test_zero_skip_weights_is_plain_stack():
    cfg = synth.config("baseline", d_model=64, n_heads=4, n_kv_heads=2, vocab=128,
                       schedule=[0, 1, 2, 3, 4])
    m = synth.make_model(cfg["arch"], seed=5)
    qm = quant.quantize_model(m)
    u = np.arange(7) * 5 % 128
    qz = dict(qm); qz["skip_w"] = np.zeros_like(m["skip_w"])
    flat = dict(qm); flat["arch"] = dict(qm["arch"], skip_kind="none", n_skip=0); flat["skip_w"] = None
    np.testing.assert_allclose(om.window_logits(qz, u), om.window_logits(flat, u), atol=1e-14)
    assert np.max(np.abs(om.window_logits(qm, u) - om.window_logits(flat, u))) > 1e-6


def test_loop_equals_flat_with_duplicated_blocks():
    cfg = synth.config("largevocab", vocab=256, d_model=64, n_heads=4, n_kv_heads=2,
                       schedule=[0, 1, 2, 1, 2, 3])
    m = synth.make_model(cfg["arch"], seed=6)
    qm = quant.quantize_model(m)
    flat = dict(qm)
    flat["arch"] = dict(qm["arch"], schedule=[0, 1, 2, 3, 4, 5])
    qb = qm["qblocks"]
    flat["qblocks"] = [qb[0], qb[1], qb[2], qb[1], qb[2], qb[3]]
    u = np.array([1, 200, 3, 17, 17, 90, 4])
    np.testing.assert_array_equal(om.window_logits(qm, u), om.window_logits(flat, u))


# ---------------------------------------------------------------- loss / bpb
def test_uniform_logits_closed_form():
    cfg, qm = _tiny()
    qm = dict(qm); qm["embed"] = np.zeros_like(qm["embed"])
    tokens, nbytes = synth.make_stream(cfg, seed=9, n_tokens=300)
    nats, mask = ow.score(qm, tokens, 128, 64)
    assert mask.all()
    np.testing.assert_allclose(nats, math.log(1024), rtol=1e-14)
    want = math.log2(1024) * len(nats) / float(nbytes[1:].sum())
    assert abs(ow.bpb(nats, nbytes) - want) < 1e-12


def test_log_softmax_matches_library():
    rng = np.random.default_rng(10)
    logits = rng.normal(0, 3, size=(12, 50))
    tgt = rng.integers(0, 50, size=12)
    want = logsumexp(logits, axis=1) - logits[np.arange(12), tgt]
    np.testing.assert_allclose(om.log_softmax_nll(logits, tgt), want, rtol=1e-13)
    np.testing.assert_allclose(om.log_softmax_nll(logits + 123.0, tgt), want, rtol=1e-12)


def test_pages_loss_bpb_pairs_share_one_ratio():
    """bpb = loss / ln 2 * tokens/bytes: all (loss, bpb) pairs printed for the
    same validation set must give one tokens/bytes ratio."""
    pairs = []
    with open(os.path.join(GOLDEN, "pages_loss_bpb.txt")) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if line:
                a, b = line.split()
                pairs.append((float(a), float(b)))
    # tokens/bytes from the 3-seed mean; reproduce every other pair through ow.bpb
    loss0, bpb0 = pairs[0]
    tpb = bpb0 * math.log(2.0) / loss0
    P = 1_000_000
    total_bytes = round(P / tpb)
    nbytes = np.zeros(P + 1, dtype=np.int64)
    nbytes[1:] = total_bytes // P
    nbytes[1:1 + total_bytes % P] += 1                   # spread the remainder
    for loss, b in pairs:
        got = ow.bpb(np.full(P, loss), nbytes)
        # half a unit in the last printed digit of each number, plus the
        # byte-count discretisation of this check (1 byte in ~2.4e6)
        half_b = 0.5 * 10.0 ** -(len(f"{b!r}".split(".")[1]))
        half_l = 0.5 * 10.0 ** -(len(f"{loss!r}".split(".")[1]))
        tol = half_b + (b / loss) * half_l + 1e-6
        assert abs(got - b) < tol, (loss, b, got)


# ---------------------------------------------------------------- windows
def test_window_plan_covers_each_prediction_once():
    for n, L, S in [(1025, 256, 256), (1000, 128, 64), (3000, 512, 100), (50, 128, 64),
                    (2, 1, 1), (1_048_576, 2048, 64), (4_194_304, 2048, 64), (65_537, 2048, 2048)]:
        plan = ow.plan_windows(n, L, S)
        P = n - 1
        cover = np.zeros(P, dtype=np.int64)
        for s, e, a in plan:
            assert 0 <= s <= a <= e <= P and e - s <= L
            cover[a:e] += 1
        assert np.all(cover == 1)
        K = 1 if P <= L else 1 + math.ceil((P - L) / S)
        assert len(plan) == K
    plan = ow.plan_windows(1_048_576, 2048, 64)
    assert len(plan) == 16_353
    s, e, a = plan[-1]
    assert e - s == 2047 and e - a == 63
    assert all(e - a == 64 for s, e, a in plan[1:-1])


def test_chunked_is_stride_equal_window():
    cfg, qm = _tiny(seed=2)
    tokens, _ = synth.make_stream(cfg, seed=2, n_tokens=4 * 32 + 1)
    nats, _ = ow.score(qm, tokens, 32, 32)
    for c in range(4):
        u = tokens[32 * c: 32 * c + 32]
        lg = om.window_logits(qm, u)
        np.testing.assert_allclose(nats[32 * c: 32 * c + 32],
                                   om.log_softmax_nll(lg, tokens[32 * c + 1: 32 * c + 33]), atol=1e-13)


def test_context_free_model_independent_of_windows():
    cfg, qm = _tiny(seed=3)
    qm = dict(qm)
    qm["qblocks"] = [dict(qb, o=(np.zeros_like(qb["o"][0]), qb["o"][1]),
                          proj=(np.zeros_like(qb["proj"][0]), qb["proj"][1]))
                     for qb in qm["qblocks"]]
    tokens, _ = synth.make_stream(cfg, seed=3, n_tokens=97)
    a, _ = ow.score(qm, tokens, 96, 96)
    b, _ = ow.score(qm, tokens, 16, 5)
    c, _ = ow.score(qm, tokens, 7, 1)
    np.testing.assert_allclose(a, b, atol=1e-12)
    np.testing.assert_allclose(a, c, atol=1e-12)


def test_stride_one_is_per_prediction_context():
    cfg, qm = _tiny(seed=4)
    tokens, _ = synth.make_stream(cfg, seed=4, n_tokens=23)
    L = 6
    nats, _ = ow.score(qm, tokens, L, 1)
    for p in range(len(tokens) - 1):
        ctx = tokens[max(0, p + 1 - L): p + 1]
        lg = om.window_logits(qm, ctx)
        want = om.log_softmax_nll(lg[-1:], tokens[p + 1: p + 2])[0]
        assert abs(nats[p] - want) < 1e-12, p


# ---------------------------------------------------------------------------
# Evaluation variants (kwkr.cn PR #363 write-up: EVAL_TEMPERATURE, LeakyReLU,
# Partial RoPE 16/64, XSA on the last layers, cyclic block schedule)
# ---------------------------------------------------------------------------

def test_partial_rope_hand_example_and_passthrough():
    # hd = 6, R = 4: pairs (0, 2) and (1, 3) with theta = 1 and 10000^(-1/2);
    # dims 4, 5 unrotated
    x = np.arange(1.0, 7.0).reshape(1, 1, 6) * np.ones((2, 1, 6))
    y = om.rope(x, 10000.0, dims=4)
    assert np.array_equal(y[0], x[0])                 # position 0: identity
    a0, a1 = 1.0, 0.01
    x1 = np.array([1.0, 2.0]); x2 = np.array([3.0, 4.0])
    c = np.cos([a0, a1]); s = np.sin([a0, a1])
    want = np.concatenate([x1 * c - x2 * s, x1 * s + x2 * c, [5.0, 6.0]])
    np.testing.assert_allclose(y[1, 0], want, rtol=0, atol=1e-15)


def test_partial_rope_reduces_to_full_rope_on_its_dims():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((9, 2, 64))
    full = om.rope(x, 10000.0)
    assert np.array_equal(om.rope(x, 10000.0, dims=64), full)
    part = om.rope(x, 10000.0, dims=16)
    np.testing.assert_array_equal(part[..., 16:], x[..., 16:])
    np.testing.assert_allclose(part[..., :16], om.rope(x[..., :16].copy(), 10000.0), rtol=0, atol=1e-14)


def test_partial_rope_scores_depend_on_relative_position_only():
    rng = np.random.default_rng(4)
    q = rng.standard_normal(64); k = rng.standard_normal(64)
    def score(m, n):
        qq = om.rope(np.tile(q, (max(m, n) + 1, 1, 1)), 10000.0, dims=16)[m, 0]
        kk = om.rope(np.tile(k, (max(m, n) + 1, 1, 1)), 10000.0, dims=16)[n, 0]
        return qq @ kk
    assert abs(score(7, 3) - score(14, 10)) < 1e-12
    assert abs(score(5, 5) - q @ k) < 1e-12


def test_xsa_removes_the_own_value_component():
    rng = np.random.default_rng(5)
    T, Hq, Hkv, hd = 6, 4, 2, 8
    o = rng.standard_normal((T, Hq, hd)); v = rng.standard_normal((T, Hkv, hd))
    y = om.exclusive_self_attention(o, v)
    for h in range(Hq):
        g = (h * Hkv) // Hq
        # orthogonal to the own-position value vector ...
        np.testing.assert_allclose(np.sum(y[:, h] * v[:, g], axis=1), 0.0, atol=1e-12)
        # ... and o minus y is parallel to it
        d = o[:, h] - y[:, h]
        cross = d[:, :, None] * v[:, g, None, :] - d[:, None, :] * v[:, g, :, None]
        np.testing.assert_allclose(cross, 0.0, atol=1e-12)
    # o along v -> 0; o orthogonal to v -> unchanged; zero v -> unchanged
    vv = rng.standard_normal((1, 1, hd))
    assert np.allclose(om.exclusive_self_attention(3.0 * vv, vv), 0.0)
    w = rng.standard_normal(hd); w -= (w @ vv[0, 0]) / (vv[0, 0] @ vv[0, 0]) * vv[0, 0]
    np.testing.assert_allclose(om.exclusive_self_attention(w.reshape(1, 1, hd), vv), w.reshape(1, 1, hd), atol=1e-13)
    assert np.array_equal(om.exclusive_self_attention(o[:1, :1], np.zeros((1, 1, hd))), o[:1, :1])


def test_xsa_single_token_window_cancels_attention():
    # one position: attention returns the value itself, so XSA leaves only
    # the MLP branch of the block
    rng = np.random.default_rng(6)
    arch = dict(n_heads=4, n_kv_heads=2, head_dim=8, norm_eps=1e-6, rope_base=10000.0,
                parallel=False, leaky_slope=0.0, rope_dims=None)
    d, F = 32, 64
    W = {"q": rng.standard_normal((d, d)), "k": rng.standard_normal((16, d)),
         "v": rng.standard_normal((16, d)), "o": rng.standard_normal((d, d)),
         "fc": rng.standard_normal((F, d)), "proj": rng.standard_normal((d, F))}
    x = rng.standard_normal((1, d))
    y = om.block_forward(x, W, arch, xsa=True)
    a2 = om.rms_norm(x, 1e-6)
    want = x + np.square(np.maximum(a2 @ W["fc"].T, 0.0)) @ W["proj"].T
    np.testing.assert_allclose(y, want, rtol=1e-12, atol=1e-12)


def test_leaky_relu_square_hand_values():
    z = np.array([-2.0, -0.5, 0.0, 3.0])
    np.testing.assert_array_equal(om.mlp_act(z, 0.5), [1.0, 0.0625, 0.0, 9.0])
    np.testing.assert_array_equal(om.mlp_act(z, 0.0), [0.0, 0.0, 0.0, 9.0])
    np.testing.assert_array_equal(om.mlp_act(z, 1.0), z * z)


def _tiny_variant_model(**kw):
    cfg = synth.config("11l_next", d_model=128, n_heads=2, n_kv_heads=1, vocab=128,
                       schedule=[0, 1, 0, 1], n_skip=2, **kw)
    model = synth.make_model(cfg["arch"], seed=7)
    return cfg, oq.quantize_model(model)


def test_temperature_scales_logits_and_two_logit_closed_form():
    cfg, qm = _tiny_variant_model()
    u = np.arange(10) % 128
    base = dict(qm); base["arch"] = dict(qm["arch"], temperature=1.0)
    hot = dict(qm); hot["arch"] = dict(qm["arch"], temperature=0.9)
    np.testing.assert_allclose(om.window_logits(hot, u), om.window_logits(base, u) / 0.9, rtol=1e-15)
    # two logits (a, b), target 0: nats = log(1 + exp((b - a)))
    a, b = 0.3, 1.7
    assert abs(om.log_softmax_nll(np.array([[a, b]]), np.array([0]))[0] - np.log1p(np.exp(b - a))) < 1e-15


def test_variants_off_reduce_to_the_base_model():
    cfg, qm = _tiny_variant_model()
    u = (np.arange(40) * 7) % 128
    off = dict(qm); off["arch"] = dict(qm["arch"], temperature=1.0, leaky_slope=0.0,
                                        rope_dims=None, xsa_last_n=0)
    plain = dict(qm); plain["arch"] = {k: v for k, v in off["arch"].items()
                                       if k not in ("temperature", "leaky_slope", "rope_dims", "xsa_last_n")}
    assert np.array_equal(om.window_logits(off, u), om.window_logits(plain, u))
    full_rope = dict(qm); full_rope["arch"] = dict(off["arch"], rope_dims=qm["arch"]["head_dim"])
    assert np.array_equal(om.window_logits(full_rope, u), om.window_logits(off, u))


def test_xsa_last_n_picks_the_last_effective_layers():
    # XSA on the last N layers = applying block_forward with xsa to exactly
    # those layers by hand (4 effective layers, U-Net 2/2)
    cfg, qm = _tiny_variant_model(xsa_last_n=1, temperature=1.0)
    arch = qm["arch"]
    u = (np.arange(12) * 5) % 128
    dense = [om.dense_weights(qb) for qb in qm["qblocks"]]
    E = qm["embed"].astype(np.float64)
    x = E[u]
    skip_w = qm["skip_w"].astype(np.float64)
    stack = []
    for e, b in enumerate(arch["schedule"]):
        if e >= 2:
            x = x + skip_w[e - 2] * stack.pop()
        x = om.block_forward(x, dense[b], arch, None, xsa=(e == 3))
        if e < 2:
            stack.append(x)
    want = om.rms_norm(x, arch["norm_eps"]) @ E.T
    np.testing.assert_allclose(om.window_logits(qm, u, dense), want, rtol=1e-13, atol=1e-13)


def test_cyclic_schedule_config():
    a = synth.CONFIGS["11l_next"]["arch"]
    assert a["schedule"] == [i % 4 for i in range(11)] and a["n_unique"] == 4
    push, pop = om.skip_plan(a)
    assert push == [True] * 5 + [False] * 6
    assert pop == [-1] * 5 + [0, 1, 2, 3, 4, -1]


# ---------------------------------------------------------------------------
# Hand-worked pins for three readings that end-to-end comparisons cannot see:
# the parallel residual lanes (pigsec.cn README mirror, leaderboard: parallel
# attention/MLP residual lanes), no bigram term at window position 0
# (kwkr.cn PR #363 write-up, BigramHash: the hash needs the previous token),
# and the final weightless RMSNorm before the tied head (pwwt.cn 11L write-up,
# 架构: tied input/output embedding).
# ---------------------------------------------------------------------------

def _context_free_qmodel(E, bigram=None, buckets=0, dim=0):
    """A d = 2, one-block model whose six matrices all have zero codes, so
    every block adds exactly 0 to the residual stream (q = k = v = 0, the
    attention output is 0, relu(0)^2 = 0): its logits depend only on the
    embedding layer, the bigram term and the head."""
    V, d = E.shape
    arch = dict(vocab=V, d_model=d, n_heads=1, n_kv_heads=1, head_dim=d, d_ff=d, rope_base=10000.0,
                norm_eps=0.0, schedule=[0], n_unique=1, n_eff=1, skip_kind="none", n_skip=0,
                parallel=False, lora_rank=0, bigram_buckets=buckets, bigram_dim=dim, temperature=1.0,
                leaky_slope=0.0, rope_dims=None, xsa_last_n=0)
    one = np.ones(d, dtype=np.float16)
    qb = {n: (np.zeros((d, d), dtype=np.int8), one) for n in ("q", "k", "v", "o", "fc", "proj")}
    return dict(arch=arch, qblocks=[qb], embed=E, skip_w=None, lora=None, bigram=bigram)


_E4 = np.array([[1.0, 0.0], [0.0, 1.0], [1.0, 1.0], [2.0, -1.0]])


def test_parallel_lanes_hand_example():
    """d = 2, one token, eps = 0, x = (3, 4): a = N(x) = (3, 4)/sqrt(12.5) =
    (0.6 sqrt2, 0.8 sqrt2).  With one position the softmax weight is 1, so
    with Wv = I the attention output is a, and Wo = [[0, 1], [1, 0]] swaps it:
    attn = (0.8 sqrt2, 0.6 sqrt2).  fc = diag(1, -1), proj = I:
    MLP(a) = (relu(0.6 sqrt2)^2, 0) = (0.72, 0).
    Parallel lanes: x + attn + MLP(a) = (3.72 + 0.8 sqrt2, 4 + 0.6 sqrt2)
    = (4.851370850, 4.848528137).
    The sequential form feeds the MLP N(x + attn) = N(4.131371, 4.848528)
    instead, giving (4.9726585, 4.8485281); a mutation that re-normalises
    after attention, drops either lane, or adds a lane twice fails here."""
    r2 = math.sqrt(2.0)
    W = {"q": np.eye(2), "k": np.eye(2), "v": np.eye(2), "o": np.array([[0.0, 1.0], [1.0, 0.0]]),
         "fc": np.diag([1.0, -1.0]), "proj": np.eye(2)}
    arch = dict(n_heads=1, n_kv_heads=1, head_dim=2, norm_eps=0.0, rope_base=10000.0, parallel=True)
    x = np.array([[3.0, 4.0]])
    par = om.block_forward(x, W, arch)
    np.testing.assert_allclose(par, [[3.72 + 0.8 * r2, 4.0 + 0.6 * r2]], rtol=0, atol=1e-14)
    np.testing.assert_allclose(par, [[4.851370850, 4.848528137]], rtol=0, atol=1e-9)
    seq = om.block_forward(x, W, dict(arch, parallel=False))
    x1 = np.array([3.0 + 0.8 * r2, 4.0 + 0.6 * r2])
    n1 = x1[0] / math.sqrt((x1[0] ** 2 + x1[1] ** 2) / 2.0)
    np.testing.assert_allclose(seq, [[x1[0] + n1 * n1, x1[1]]], rtol=0, atol=1e-13)
    assert abs(seq[0, 0] - par[0, 0]) > 0.1
    # the large-vocabulary configuration is the one that runs parallel lanes
    assert synth.config("largevocab")["arch"]["parallel"] is True
    assert all(not synth.config(n)["arch"]["parallel"] for n in ("tiny", "baseline", "11l", "midcycle"))


def test_bigram_absent_at_window_position_zero():
    """Context-free model, V = 4, d = 2, bigram table of 8 buckets x 1 with
    every row non-zero (B[h] = (h + 1) / 2) and projection P = (1, -1)^T.
    Window u = (1, 2): position 1 hashes (1 * 1000003 + 2) mod 8 = 5, so
    x0[1] = E[2] + P B[5] = (1, 1) + 3 (1, -1) = (4, -2); position 0 has no
    previous token and keeps x0[0] = E[1] = (0, 1) exactly (a term from any
    bucket would change it).  Logits are N(x0) E^T:
    row 0 = sqrt2 (0, 1, 1, -1); row 1 = (4, -2)/sqrt10 . E^T
    = (4, -2, 2, 10)/sqrt10."""
    table = ((np.arange(8, dtype=np.float64) + 1.0) / 2.0)[:, None]
    proj = np.array([[1.0], [-1.0]])
    qm = _context_free_qmodel(_E4, {"table": table, "proj": proj}, buckets=8, dim=1)
    assert (1 * 1000003 + 2) % 8 == 5
    lg = om.window_logits(qm, np.array([1, 2]))
    r2, r10 = math.sqrt(2.0), math.sqrt(10.0)
    np.testing.assert_allclose(lg[0], [0.0, r2, r2, -r2], rtol=0, atol=1e-14)
    np.testing.assert_allclose(lg[1], np.array([4.0, -2.0, 2.0, 10.0]) / r10, rtol=0, atol=1e-14)
    # the same window without the bigram: row 1 becomes N(1, 1) E^T = (1, 1, 2, 1)
    lg0 = om.window_logits(_context_free_qmodel(_E4), np.array([1, 2]))
    np.testing.assert_allclose(lg0[1], [1.0, 1.0, 2.0, 1.0], rtol=0, atol=1e-14)
    np.testing.assert_allclose(lg0[0], lg[0], rtol=0, atol=0)


def test_final_norm_before_tied_head_hand_example():
    """Context-free model: the logits are N(E[u]) E^T with the weightless
    RMSNorm of the final residual.  u = (3, 0): E[3] = (2, -1),
    N = (2, -1)/sqrt(2.5), logits = (2, -1, 1, 5)/sqrt(2.5)
    = (1.2649111, -0.6324555, 0.6324555, 3.1622777); E[0] = (1, 0),
    N = (sqrt2, 0), logits = sqrt2 (1, 0, 1, 2).  Without the final norm they
    would be (2, -1, 1, 5) and (1, 0, 1, 2).  The nats of predicting token 0
    after u0 = 3 are logsumexp(row 0) - row0[0], computed here by hand."""
    qm = _context_free_qmodel(_E4)
    lg = om.window_logits(qm, np.array([3, 0]))
    s = math.sqrt(2.5)
    np.testing.assert_allclose(lg[0], [2.0 / s, -1.0 / s, 1.0 / s, 5.0 / s], rtol=0, atol=1e-14)
    np.testing.assert_allclose(lg[0], [1.2649111, -0.6324555, 0.6324555, 3.1622777], rtol=0, atol=1e-7)
    np.testing.assert_allclose(lg[1], [math.sqrt(2.0), 0.0, math.sqrt(2.0), 2.0 * math.sqrt(2.0)],
                               rtol=0, atol=1e-14)
    tokens = np.array([3, 0, 2])
    nats, mask = ow.score(qm, tokens, 2, 2)
    assert mask.all()
    row0 = [2.0 / s, -1.0 / s, 1.0 / s, 5.0 / s]
    want0 = math.log(sum(math.exp(v) for v in row0)) - row0[0]
    row1 = [math.sqrt(2.0), 0.0, math.sqrt(2.0), 2.0 * math.sqrt(2.0)]
    want1 = math.log(sum(math.exp(v) for v in row1)) - row1[2]
    np.testing.assert_allclose(nats, [want0, want1], rtol=0, atol=1e-13)
