"""Seeded synthetic inputs shared by the CPU oracle and the HIP path.

This module only draws random numbers and lays them out; it holds none of the
scoring method's arithmetic (no quantisation, no norm, no attention, no loss).
Both sides receive the same arrays from here and do their own work on them.

Workload shapes follow the five evaluation set-ups of this project:

* ``tiny``       2 layers, d=128, 4/2 heads, MLP 2x, fp32 tied embedding,
                 int8 rows with a plain amax scale, 4 sequences of 256 tokens.
* ``baseline``   9 layers, d=512, 8/4 heads, MLP 2x, fp16 embedding, U-Net
                 4 enc / 5 dec, int8 rows with the 99.99984th-percentile clip,
                 64 sequences of 1024 tokens.
* ``11l``        11 layers, d=512, 8/4 heads, MLP 3x, U-Net 5/6, int6 rows,
                 sliding window 2048 / stride 64 over 1,048,576 tokens.
* ``midcycle``   d=640, 8/4 heads (head dim 80), MLP 3x, 3 stem -> 3 core x 3
                 -> 3 tail blocks with stem->tail skips, rank-4 Q/V LoRA per
                 effective depth, BigramHash 4096 x 128, int6, 32 x 2048.
* ``largevocab`` vocab 8192, 11 layers, d=512, MLP 4x, layers 4-5 run twice,
                 parallel attention/MLP lanes, int6, window 2048 / stride 64
                 over 4,194,304 tokens.

Token streams are truncated Zipf (rank r has weight r^-s, id = r-1); byte
counts are i.i.d. uniform integers.  Random streams come from NumPy's PCG64
through ``SeedSequence(seed).spawn(3)`` -> (weights, tokens, bytes).
"""
from __future__ import annotations

import copy
import numpy as np

SEEDS = (1337, 42, 123)

SKIP_NONE = "none"
SKIP_UNET = "unet"
SKIP_STEM_TAIL = "stem_tail"

_BASE = dict(
    rope_base=10000.0,
    norm_eps=1e-6,
    skip_kind=SKIP_NONE,
    n_skip=0,
    parallel=False,
    lora_rank=0,
    bigram_buckets=0,
    bigram_dim=0,
    embed_dtype="fp16",
    bits=6,
    clip_q=0.9999984,
    # mixed precision: bits of the attention (q, k, v, o) and MLP (fc, proj)
    # matrices when they differ from ``bits`` (None = ``bits``)
    bits_attn=None,
    bits_mlp=None,
    # evaluation variants (off by default): logits divided by the
    # temperature, MLP activation leaky_relu(x, slope)^2, RoPE on the first
    # rope_dims dims of each head (None = all), exclusive self attention on
    # the last xsa_last_n effective layers
    temperature=1.0,
    leaky_slope=0.0,
    rope_dims=None,
    xsa_last_n=0,
)


def _arch(**kw):
    a = dict(_BASE)
    a.update(kw)
    a["head_dim"] = a["d_model"] // a["n_heads"]
    a["d_ff"] = a["mlp_mult"] * a["d_model"]
    a["n_unique"] = 1 + max(a["schedule"])
    a["n_eff"] = len(a["schedule"])
    return a


CONFIGS = {
    "tiny": dict(
        arch=_arch(vocab=1024, d_model=128, n_heads=4, n_kv_heads=2, mlp_mult=2,
                   schedule=[0, 1], embed_dtype="fp32", bits=8, clip_q=1.0),
        n_tokens=4 * 256 + 1, zipf=1.1, bytes_max=6, window=256, stride=256,
    ),
    "baseline": dict(
        arch=_arch(vocab=1024, d_model=512, n_heads=8, n_kv_heads=4, mlp_mult=2,
                   schedule=list(range(9)), skip_kind=SKIP_UNET, n_skip=4,
                   bits=8, clip_q=0.9999984),
        n_tokens=64 * 1024 + 1, zipf=1.1, bytes_max=8, window=1024, stride=1024,
    ),
    "11l": dict(
        arch=_arch(vocab=1024, d_model=512, n_heads=8, n_kv_heads=4, mlp_mult=3,
                   schedule=list(range(11)), skip_kind=SKIP_UNET, n_skip=5),
        n_tokens=1_048_576, zipf=1.1, bytes_max=8, window=2048, stride=64,
    ),
    "midcycle": dict(
        arch=_arch(vocab=1024, d_model=640, n_heads=8, n_kv_heads=4, mlp_mult=3,
                   schedule=[0, 1, 2] + [3, 4, 5] * 3 + [6, 7, 8],
                   skip_kind=SKIP_STEM_TAIL, n_skip=3, lora_rank=4,
                   bigram_buckets=4096, bigram_dim=128),
        n_tokens=32 * 2048 + 1, zipf=1.1, bytes_max=8, window=2048, stride=2048,
    ),
    # the 11-layer model with the evaluation variants the pages list next:
    # temperature 0.90, LeakyReLU(0.5)^2, partial RoPE 16/64, XSA on the last
    # 4 effective layers, and a cyclic schedule i % 4 over 11 effective
    # layers with U-Net skips over the effective depth
    "11l_next": dict(
        arch=_arch(vocab=1024, d_model=512, n_heads=8, n_kv_heads=4, mlp_mult=3,
                   schedule=[i % 4 for i in range(11)], skip_kind=SKIP_UNET, n_skip=5,
                   temperature=0.90, leaky_slope=0.5, rope_dims=16, xsa_last_n=4),
        n_tokens=1_048_576, zipf=1.1, bytes_max=8, window=2048, stride=64,
    ),
    # the flat 11-layer model exported with every block matrix at int5
    # (MLP_INT5 and ATTN_INT5 in the PR #363 write-up's run commands)
    "11l_int5": dict(
        arch=_arch(vocab=1024, d_model=512, n_heads=8, n_kv_heads=4, mlp_mult=3,
                   schedule=list(range(11)), skip_kind=SKIP_UNET, n_skip=5, bits=5),
        n_tokens=1_048_576, zipf=1.1, bytes_max=8, window=2048, stride=64,
    ),
    # 10 layers with int5 MLP matrices and int6 attention matrices (the
    # mixed int5 / int6 "10L Int5-MLP" entry of the records table)
    "10l_int5mlp": dict(
        arch=_arch(vocab=1024, d_model=512, n_heads=8, n_kv_heads=4, mlp_mult=3,
                   schedule=list(range(10)), skip_kind=SKIP_UNET, n_skip=5, bits=6, bits_mlp=5),
        n_tokens=1_048_576, zipf=1.1, bytes_max=8, window=2048, stride=64,
    ),
    "largevocab": dict(
        arch=_arch(vocab=8192, d_model=512, n_heads=8, n_kv_heads=4, mlp_mult=4,
                   schedule=[0, 1, 2, 3, 4, 5, 4, 5, 6, 7, 8, 9, 10],
                   parallel=True),
        n_tokens=4_194_304, zipf=1.05, bytes_max=12, window=2048, stride=64,
    ),
}

MATRICES = ("q", "k", "v", "o", "fc", "proj")


def matrix_shapes(arch):
    """[out, in] shape of each of the six block matrices."""
    d, f = arch["d_model"], arch["d_ff"]
    kvd = arch["n_kv_heads"] * arch["head_dim"]
    return {"q": (d, d), "k": (kvd, d), "v": (kvd, d), "o": (d, d),
            "fc": (f, d), "proj": (d, f)}


def config(name, **overrides):
    """A deep copy of a named set-up; ``overrides`` replace arch or workload keys."""
    c = copy.deepcopy(CONFIGS[name])
    arch_keys = set(c["arch"]) | {"mlp_mult"}
    for k, v in overrides.items():
        if k in arch_keys:
            c["arch"][k] = v
        else:
            c[k] = v
    a = c["arch"]
    a["head_dim"] = a["d_model"] // a["n_heads"]
    a["d_ff"] = a["mlp_mult"] * a["d_model"]
    a["n_unique"] = 1 + max(a["schedule"])
    a["n_eff"] = len(a["schedule"])
    return c


def _streams(seed):
    ss = np.random.SeedSequence(seed)
    w, t, b = ss.spawn(3)
    return (np.random.Generator(np.random.PCG64(w)),
            np.random.Generator(np.random.PCG64(t)),
            np.random.Generator(np.random.PCG64(b)))


def make_model(arch, seed=1337, lora_b_std=0.01, bigram_scale=1.0, skip_scale=1.0):
    """Random-init weights for ``arch``.

    Block matrices are fp32 N(0, 0.02) [out, in] (to be row-quantised by each
    side).  The tied embedding, skip weights, LoRA factors and bigram tensors
    are stored the way they are kept at export: fp16 (embedding fp32 for the
    tiny set-up).  ``lora_b_std``, ``bigram_scale`` and ``skip_scale`` let
    tests amplify small components.
    """
    rw, _, _ = _streams(seed)
    V, d = arch["vocab"], arch["d_model"]
    shapes = matrix_shapes(arch)
    blocks = []
    for _ in range(arch["n_unique"]):
        blocks.append({m: rw.normal(0.0, 0.02, size=shapes[m]).astype(np.float32)
                       for m in MATRICES})
    emb = rw.normal(0.0, 0.02, size=(V, d))
    emb = emb.astype(np.float32 if arch["embed_dtype"] == "fp32" else np.float16)
    model = {"arch": dict(arch), "blocks": blocks, "embed": emb,
             "skip_w": None, "lora": None, "bigram": None}
    if arch["n_skip"] > 0:
        model["skip_w"] = (rw.uniform(0.5, 1.5, size=(arch["n_skip"], d))
                           * skip_scale).astype(np.float16)
    r = arch["lora_rank"]
    if r > 0:
        ne, kvd = arch["n_eff"], arch["n_kv_heads"] * arch["head_dim"]
        model["lora"] = {
            "aq": rw.normal(0.0, 0.02, size=(ne, r, d)).astype(np.float16),
            "bq": rw.normal(0.0, lora_b_std, size=(ne, d, r)).astype(np.float16),
            "av": rw.normal(0.0, 0.02, size=(ne, r, d)).astype(np.float16),
            "bv": rw.normal(0.0, lora_b_std, size=(ne, kvd, r)).astype(np.float16),
        }
    if arch["bigram_buckets"] > 0:
        nb, bd = arch["bigram_buckets"], arch["bigram_dim"]
        model["bigram"] = {
            "table": (rw.normal(0.0, 0.02, size=(nb, bd)) * bigram_scale).astype(np.float16),
            "proj": rw.normal(0.0, 0.02, size=(d, bd)).astype(np.float16),
        }
    return model


def zipf_tokens(n, vocab, s, rng):
    """Truncated Zipf over ``vocab`` ids: P(id = r-1) proportional to r^-s."""
    ranks = np.arange(1, vocab + 1, dtype=np.float64)
    p = ranks ** (-s)
    p /= p.sum()
    return rng.choice(vocab, size=n, p=p).astype(np.int32)


def make_stream(cfg, seed=1337, n_tokens=None):
    """(tokens int32[N], bytes int32[N]) for a workload; bytes[i] is the byte
    count of token i, uniform on 1..bytes_max."""
    _, rt, rb = _streams(seed)
    n = cfg["n_tokens"] if n_tokens is None else n_tokens
    tokens = zipf_tokens(n, cfg["arch"]["vocab"], cfg["zipf"], rt)
    nbytes = rb.integers(1, cfg["bytes_max"] + 1, size=n).astype(np.int32)
    return tokens, nbytes


def gemm_rows(arch):
    """Total number of quantised rows and weights in a model (for reporting)."""
    shapes = matrix_shapes(arch)
    rows = sum(s[0] for s in shapes.values()) * arch["n_unique"]
    weights = sum(s[0] * s[1] for s in shapes.values()) * arch["n_unique"]
    return rows, weights


def adversarial_rows(rng, cols):
    """Rows that stress the quantiser's edge cases (ties, zeros, one-hot,
    tiny magnitudes whose fp16 scale is subnormal or zero, huge outliers)."""
    rows = []
    rows.append(np.zeros(cols, np.float32))
    one = np.zeros(cols, np.float32)
    one[cols // 3] = 0.75
    rows.append(one)
    rows.append(-one)
    rows.append(np.full(cols, 0.0123, np.float32))
    alt = np.where(np.arange(cols) % 2 == 0, 1.0, -1.0).astype(np.float32)
    rows.append(alt)
    # exact half-way points of the first rounding: w = (k + 1/2) * scale
    hw = (np.arange(cols) % 9 - 4 + 0.5).astype(np.float32) * np.float32(127.0 / 4.5)
    rows.append(hw / np.float32(127.0))
    rows.append(rng.normal(0, 1e-7, cols).astype(np.float32))    # subnormal fp16 scale
    rows.append(rng.normal(0, 1e-12, cols).astype(np.float32))   # scale underflows fp16
    big = rng.normal(0, 0.02, cols).astype(np.float32)
    big[5] = 3.0
    big[cols - 7] = -2.5
    rows.append(big)
    rows.append(rng.standard_cauchy(cols).astype(np.float32) * np.float32(0.01))
    rows.append(rng.uniform(-1, 1, cols).astype(np.float32))
    return np.stack(rows)
