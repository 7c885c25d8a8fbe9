"""Transformer forward for one window, in float64 with dequantised weights.

Sources (page, section):
  * pwwt.cn "parameter-golf 16MB 极限压缩实战 …", section 架构：11 层 U-Net 变压器:
    GQA attention (8 query / 4 KV heads) with RoPE, ReLU^2 MLP
    ``proj(relu(fc(x))^2)``, tied input/output embedding, U-Net skips
    (num_encoder_layers = num_layers // 2; encoder outputs pushed on a stack,
    decoder layers pop in reverse order and add skip_weights[i] * skip).
  * kwkr.cn PR #363 write-up, section on the Middle-Cycle layout:
    [Stem] -> [Core x R] -> [Tail], stem outputs added with learned weights to
    tail inputs; DepthLoRA (low-rank Q/V adapter per virtual depth);
    BigramHash (adjacent-token hash into an embedding table, then projected).
  * pigsec.cn openai/parameter-golf README mirror, leaderboard entries:
    parallel attention/MLP residual lanes; layers 4-5 looped.

Evaluation variants from the PR #363 write-up (off by default): logits
divided by a temperature; LeakyReLU(slope)^2 in place of ReLU^2; RoPE on the
first R dims of each head; exclusive self attention on the last N effective
layers.

Readings of the pages: pre-norm RMSNorm without gain, eps 1e-6, and a
final norm before the tied head; attention scale 1/sqrt(head_dim), no other
logit transforms; query head h reads KV head floor(h*Hkv/Hq); RoPE on all
head dims with half-split pairs (i, i+hd/2), theta_i = base^(-2i/hd), at
window-relative positions; LoRA acts on the normed input, scale 1; the bigram
hash is (prev*1000003 + cur) mod buckets in exact integers, absent at window
position 0; U-Net decoder layers 0..n_enc-1 pop, the last gets none; tail
block j receives stem block (n_stem-1-j)'s output with weight j.
"""
from __future__ import annotations

import numpy as np

from .quant import dequantize

F64 = np.float64


def rms_norm(z: np.ndarray, eps: float) -> np.ndarray:
    """z / sqrt(mean(z^2) + eps) over the last axis (no gain)."""
    return z / np.sqrt(np.mean(z * z, axis=-1, keepdims=True) + eps)


def rope(x: np.ndarray, base: float, positions=None, dims=None) -> np.ndarray:
    """Rotary embedding of x [T, H, hd]: pairs (i, i + R/2) rotated by angle
    p * base^(-2i/R) at position p, for the first R = dims dims of each head
    (all of them when dims is None); the other hd - R dims pass unchanged
    (partial RoPE, kwkr.cn PR #363 write-up, "Partial RoPE 16/64")."""
    T, _, hd = x.shape
    R = hd if dims is None else int(dims)
    half = R // 2
    if positions is None:
        positions = np.arange(T, dtype=F64)
    theta = base ** (-2.0 * np.arange(half, dtype=F64) / R)
    ang = np.asarray(positions, dtype=F64)[:, None] * theta[None, :]
    cos = np.cos(ang)[:, None, :]
    sin = np.sin(ang)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:R]
    return np.concatenate([x1 * cos - x2 * sin, x1 * sin + x2 * cos, x[..., R:]], axis=-1)


def exclusive_self_attention(o: np.ndarray, v: np.ndarray) -> np.ndarray:
    """XSA (kwkr.cn PR #363 write-up, XSA paragraph): remove from each query
    head's attention output o_h[j] its component along the value vector of
    the same position, v_g[j] (g = the head's KV head); a zero value vector
    leaves o unchanged.  o [T, Hq, hd], v [T, Hkv, hd]."""
    T, Hq, hd = o.shape
    Hkv = v.shape[1]
    out = o.copy()
    for h in range(Hq):
        g = (h * Hkv) // Hq
        vv = v[:, g, :]
        nn = np.sum(vv * vv, axis=1)
        dot = np.sum(o[:, h, :] * vv, axis=1)
        coef = np.where(nn > 0, dot / np.where(nn > 0, nn, 1.0), 0.0)
        out[:, h, :] = o[:, h, :] - coef[:, None] * vv
    return out


def mlp_act(z: np.ndarray, slope: float) -> np.ndarray:
    """(leaky_relu(z, slope))^2; slope 0 is the ReLU^2 of [11L] 架构."""
    return np.square(np.where(z >= 0.0, z, slope * z))


def causal_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray) -> np.ndarray:
    """Softmax(q k^T / sqrt(hd) + causal mask) v per query head.

    q [T, Hq, hd], k and v [T, Hkv, hd]; query head h uses KV head
    floor(h * Hkv / Hq).  Returns [T, Hq, hd]."""
    T, Hq, hd = q.shape
    Hkv = k.shape[1]
    out = np.empty_like(q)
    allowed = np.tril(np.ones((T, T), dtype=bool))
    for h in range(Hq):
        g = (h * Hkv) // Hq
        s = (q[:, h, :] @ k[:, g, :].T) / np.sqrt(hd)
        s = np.where(allowed, s, -np.inf)
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=1, keepdims=True)
        out[:, h, :] = p @ v[:, g, :]
    return out


def dense_weights(qblock: dict) -> dict:
    """Dequantised float64 [out, in] matrices of one block."""
    return {name: dequantize(*cs) for name, cs in qblock.items()}


def block_forward(x, W, arch, lora=None, xsa=False):
    """One transformer block on x [T, d] (float64).

    ``W`` holds dequantised [out, in] matrices q, k, v, o, fc, proj.
    ``lora`` is None or (Aq [r,d], Bq [d,r], Av [r,kvd], Bv [kvd,r]) as float64.
    ``xsa`` applies exclusive self attention to this layer's attention output.
    """
    T, d = x.shape
    Hq, Hkv, hd = arch["n_heads"], arch["n_kv_heads"], arch["head_dim"]
    eps = arch["norm_eps"]
    a = rms_norm(x, eps)
    q = a @ W["q"].T
    k = a @ W["k"].T
    v = a @ W["v"].T
    if lora is not None:
        aq, bq, av, bv = lora
        q = q + (a @ aq.T) @ bq.T
        v = v + (a @ av.T) @ bv.T
    rd = arch.get("rope_dims")
    q = rope(q.reshape(T, Hq, hd), arch["rope_base"], dims=rd)
    k = rope(k.reshape(T, Hkv, hd), arch["rope_base"], dims=rd)
    v = v.reshape(T, Hkv, hd)
    o = causal_attention(q, k, v)
    if xsa:
        o = exclusive_self_attention(o, v)
    attn_out = o.reshape(T, Hq * hd) @ W["o"].T
    slope = arch.get("leaky_slope", 0.0)
    if arch["parallel"]:
        mlp_out = mlp_act(a @ W["fc"].T, slope) @ W["proj"].T
        return x + attn_out + mlp_out
    x = x + attn_out
    a2 = rms_norm(x, eps)
    return x + mlp_act(a2 @ W["fc"].T, slope) @ W["proj"].T


def skip_plan(arch):
    """(push_after[e], pop_before[e]) for every effective layer e.

    pop_before[e] is the skip-weight index to apply (or -1).  The stack is
    LIFO, so each pop takes the most recent unpopped push."""
    ne = arch["n_eff"]
    push = [False] * ne
    pop = [-1] * ne
    kind = arch["skip_kind"]
    if kind == "unet":
        n_enc = ne // 2
        for e in range(n_enc):
            push[e] = True
        for i in range(n_enc):            # decoder layers 0..n_enc-1
            pop[n_enc + i] = i
    elif kind == "stem_tail":
        n = arch["n_skip"]
        for e in range(n):
            push[e] = True
        for j in range(n):                # tail block j is effective layer ne-n+j
            pop[ne - n + j] = j
    return push, pop


def bigram_buckets(u: np.ndarray, n_buckets: int) -> np.ndarray:
    """h_j = (u[j-1] * 1000003 + u[j]) mod n_buckets for j >= 1 (exact ints)."""
    out = np.zeros(len(u), dtype=np.int64)
    for j in range(1, len(u)):
        out[j] = (int(u[j - 1]) * 1000003 + int(u[j])) % n_buckets
    return out


def window_logits(qmodel: dict, u: np.ndarray, dense=None) -> np.ndarray:
    """Logits [T, V] of the tied head for window inputs u[0..T-1]."""
    arch = qmodel["arch"]
    eps = arch["norm_eps"]
    E = qmodel["embed"].astype(F64)
    u = np.asarray(u, dtype=np.int64)
    x = E[u]
    if qmodel.get("bigram") is not None:
        tab = qmodel["bigram"]["table"].astype(F64)
        proj = qmodel["bigram"]["proj"].astype(F64)
        h = bigram_buckets(u, arch["bigram_buckets"])
        add = tab[h] @ proj.T
        add[0] = 0.0                                    # no previous token at position 0
        x = x + add
    if dense is None:
        dense = [dense_weights(qb) for qb in qmodel["qblocks"]]
    push, pop = skip_plan(arch)
    skip_w = None if qmodel.get("skip_w") is None else qmodel["skip_w"].astype(F64)
    stack = []
    lora = qmodel.get("lora")
    n_eff = len(arch["schedule"])
    xsa_from = n_eff - arch.get("xsa_last_n", 0)
    for e, b in enumerate(arch["schedule"]):
        if pop[e] >= 0:
            x = x + skip_w[pop[e]] * stack.pop()
        lo = None
        if lora is not None:
            lo = tuple(lora[n][e].astype(F64) for n in ("aq", "bq", "av", "bv"))
        x = block_forward(x, dense[b], arch, lo, xsa=e >= xsa_from)
        if push[e]:
            stack.append(x)
    z = rms_norm(x, eps)
    # evaluation temperature (kwkr.cn PR #363 write-up, EVAL_TEMPERATURE):
    # the logits the softmax sees are divided by T
    return (z @ E.T) / arch.get("temperature", 1.0)


def log_softmax_nll(logits: np.ndarray, targets: np.ndarray) -> np.ndarray:
    """nats_j = logsumexp(logits_j) - logits_j[target_j]."""
    m = logits.max(axis=1, keepdims=True)
    lse = m[:, 0] + np.log(np.exp(logits - m).sum(axis=1))
    return lse - logits[np.arange(len(targets)), targets]
