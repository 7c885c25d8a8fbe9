"""The algorithmic work the scoring pass reports per kernel class, which is
the numerator of every roofline fraction the bench prints, against closed
forms written here from the model shapes and the window plan.

Sliding windows as in pwwt.cn "parameter-golf 16MB 极限压缩实战 …", section
滑动窗口评估 (window k holds positions [kS, min(kS + L, P)) and scores
[max(kS, e_{k-1}), e_k)); block shapes from the same write-up's 架构 section
(GQA 8 / 4 heads of 64, ReLU^2 MLP 3x, tied 1024-token head).

Per row of a window and per layer: q/k/v 2 (d + 2 kvd) d, output projection
2 d^2, fc and proj 2 F d each; attention 4 hd Hq per causal (query, key)
pair; the head 2 V d per scored prediction.  Whatever kernels carry them
(the fused block tail also computes the next layer's q/k/v), the classes
together must add up to these counts exactly; with the final layer pruned,
its output projection, MLP and attention count only the scored rows and
the pairs of scored queries.  The full 11-layer stream is also checked
against the totals worked out by hand for it: 1738.3 TFLOP of GEMMs,
773.0 TFLOP of attention, 1.1 TFLOP of head.
"""
import numpy as np
import pytest

import synth
from oracle import windows as ow
from gpu_common import gpu_model, make_case, need_gpu, print_case

pytestmark = pytest.mark.gpu


def closed_form(arch, n_tokens, L, S, prune):
    """(GEMM, attention, head) FLOPs of one scoring pass."""
    d, F, V = arch["d_model"], arch["d_ff"], arch["vocab"]
    hd, Hq, Hkv = arch["head_dim"], arch["n_heads"], arch["n_kv_heads"]
    n_eff = arch["n_eff"]
    per_row_layer = 2 * (d + 2 * Hkv * hd) * d + 2 * d * d + 4 * F * d
    qkv_row = 2 * (d + 2 * Hkv * hd) * d
    gemm = attn = 0
    scored = 0
    for s, e, a in ow.plan_windows(n_tokens, L, S):
        T, j0, R = e - s, a - s, e - a
        scored += R
        pairs = T * (T + 1) // 2
        if prune:
            gemm += (n_eff - 1) * T * per_row_layer + T * qkv_row + R * (per_row_layer - qkv_row)
            attn += 4 * hd * Hq * ((n_eff - 1) * pairs + (pairs - j0 * (j0 + 1) // 2))
        else:
            gemm += n_eff * T * per_row_layer
            attn += 4 * hd * Hq * n_eff * pairs
    assert scored == n_tokens - 1
    return float(gemm), float(attn), float(2 * scored * V * d)


def measured(g, name, n_tokens, L, S, prune, fused_tail=True):
    import torch
    cfg, model = make_case(name)
    tokens, nbytes = synth.make_stream(cfg, seed=1337, n_tokens=n_tokens)
    print_case("accounting", name, "N", len(tokens), "L", L, "S", S, "prune", prune, "fused_tail", fused_tail)
    gm, _ = gpu_model(g, model)
    gm.set_prune_last(prune)
    gm.set_fused_tail(fused_tail)
    gm.set_timing(True)
    gm.score(torch.from_numpy(tokens).cuda(), torch.from_numpy(nbytes).cuda(), L, S)
    torch.cuda.synchronize()
    fl = {c: gm.timing(c)[2] for c in ("qkv", "attn", "oproj", "fc", "proj", "tail", "head", "lora")}
    gemm = fl["qkv"] + fl["oproj"] + fl["fc"] + fl["proj"] + fl["tail"]
    return cfg, len(tokens), gemm, fl["attn"], fl["head"], fl["lora"]


@pytest.mark.parametrize("name,N,L,S,prune,fused", [
    ("11l", 5000, 512, 64, False, True), ("11l", 5000, 512, 64, True, True),
    ("11l", 5000, 512, 64, True, False), ("11l", 700, 300, 7, True, True),
    ("largevocab", 3000, 256, 64, True, True), ("baseline", 2049, 1024, 1024, True, True),
])
def test_reported_flops_match_the_closed_form(name, N, L, S, prune, fused):
    g = need_gpu()
    cfg, n, gemm, attn, head, lora = measured(g, name, N, L, S, prune, fused)
    want = closed_form(cfg["arch"], n, L, S, prune)
    assert lora == 0.0
    np.testing.assert_allclose([gemm, attn, head], want, rtol=1e-12)


def test_full_11l_stream_matches_the_hand_worked_totals():
    """Unpruned, as the hand count has it; the counts printed to 0.1 TFLOP."""
    g = need_gpu()
    cfg, n, gemm, attn, head, _ = measured(g, "11l", None, 2048, 64, False)
    assert n == 1_048_576
    np.testing.assert_allclose([gemm, attn, head], closed_form(cfg["arch"], n, 2048, 64, False), rtol=1e-12)
    assert abs(gemm / 1e12 - 1738.3) < 0.05
    assert abs(attn / 1e12 - 773.0) < 0.05
    assert abs(head / 1e12 - 1.1) < 0.05
