"""Sliding-window evaluation plan and bits-per-byte.

Source: pwwt.cn "parameter-golf 16MB 极限压缩实战 …", section 滑动窗口评估：每
64 token 计一次分 (stride-64 windows of the evaluation length; only the
last ``stride`` positions of a window are scored; every token is evaluated
with up to a full window of context; the plain chunked eval cuts the stream
into independent chunks) and the pigsec.cn openai/parameter-golf README
mirror (the score is tokenizer-agnostic bits per byte).

Readings of the pages: window k starts at s_k = k*S and ends at
e_k = min(s_k + L, P) with P = N-1 predictions; it scores predictions
p in [max(s_k, e_{k-1}), e_k) (e_{-1} = 0) so window 0 scores all of its
positions, later full windows their last S, and every prediction is scored
exactly once; K = 1 + ceil((P-L)/S) windows (1 if P <= L).  Prediction p
predicts token p+1; bpb = sum_p nats_p / (ln 2 * sum_p bytes[p+1]).
The chunked eval is the case S = L.
"""
from __future__ import annotations

import math
import numpy as np

from .model import window_logits, log_softmax_nll, dense_weights


def plan_windows(n_tokens: int, L: int, S: int):
    """List of (s_k, e_k, a_k): inputs t[s_k:e_k], scored predictions
    p in [a_k, e_k)."""
    if n_tokens < 2 or L < 1 or S < 1 or S > L:
        raise ValueError("need n_tokens >= 2 and 1 <= stride <= window")
    P = n_tokens - 1
    K = 1 if P <= L else 1 + math.ceil((P - L) / S)
    out = []
    e_prev = 0
    for k in range(K):
        s = k * S
        e = min(s + L, P)
        a = max(s, e_prev)
        out.append((s, e, a))
        e_prev = e
    return out


def score(qmodel: dict, tokens: np.ndarray, L: int, S: int, which=None):
    """Per-prediction nats over a token stream.

    Returns ``(nats, mask)``: float64 [P] and bool [P] telling which
    predictions were computed (all of them unless ``which`` selects a subset
    of window indices)."""
    tokens = np.asarray(tokens, dtype=np.int64)
    P = len(tokens) - 1
    plan = plan_windows(len(tokens), L, S)
    nats = np.zeros(P, dtype=np.float64)
    mask = np.zeros(P, dtype=bool)
    dense = [dense_weights(qb) for qb in qmodel["qblocks"]]
    ks = range(len(plan)) if which is None else which
    for k in ks:
        s, e, a = plan[k]
        u = tokens[s:e]
        logits = window_logits(qmodel, u, dense)
        j0 = a - s
        tgt = tokens[a + 1:e + 1]
        nats[a:e] = log_softmax_nll(logits[j0:], tgt)
        mask[a:e] = True
    return nats, mask


def bpb(nats: np.ndarray, nbytes: np.ndarray) -> float:
    """Bits per byte: total nats / (ln 2 * total bytes of the target tokens);
    ``nbytes`` is the per-token byte count of the whole stream (length P+1)."""
    total_bytes = int(np.asarray(nbytes[1:len(nats) + 1], dtype=np.int64).sum())
    return float(np.sum(nats) / (math.log(2.0) * total_bytes))
