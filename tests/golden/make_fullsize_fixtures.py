"""Write the oracle's per-prediction nats for the full-size workloads.

Calls only ``oracle/`` (and the seeded input generators in ``synth/``); the
HIP library is never imported.  For each workload the fixture holds the
oracle's float64 nats of a fixed set of windows, the predictions those
windows score, and the bits per byte over those predictions, so that the GPU
tests can compare a full-size pass against the oracle without running it.

* baseline, midcycle (chunked evaluation: 64 x 1024 and 32 x 2048): every
  window, i.e. every prediction of the stream;
* 11l, largevocab (sliding windows 2048 / stride 64 over 1,048,576 and
  4,194,304 tokens): 256 windows, the first and the last plus 254 drawn
  without replacement with ``numpy.random.default_rng(20240611)``.

Sliding-window plan and bits per byte as pwwt.cn "parameter-golf 16MB 极限压缩
实战 …", 滑动窗口评估, and the pigsec.cn openai/parameter-golf README mirror
(bits per byte) define them; model inputs as ``synth`` draws them at seed
1337.  Usage (from the repository root; about an hour on 8 cores):

    python tests/golden/make_fullsize_fixtures.py [name ...]
"""
from __future__ import annotations

import hashlib
import math
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import synth  # noqa: E402
from oracle import quant as oq, windows as ow  # noqa: E402

SEED = 1337
SAMPLE_SEED = 20240611
N_SAMPLE = 256
WORKLOADS = ("baseline", "midcycle", "11l", "largevocab")


def path(name):
    return os.path.join(HERE, f"fullsize_{name}.npz")


def stream_digest(tokens, nbytes):
    h = hashlib.sha256()
    h.update(np.ascontiguousarray(tokens, dtype=np.int32).tobytes())
    h.update(np.ascontiguousarray(nbytes, dtype=np.int32).tobytes())
    return h.hexdigest()


def windows_for(name, n_windows):
    if name in ("baseline", "midcycle"):
        return np.arange(n_windows, dtype=np.int64)
    rng = np.random.default_rng(SAMPLE_SEED)
    inner = rng.choice(np.arange(1, n_windows - 1), size=N_SAMPLE - 2, replace=False)
    return np.sort(np.concatenate([[0, n_windows - 1], inner])).astype(np.int64)


def make(name):
    cfg = synth.config(name)
    L, S = cfg["window"], cfg["stride"]
    model = synth.make_model(cfg["arch"], seed=SEED)
    tokens, nbytes = synth.make_stream(cfg, seed=SEED)
    qm = oq.quantize_model(model)
    plan = ow.plan_windows(len(tokens), L, S)
    which = windows_for(name, len(plan))
    t0 = time.time()
    nats = np.zeros(len(tokens) - 1)
    mask = np.zeros(len(tokens) - 1, dtype=bool)
    for i in range(0, len(which), 16):
        part, m = ow.score(qm, tokens, L, S, which=[int(k) for k in which[i:i + 16]])
        nats[m] = part[m]
        mask |= m
        print(f"[fixture] {name}: {min(i + 16, len(which))}/{len(which)} windows, "
              f"{time.time() - t0:.0f} s", flush=True)
    preds = np.nonzero(mask)[0].astype(np.int64)
    vals = nats[preds]
    total_bytes = int(nbytes[preds + 1].astype(np.int64).sum())
    bpb = float(vals.sum() / (math.log(2.0) * total_bytes))
    np.savez_compressed(path(name), name=name, seed=SEED, window=L, stride=S, n_tokens=len(tokens),
                        digest=stream_digest(tokens, nbytes), windows=which, preds=preds,
                        nats=vals, bpb=bpb, sum_nats=float(vals.sum()), sum_bytes=total_bytes)
    print(f"[fixture] {name}: {len(preds)} predictions, bpb {bpb:.8f}, wrote {path(name)}", flush=True)


if __name__ == "__main__":
    for n in (sys.argv[1:] or WORKLOADS):
        make(n)
