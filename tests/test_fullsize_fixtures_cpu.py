"""The stored full-size oracle results (tests/golden/fullsize_*.npz) on the
CPU: they belong to the streams synth draws today, their bits per byte is
their nats over their bytes, and the oracle reproduces the first and the
last stored windows.  The GPU parity test relies on these files."""
import hashlib
import math
import os

import numpy as np
import pytest

import synth
from oracle import quant as oq, windows as ow

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
NAMES = ["baseline", "midcycle", "11l", "largevocab"]


def _load(name):
    path = os.path.join(GOLDEN, f"fullsize_{name}.npz")
    if not os.path.exists(path):
        pytest.fail(f"{path} is missing: run tests/golden/make_fullsize_fixtures.py {name}")
    return np.load(path)


@pytest.mark.parametrize("name", NAMES)
def test_fixture_matches_stream_and_oracle(name):
    fx = _load(name)
    cfg = synth.config(name)
    L, S, seed = int(fx["window"]), int(fx["stride"]), int(fx["seed"])
    assert (L, S, int(fx["n_tokens"])) == (cfg["window"], cfg["stride"], cfg["n_tokens"])
    tokens, nbytes = synth.make_stream(cfg, seed=seed)
    h = hashlib.sha256()
    h.update(np.ascontiguousarray(tokens, dtype=np.int32).tobytes())
    h.update(np.ascontiguousarray(nbytes, dtype=np.int32).tobytes())
    assert h.hexdigest() == str(fx["digest"])
    preds, nats, windows = fx["preds"], fx["nats"], fx["windows"]
    plan = ow.plan_windows(len(tokens), L, S)
    # the stored predictions are exactly those the stored windows score
    want = np.concatenate([np.arange(plan[k][2], plan[k][1]) for k in windows])
    assert np.array_equal(np.sort(want), preds)
    assert windows[0] == 0 and windows[-1] == len(plan) - 1
    assert np.all(np.isfinite(nats)) and np.all(nats > 0)
    bpb = nats.sum() / (math.log(2.0) * nbytes[preds + 1].astype(np.int64).sum())
    assert abs(bpb - float(fx["bpb"])) < 1e-12
    # the oracle recomputes the first and the last stored windows
    qm = oq.quantize_model(synth.make_model(cfg["arch"], seed=seed))
    ref, mask = ow.score(qm, tokens, L, S, which=[int(windows[0]), int(windows[-1])])
    pos = np.searchsorted(preds, np.nonzero(mask)[0])
    np.testing.assert_allclose(nats[pos], ref[mask], rtol=1e-12, atol=0)
