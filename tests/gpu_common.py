"""Shared set-up for the GPU parity tests: seeded synthetic models, the
oracle's results and the HIP path's results on the same inputs."""
import math
import os

import numpy as np
import pytest

import synth
from oracle import quant as oq, windows as ow

NATS_RTOL = 2e-3     # per-token nats, relative (the project's stated tolerance)
BPB_ATOL = 1e-4      # bits per byte, absolute


def need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import int6_row_gemm_amd as g
    g.lib()          # raises ImportError when the HIP library is missing
    return g


def make_case(name, seed=1337, model_kw=None, **overrides):
    cfg = synth.config(name, **overrides)
    model = synth.make_model(cfg["arch"], seed=seed, **(model_kw or {}))
    return cfg, model


def oracle_quantized(model):
    return oq.quantize_model(model)


def gpu_model(g, model):
    q = g.quantize_model(model)
    return g.load(model, q), q


def compare_nats(gpu_nats, ref_nats, mask=None, label=""):
    gpu_nats = np.asarray(gpu_nats, dtype=np.float64)
    if mask is not None:
        gpu_nats, ref_nats = gpu_nats[mask], ref_nats[mask]
    assert np.all(np.isfinite(gpu_nats)), label
    rel = np.abs(gpu_nats - ref_nats) / np.abs(ref_nats)
    worst = int(np.argmax(rel))
    assert rel.max() <= NATS_RTOL, (
        f"{label}: max rel err {rel.max():.3e} at {worst} (gpu {gpu_nats[worst]:.6f} "
        f"oracle {ref_nats[worst]:.6f}); mean rel {rel.mean():.2e}")
    return float(rel.max()), float(rel.mean())


def print_case(*parts):
    print("[case]", *parts, flush=True)
