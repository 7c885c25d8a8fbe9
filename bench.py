"""Throughput of the int6 per-row scoring pass on one MI355X.

One step = the whole hot path over the 11-layer, d=512 int6 workload:
row-quantise all 66 block matrices (fp32 weights already in HBM, one
i6g_quantize_rows_many call), then score
the 1,048,576-token synthetic stream with sliding windows of 2048 / stride 64
(16,353 windows, 1,048,575 scored predictions) down to bits per byte.
Inputs are resident in HBM before the timed region starts.

Prints one JSON line with scored tokens/s, the roofline of the dominant
kernel (per-launch HIP-event durations of that kernel over the timed steps),
every kernel class's share from an instrumented warmup step, and the CPU
oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense 16-bit MFMA (binary16 and bfloat16)
PEAK_HBM_GBS = 8000.0
# kernel classes that are dense contractions on the MFMA roofline: the
# GEMMs (q/k/v projection; output projection, MLP up and down projections as
# three launches or as the fused block tail) and attention
GEMM_CLASSES = ("qkv", "oproj", "fc", "proj", "tail")
MFMA_CLASSES = GEMM_CLASSES + ("attn",)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--config", default="11l")
    ap.add_argument("--seed", type=int, default=1337)
    ap.add_argument("--batch-windows", type=int, default=0)
    ap.add_argument("--streams", type=int, default=0, help="1 or 2 streams for the batches (0 = default)")
    ap.add_argument("--cpu-windows", type=int, default=10,
                    help="full windows the CPU oracle scores for its baseline (0 = skip)")
    ap.add_argument("--no-timing", action="store_true", help="no per-launch events")
    ap.add_argument("--tokens", type=int, default=0,
                    help="score a shorter stream (counter runs only; 0 = the full workload)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (to scale the HBM byte counters)")
    ap.add_argument("--traffic", default=os.path.join(ROOT, "profiles", "hbm_traffic_11l.md"),
                    help="summary of the FETCH_SIZE / WRITE_SIZE counter runs (key: value lines)")
    return ap.parse_args()


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "the scoring pass runs on one GPU; --gpus must be 1",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)

    import numpy as np
    import torch
    import int6_row_gemm_amd as g
    import synth

    torch.cuda.set_device(0)
    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": 4 * n, "launches": 3}), flush=True)
        return
    cfg = synth.config(args.config)
    arch = cfg["arch"]
    L, S = cfg["window"], cfg["stride"]
    model = synth.make_model(arch, seed=args.seed)
    tokens_np, nbytes_np = synth.make_stream(cfg, seed=args.seed,
                                             n_tokens=args.tokens if args.tokens else None)
    N = len(tokens_np)
    P = N - 1

    # device-resident inputs
    w_dev = [{k: torch.from_numpy(v).cuda() for k, v in blk.items()} for blk in model["blocks"]]
    codes = [{k: torch.empty(v.shape, dtype=torch.int8, device="cuda") for k, v in blk.items()}
             for blk in w_dev]
    scales = [{k: torch.empty(v.shape[0], dtype=torch.int16, device="cuda") for k, v in blk.items()}
              for blk in w_dev]
    tokens = torch.from_numpy(tokens_np).cuda()
    nbytes = torch.from_numpy(nbytes_np).cuda()
    nats = torch.empty(P, dtype=torch.float32, device="cuda")
    totals = torch.empty(4, dtype=torch.float64, device="cuda")
    lib = g.lib()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    # every block matrix of the model in one i6g_quantize_rows_many call per
    # bit width (one launch per 80 matrices)
    by_bits = {}
    for wb, cb, sb in zip(w_dev, codes, scales):
        for k in wb:
            w = wb[k]
            by_bits.setdefault(g.matrix_bits(arch, k), []).append(
                g._QuantJob(w.data_ptr(), cb[k].data_ptr(), sb[k].data_ptr(), w.shape[0], w.shape[1]))
    job_arrays = {b: (g._QuantJob * len(js))(*js) for b, js in by_bits.items()}

    def quantize_all():
        for b, jobs in job_arrays.items():
            rc = lib.i6g_quantize_rows_many(ctypes.cast(jobs, ctypes.c_void_p), len(jobs), b,
                                            float(arch["clip_q"]), None, stream)
            if rc != 0:
                raise g.I6GError(rc, lib.i6g_last_error().decode())

    quantize_all()
    torch.cuda.synchronize()
    qblocks = [{k: (cb[k], sb[k]) for k in cb} for cb, sb in zip(codes, scales)]
    gm = g.load(model, qblocks)
    if args.batch_windows:
        gm.set_batch_windows(args.batch_windows)
    if args.streams:
        gm.set_streams(args.streams)

    def step():
        quantize_all()
        rc = lib.i6g_score_tokens(gm._h, ctypes.c_void_p(tokens.data_ptr()),
                                  ctypes.c_void_p(nbytes.data_ptr()), N, L, S,
                                  ctypes.c_void_p(nats.data_ptr()), ctypes.c_void_p(totals.data_ptr()),
                                  stream)
        if rc != 0:
            raise g.I6GError(rc, lib.i6g_last_error().decode())

    # Warmup.  The first warmup step records an event pair around every
    # launch to get the per-class breakdown and pick the dominant kernel.
    kernels = {}
    for i in range(max(args.warmup, 0 if args.no_timing else 1)):
        t0 = time.time()
        instrument = (i == 0 and not args.no_timing)
        if instrument:
            gm.set_timing(True)
        step()
        torch.cuda.synchronize()
        if instrument:
            for cls in g.KERNEL_CLASSES:
                ms, n, fl, by = gm.timing(cls)
                if n:
                    kernels[cls] = {"ms_total": ms, "launches": n, "avg_us": 1000.0 * ms / n,
                                    "tflops": fl / (ms * 1e9) if ms > 0 else None,
                                    "gbs": by / (ms * 1e6) if ms > 0 else None}
            gm.set_timing(False)
        print(f"[bench] warmup {i} {time.time() - t0:.2f}s", file=sys.stderr, flush=True)
    gm.status()
    dom = max(kernels, key=lambda c: kernels[c]["ms_total"]) if kernels else None

    # Timed steps: only the dominant kernel class carries HIP events (on the
    # library's stream), so its launch durations are measured live over the
    # timed region without instrumenting the other ~45,000 launches per step.
    if dom:
        gm.set_timing(True, [dom])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step()
        print(f"[bench] step {i} enqueued {time.perf_counter() - t0:.2f}s", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    gm.status()
    ms_per_step = 1000.0 * elapsed / args.steps
    value = P * args.steps / elapsed
    tot = totals.cpu().numpy()

    roofline = None
    gemm_frac = attn_frac = e2e_frac = head = None
    if dom:
        ms, n, fl, by = gm.timing(dom)
        gm.set_timing(False)
        avg_us = 1000.0 * ms / n
        # The dense contractions (the GEMM classes and attention) are priced
        # on the 16-bit MFMA roofline, 2.5 PFLOP/s dense (binary16 and
        # bfloat16 share it on MI355X); their algorithmic HBM bytes at 8 TB/s
        # are reported beside it.  Other kernels take whichever peak their
        # work needs longer on.
        if dom in MFMA_CLASSES or by / (PEAK_HBM_GBS * 1e9) < fl / (PEAK_BF16_TFLOPS * 1e12):
            ach, peak, unit, bound, per = fl / (ms * 1e9), PEAK_BF16_TFLOPS, "TFLOP/s", "mfma", fl / n
        else:
            ach, peak, unit, bound, per = by / (ms * 1e6), PEAK_HBM_GBS, "GB/s", "hbm", by / n
        # the committed counters were taken on the 11-layer workload with its
        # default batching and one stream; any other set-up reports none
        same_setup = args.config == "11l" and args.batch_windows in (0, 64) and args.streams in (0, 1)
        roofline = {"kernel": dom, "bound": bound, "achieved": ach, "peak": peak, "unit": unit,
                    "frac": ach / peak, "traffic": counter_traffic(args.traffic, dom) if same_setup else None,
                    "avg_launch_us": avg_us, "launches": n, "algorithmic_per_launch": per,
                    "algorithmic_flops_per_launch": fl / n, "algorithmic_bytes_per_launch": by / n,
                    "mfma_tflops": fl / (ms * 1e9),
                    "hbm": {"achieved_gbs": by / (ms * 1e6), "peak_gbs": PEAK_HBM_GBS,
                            "frac": by / (ms * 1e6) / PEAK_HBM_GBS}}
        gsum_ms = sum(kernels[c]["ms_total"] for c in GEMM_CLASSES if c in kernels)
        gsum_fl = sum(kernels[c]["tflops"] * kernels[c]["ms_total"] for c in GEMM_CLASSES if c in kernels)
        gemm_frac = (gsum_fl / gsum_ms) / PEAK_BF16_TFLOPS if gsum_ms else None
        # attention and the whole pass the same way: algorithmic FLOPs over
        # the kernel time of the instrumented warmup step, against the 16-bit
        # MFMA peak; and the head + cross-entropy kernel's HBM and FLOP rates
        if "attn" in kernels:
            attn_frac = kernels["attn"]["tflops"] / PEAK_BF16_TFLOPS
        all_ms = sum(v["ms_total"] for v in kernels.values())
        all_fl = sum((v["tflops"] or 0.0) * v["ms_total"] for v in kernels.values())
        e2e_frac = (all_fl / all_ms) / PEAK_BF16_TFLOPS if all_ms else None
        if "head" in kernels:
            hk = kernels["head"]
            head = {"avg_us": hk["avg_us"], "gbs": hk["gbs"], "tflops": hk["tflops"],
                    "frac_hbm": hk["gbs"] / PEAK_HBM_GBS, "frac_mfma": hk["tflops"] / PEAK_BF16_TFLOPS}

    # Stand-alone HBM-bound kernels are timed cold: before every repetition a
    # read of 512 MiB evicts their data from the 256 MB Infinity Cache (a
    # read, so that no dirty lines are written back inside the timed
    # kernel), and HIP events bracket the kernel alone; "warm_us" repeats it
    # back to back.
    flush = torch.ones(128 << 20, dtype=torch.float32, device="cuda") if not args.no_timing else None

    def timed(fn, reps=20):
        fn()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for e0, e1 in ev:
            flush.sum()
            e0.record()
            fn()
            e1.record()
        w0, w1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        w0.record()
        for _ in range(reps):
            fn()
        w1.record()
        torch.cuda.synchronize()
        cold = 1000.0 * sum(e0.elapsed_time(e1) for e0, e1 in ev) / reps
        return cold, 1000.0 * w0.elapsed_time(w1) / reps

    def hbm_entry(us, warm, by):
        return {"us": us, "warm_us": warm, "algorithmic_bytes": by, "gbs": by / (us * 1e3),
                "frac_hbm": by / (us * 1e3) / PEAK_HBM_GBS}

    # The quantiser on its own: all 66 matrices in one call; its algorithmic
    # bytes are 4 B read + 1 B written per weight + 2 B per row.
    quant = None
    if not args.no_timing:
        n_w = sum(w.numel() for wb in w_dev for w in wb.values())
        n_r = sum(w.shape[0] for wb in w_dev for w in wb.values())
        us, warm = timed(quantize_all, reps=100)
        quant = dict(matrices=sum(len(wb) for wb in w_dev), weights=n_w,
                     **hbm_entry(us, warm, 5.0 * n_w + 2.0 * n_r))
        quant["us_per_pass"] = us

    # The export side on the model's codes, each a kernel over the block
    # matrices of one bit width laid end to end: packing (1 B read + b/8 B
    # written per code), decoding the packed matrices to bfloat16 (b/8 B +
    # 2 B per code + 2 B per row; one launch per row length) and the code
    # histogram over every matrix (1 B per code).
    export = None
    if not args.no_timing:
        flat = torch.cat([cb[k].reshape(-1) for cb in codes for k in cb])
        hist = torch.empty(256, dtype=torch.int64, device="cuda")
        export = {"codes": flat.numel()}
        parts = {}
        keep = []
        for b in sorted({g.matrix_bits(arch, k) for k in codes[0]}):
            if b == 8:
                continue
            mats = [(cb[k], sb[k]) for cb, sb in zip(codes, scales) for k in cb if g.matrix_bits(arch, k) == b]
            fb = torch.cat([c.reshape(-1) for c, _ in mats])
            by_cols = {}
            for c, s_ in mats:
                by_cols.setdefault(c.shape[1], []).append((c, s_))
            stacks = [(torch.cat([c for c, _ in v]), torch.cat([s_ for _, s_ in v])) for v in by_cols.values()]
            stacks = [(g.pack_codes(c.reshape(-1), b), s_, c.shape[0], c.shape[1]) for c, s_ in stacks]
            pk = g.pack_codes(fb, b)
            outs = [torch.empty((r, c), dtype=torch.bfloat16, device="cuda") for _, _, r, c in stacks]
            keep += [fb, pk, stacks, outs]
            n_c, n_r = fb.numel(), sum(r for _, _, r, _ in stacks)

            def dq(stacks=stacks, outs=outs, b=b):
                for (p, s_, r, c), o in zip(stacks, outs):
                    rc = lib.i6g_dequantize_packed(ctypes.c_void_p(p.data_ptr()), b, ctypes.c_void_p(s_.data_ptr()),
                                                   r, c, g.DTYPE_BF16, ctypes.c_void_p(o.data_ptr()), stream)
                    if rc:
                        raise g.I6GError(rc, lib.i6g_last_error().decode())

            parts[f"pack_int{b}"] = (lambda fb=fb, pk=pk, b=b: g.pack_codes(fb, b, out=pk), (1 + b / 8) * n_c)
            parts[f"dequantize_packed_int{b}_bf16"] = (dq, (b / 8 + 2) * n_c + 2.0 * n_r)
        parts["code_histogram"] = (lambda: g.code_histogram(flat, hist), 1.0 * flat.numel())
        for name, (fn, by) in parts.items():
            export[name] = hbm_entry(*timed(fn), by)
        names = [k for k in codes[0]]
        export["artifact_bytes"] = g.artifact_bytes(
            [cb[k].shape for cb in codes for k in names],
            model["embed"].size + (model["skip_w"].size if model["skip_w"] is not None else 0),
            [g.matrix_bits(arch, k) for _ in codes for k in names])
        export["entropy_bits"] = g.code_entropy(g.code_histogram(flat, hist)).item()
        del flat, keep
    # Forward-only QAT weights on the model's 512-column matrices stacked
    # (q, k, v, o and fc of every block): fake quantisation and Noisy-QAT
    # noise, each 4 B read + 2 B written (bfloat16) per weight (the row is
    # read twice by the kernel, the second time mostly from cache).
    qat = None
    if not args.no_timing:
        w512 = torch.cat([w for wb in w_dev for w in wb.values() if w.shape[1] == arch["d_model"]])
        o16 = torch.empty(w512.shape, dtype=torch.bfloat16, device="cuda")
        n_w512 = w512.numel()

        def fq():
            rc = lib.i6g_fake_quantize_rows(ctypes.c_void_p(w512.data_ptr()), w512.shape[0], w512.shape[1],
                                            g.matrix_bits(arch, "fc"), 1.0, g.DTYPE_BF16,
                                            ctypes.c_void_p(o16.data_ptr()), None, stream)
            if rc:
                raise g.I6GError(rc, lib.i6g_last_error().decode())

        def nz():
            rc = lib.i6g_noisy_weights(ctypes.c_void_p(w512.data_ptr()), w512.shape[0], w512.shape[1], 127.0,
                                       1234, g.DTYPE_BF16, ctypes.c_void_p(o16.data_ptr()), None, stream)
            if rc:
                raise g.I6GError(rc, lib.i6g_last_error().decode())

        qat = {"weights": n_w512, "shape": list(w512.shape),
               "fake_quantize_bf16": hbm_entry(*timed(fq), 6.0 * n_w512),
               "noisy_weights_bf16": hbm_entry(*timed(nz), 6.0 * n_w512)}
        del w512, o16
    del flush

    cpu = None
    if args.cpu_windows > 0:
        cpu = cpu_baseline(model, tokens_np, L, S, args.cpu_windows)

    widths = sorted({g.matrix_bits(arch, k) for k in ("q", "fc")})
    bits_label = "/".join(f"int{b}" for b in widths)
    out = {
        # the MFMA share of the metric is reported as gemm_mfma_frac (the GEMMs'
        # FLOPs over their time, against the 16-bit dense MFMA peak) beside value
        "metric": "scored tokens/sec + % bf16 MFMA peak, 11L-512d int6 sliding-window bpb eval",
        "value": value,
        "unit": "scored tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic (seeded Zipf tokens, uniform byte counts, N(0,0.02) weights)",
        "config": {"workload": f"{args.config}: {arch['n_eff']} layers d={arch['d_model']} "
                               f"{bits_label} sliding window {L} stride {S} over {N} tokens",
                   "tokens": N, "scored": P, "window": L, "stride": S, "seed": args.seed,
                   "parallelism": "single GPU"},
        "bpb": float(tot[3]),
        "gemm_mfma_frac": gemm_frac,
        "attention_mfma_frac": attn_frac,
        "end_to_end_mfma_frac": e2e_frac,
        "head_ce": head,
        "roofline": roofline,
        "kernels_warmup_step": kernels,
        "quantize_rows": quant,
        "export": export,
        "qat": qat,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


# the sources each kernel class is compiled from (its file and the headers
# holding its device code); their hash ties a counter summary to the code
_HDRS = ("common.h", "mfma_util.h")
KERNEL_SOURCES = {"attn": ("attention.hip",) + _HDRS, "qkv": ("qkv.hip", "qkv_phase.h", "gemm.hip") + _HDRS,
                  "oproj": ("gemm.hip",) + _HDRS, "fc": ("gemm.hip",) + _HDRS, "proj": ("gemm.hip",) + _HDRS,
                  "tail": ("tail.hip", "qkv_phase.h") + _HDRS, "head": ("aux.hip",) + _HDRS,
                  "embed": ("aux.hip",) + _HDRS, "reduce": ("aux.hip",) + _HDRS}


def sources_sha256(kernel):
    """sha256 over the concatenated sources of a kernel class, or None."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES.get(kernel, ()):
        p = os.path.join(ROOT, "int6_row_gemm_amd", "csrc", f)
        if not os.path.exists(p):
            return None
        h.update(open(p, "rb").read())
    return h.hexdigest() if kernel in KERNEL_SOURCES else None


def counter_traffic(path, kernel):
    """HBM bytes per launch of `kernel` from the committed counter summary, or
    None when there is none or the kernel source changed since it was taken."""
    if not path or not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith(("#", "|", "`")):
            k, v = line.split(":", 1)
            kv[k.strip().lstrip("- ")] = v.strip().strip("`")
    if kv.get("kernel") != kernel or sources_sha256(kernel) != kv.get("source_sha256"):
        return None
    try:
        return float(kv["bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(model, tokens, L, S, n_windows):
    """The CPU oracle, as it stands, on full windows from the middle of the
    stream (each scores `stride` predictions); block quantisation is done once
    before timing (it is amortised over the whole stream)."""
    import numpy as np
    from oracle import quant as oq, windows as ow
    try:
        from threadpoolctl import threadpool_info
    except ImportError:
        threadpool_info = lambda: []  # noqa: E731
    qm = oq.quantize_model(model)
    plan = ow.plan_windows(len(tokens), L, S)
    mid = len(plan) // 2
    which = list(range(mid, mid + n_windows))
    t0 = time.perf_counter()
    nats, mask = ow.score(qm, tokens, L, S, which=which)
    dt = time.perf_counter() - t0
    scored = int(mask.sum())
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [os.cpu_count() or 1])
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": scored / dt, "unit": "scored tokens/s", "cores": threads, "kind": "oracle",
            "cpu": cpu_model, "nproc": os.cpu_count(),
            "sample": f"{n_windows} full windows ({scored} scored predictions) from the middle of the "
                      f"stream, float64 NumPy, {dt:.1f} s"}


if __name__ == "__main__":
    main()
