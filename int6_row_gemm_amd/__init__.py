"""Python binding of ``libi6g.so``, the int6/int8 per-row scoring library.

Argument marshalling only: every step of the scoring pass runs in the HIP
kernels behind the C ABI declared in ``include/i6g.h``.  PyTorch provides
device memory and the current HIP stream.  There is no CPU fallback: if the
library has not been built, importing the functions below raises.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libi6g.so")

I6G_OK = 0
STATUS = {0: "I6G_OK", -1: "I6G_EINVAL", -2: "I6G_ENOMEM", -3: "I6G_EDEVICE",
          -4: "I6G_ENONFINITE", -5: "I6G_ETOKEN", -6: "I6G_EUNSUPPORTED", -7: "I6G_EBYTES"}
SKIP_KINDS = {"none": 0, "unet": 1, "stem_tail": 2}
KERNEL_CLASSES = ["embed", "qkv", "attn", "oproj", "fc", "proj", "head", "reduce", "lora", "tail"]

EXPORTED = [
    "i6g_quantize_rows", "i6g_quantize_rows_many", "i6g_weights_status", "i6g_load_model", "i6g_score_tokens", "i6g_model_status",
    "i6g_free_model", "i6g_last_error", "i6g_plan_windows", "i6g_set_option",
    "i6g_set_timing", "i6g_get_timing",
    "i6g_pack_codes", "i6g_unpack_codes", "i6g_dequantize_rows", "i6g_dequantize_packed",
    "i6g_code_histogram", "i6g_code_histogram_noalloc", "i6g_code_entropy", "i6g_artifact_bytes",
    "i6g_fake_quantize_rows", "i6g_noisy_weights",
]
DTYPE_F32, DTYPE_BF16 = 1, 2
FLAG_CODE = 8
ARTIFACT_LIMIT = 16_000_000


class I6GError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"{STATUS.get(code, code)}: {msg}")
        self.code = code


class _Matrix(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p)]


class _Block(ctypes.Structure):
    _fields_ = [(n, _Matrix) for n in ("q", "k", "v", "o", "fc", "proj")]


class _QuantJob(ctypes.Structure):
    _fields_ = [("w", ctypes.c_void_p), ("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("rows", ctypes.c_int64), ("cols", ctypes.c_int64)]


class _Desc(ctypes.Structure):
    _fields_ = [
        ("vocab", ctypes.c_int32), ("d_model", ctypes.c_int32), ("n_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("d_ff", ctypes.c_int32),
        ("rope_base", ctypes.c_double), ("norm_eps", ctypes.c_double),
        ("n_unique", ctypes.c_int32), ("n_eff", ctypes.c_int32),
        ("schedule", ctypes.c_void_p), ("blocks", ctypes.c_void_p),
        ("embed_dtype", ctypes.c_int32), ("embed", ctypes.c_void_p),
        ("skip_kind", ctypes.c_int32), ("n_skip", ctypes.c_int32), ("skip_weights", ctypes.c_void_p),
        ("parallel_residual", ctypes.c_int32), ("lora_rank", ctypes.c_int32),
        ("lora_aq", ctypes.c_void_p), ("lora_bq", ctypes.c_void_p),
        ("lora_av", ctypes.c_void_p), ("lora_bv", ctypes.c_void_p),
        ("bigram_buckets", ctypes.c_int32), ("bigram_dim", ctypes.c_int32),
        ("bigram_table", ctypes.c_void_p), ("bigram_proj", ctypes.c_void_p),
        ("logit_temperature", ctypes.c_double), ("leaky_slope", ctypes.c_double),
        ("rope_dims", ctypes.c_int32), ("xsa_last_n", ctypes.c_int32),
    ]


_lib = None


def lib():
    """The loaded C library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -c 'import __graft_entry__ as g; g.build()'`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, i32, dbl = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_double
        L.i6g_quantize_rows.argtypes = [vp, i64, i64, ctypes.c_int, dbl, vp, vp, vp, vp]
        L.i6g_quantize_rows_many.argtypes = [vp, i32, ctypes.c_int, dbl, vp, vp]
        L.i6g_weights_status.argtypes = [vp]
        L.i6g_load_model.argtypes = [vp, vp, ctypes.POINTER(vp)]
        L.i6g_score_tokens.argtypes = [vp, vp, vp, i64, i32, i32, vp, vp, vp]
        L.i6g_model_status.argtypes = [vp, vp]
        L.i6g_free_model.argtypes = [vp]
        L.i6g_free_model.restype = None
        L.i6g_last_error.restype = ctypes.c_char_p
        L.i6g_plan_windows.argtypes = [i64, i32, i32, vp, vp, vp, vp, i64]
        L.i6g_set_option.argtypes = [vp, ctypes.c_int, i64]
        L.i6g_set_timing.argtypes = [vp, ctypes.c_int, ctypes.c_uint32]
        L.i6g_get_timing.argtypes = [vp, ctypes.c_int, vp, vp, vp, vp]
        L.i6g_pack_codes.argtypes = [vp, i64, ctypes.c_int, vp, vp, vp]
        L.i6g_unpack_codes.argtypes = [vp, i64, ctypes.c_int, vp, vp]
        L.i6g_dequantize_rows.argtypes = [vp, vp, i64, i64, ctypes.c_int, vp, vp]
        L.i6g_dequantize_packed.argtypes = [vp, ctypes.c_int, vp, i64, i64, ctypes.c_int, vp, vp]
        L.i6g_code_histogram.argtypes = [vp, i64, ctypes.c_int, vp, vp]
        L.i6g_code_histogram_noalloc.argtypes = [vp, i64, ctypes.c_int, vp, vp]
        L.i6g_code_entropy.argtypes = [vp, vp, vp]
        L.i6g_artifact_bytes.argtypes = [vp, vp, i32, i64, vp]
        L.i6g_fake_quantize_rows.argtypes = [vp, i64, i64, ctypes.c_int, dbl, ctypes.c_int, vp, vp, vp]
        L.i6g_noisy_weights.argtypes = [vp, i64, i64, dbl, ctypes.c_uint64, ctypes.c_int, vp, vp, vp]
        _lib = L
    return _lib


def _check(rc):
    if rc != I6G_OK:
        raise I6GError(rc, lib().i6g_last_error().decode())


def _stream():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def plan_windows(n_tokens, window, stride):
    """Host-side window plan: arrays (starts, ends, score_from)."""
    n = ctypes.c_int64(0)
    _check(lib().i6g_plan_windows(n_tokens, window, stride, ctypes.byref(n), None, None, None, 0))
    K = n.value
    st, en, sf = (np.zeros(K, np.int64) for _ in range(3))
    _check(lib().i6g_plan_windows(n_tokens, window, stride, ctypes.byref(n),
                                  st.ctypes.data, en.ctypes.data, sf.ctypes.data, K))
    return st, en, sf


def weights_status():
    """Synchronise the current stream and raise I6GError (I6G_ENONFINITE)
    if a quantiser or QAT call made without a flag tensor met NaN / Inf."""
    _check(lib().i6g_weights_status(_stream()))


def quantize_rows(w, bits, clip_quantile, flags=None, check=True):
    """Row-quantise a device fp32 matrix.  Returns (codes int8, scales) where
    ``scales`` is an int16 tensor holding binary16 bit patterns
    (``scales.view(torch.float16)`` reads them).  Without a ``flags`` tensor
    a NaN / Inf row raises I6GError (I6G_ENONFINITE) after a stream
    synchronisation (``check=False`` leaves that to a later
    weights_status())."""
    import torch
    if not (w.is_cuda and w.dtype == torch.float32 and w.dim() == 2):
        raise ValueError("w must be a 2-D float32 CUDA tensor")
    w = w.contiguous()
    rows, cols = w.shape
    codes = torch.empty((rows, cols), dtype=torch.int8, device=w.device)
    scales = torch.empty((rows,), dtype=torch.int16, device=w.device)
    _check(lib().i6g_quantize_rows(_ptr(w), rows, cols, bits, float(clip_quantile),
                                   _ptr(codes), _ptr(scales), _ptr(flags), _stream()))
    if flags is None and check:
        weights_status()
    return codes, scales


def quantize_rows_many(jobs, bits, clip_quantile, flags=None):
    """Row-quantise several device fp32 matrices with one launch per 80.
    ``jobs`` is a list of (w, codes, scales) CUDA tensors (outputs written in
    place: codes int8 [rows, cols], scales int16 [rows] of binary16 bits)."""
    import torch
    arr = (_QuantJob * len(jobs))()
    for i, (w, codes, scales) in enumerate(jobs):
        if not (w.is_cuda and w.dtype == torch.float32 and w.dim() == 2 and w.is_contiguous()):
            raise ValueError("each w must be a contiguous 2-D float32 CUDA tensor")
        if codes.shape != w.shape or codes.dtype != torch.int8 or scales.shape != (w.shape[0],):
            raise ValueError("codes must be int8 like w and scales [rows]")
        arr[i] = _QuantJob(w.data_ptr(), codes.data_ptr(), scales.data_ptr(), w.shape[0], w.shape[1])
    _check(lib().i6g_quantize_rows_many(ctypes.cast(arr, ctypes.c_void_p), len(jobs), bits,
                                        float(clip_quantile), _ptr(flags), _stream()))


def _dev(x, dtype=None):
    import torch
    if isinstance(x, np.ndarray):
        t = torch.from_numpy(np.ascontiguousarray(x))
    else:
        t = x
    if dtype is not None:
        t = t.to(dtype)
    return t.to("cuda").contiguous()


def _f16_bits(x):
    import torch
    if isinstance(x, np.ndarray):
        x = np.ascontiguousarray(x.astype(np.float16)).view(np.int16)
        return _dev(x)
    return _dev(x.to(torch.float16).view(torch.int16))


class Model:
    """A model loaded into library-owned device memory.

    ``arch`` uses the keys of the synthetic configurations (vocab, d_model,
    n_heads, n_kv_heads, head_dim, d_ff, rope_base, norm_eps, schedule,
    skip_kind, n_skip, parallel, lora_rank, bigram_buckets, bigram_dim,
    embed_dtype, and the evaluation variants temperature, leaky_slope,
    rope_dims, xsa_last_n).  ``qblocks`` is a list of dicts name -> (codes, scales)
    for q, k, v, o, fc, proj (device or host tensors / arrays)."""

    def __init__(self, arch, qblocks, embed, skip_w=None, lora=None, bigram=None):
        import torch
        keep = []
        blocks = (_Block * len(qblocks))()
        for i, qb in enumerate(qblocks):
            for name in ("q", "k", "v", "o", "fc", "proj"):
                c, s = qb[name]
                c = _dev(c, torch.int8)
                s = _dev(s) if not isinstance(s, np.ndarray) else _dev(s.view(np.int16))
                keep += [c, s]
                setattr(blocks[i], name, _Matrix(c.data_ptr(), s.data_ptr()))
        sched = (ctypes.c_int32 * len(arch["schedule"]))(*arch["schedule"])
        f32 = arch.get("embed_dtype", "fp16") == "fp32"
        emb = _dev(embed, torch.float32) if f32 else _f16_bits(embed)
        keep.append(emb)
        d = _Desc()
        d.vocab, d.d_model = arch["vocab"], arch["d_model"]
        d.n_heads, d.n_kv_heads, d.head_dim = arch["n_heads"], arch["n_kv_heads"], arch["head_dim"]
        d.d_ff = arch["d_ff"]
        d.rope_base, d.norm_eps = float(arch["rope_base"]), float(arch["norm_eps"])
        d.n_unique, d.n_eff = len(qblocks), len(arch["schedule"])
        d.schedule = ctypes.cast(sched, ctypes.c_void_p)
        d.blocks = ctypes.cast(blocks, ctypes.c_void_p)
        d.embed_dtype = 1 if f32 else 0
        d.embed = emb.data_ptr()
        kind = arch.get("skip_kind", "none")
        d.skip_kind = SKIP_KINDS[kind] if isinstance(kind, str) else int(kind)
        d.n_skip = arch.get("n_skip", 0)
        if skip_w is not None and d.skip_kind != 0:
            sw = _f16_bits(skip_w); keep.append(sw); d.skip_weights = sw.data_ptr()
        d.parallel_residual = int(bool(arch.get("parallel", False)))
        d.lora_rank = arch.get("lora_rank", 0) if lora is not None else 0
        if d.lora_rank:
            for n in ("aq", "bq", "av", "bv"):
                t = _f16_bits(lora[n]); keep.append(t); setattr(d, "lora_" + n, t.data_ptr())
        if bigram is not None and arch.get("bigram_buckets", 0) > 0:
            d.bigram_buckets, d.bigram_dim = arch["bigram_buckets"], arch["bigram_dim"]
            t1, t2 = _f16_bits(bigram["table"]), _f16_bits(bigram["proj"])
            keep += [t1, t2]
            d.bigram_table, d.bigram_proj = t1.data_ptr(), t2.data_ptr()
        d.logit_temperature = float(arch.get("temperature", 1.0))
        d.leaky_slope = float(arch.get("leaky_slope", 0.0))
        d.rope_dims = int(arch.get("rope_dims") or 0)
        d.xsa_last_n = int(arch.get("xsa_last_n", 0))
        torch.cuda.synchronize()
        h = ctypes.c_void_p(0)
        _check(lib().i6g_load_model(ctypes.byref(d), _stream(), ctypes.byref(h)))
        torch.cuda.synchronize()
        self._h = h
        self.arch = dict(arch)

    def __del__(self):
        h = getattr(self, "_h", None)
        if h and h.value and _lib is not None:
            _lib.i6g_free_model(h)
            self._h = None

    def set_batch_windows(self, n):
        _check(lib().i6g_set_option(self._h, 0, n))

    def set_prune_last(self, on):
        _check(lib().i6g_set_option(self._h, 1, int(bool(on))))

    def set_streams(self, n):
        """1 (default): every batch on the caller's stream; 2: batches
        alternate with a second stream owned by the model."""
        _check(lib().i6g_set_option(self._h, 2, int(n)))

    def set_register_codes(self, on):
        """True (default): the fc and proj GEMMs load their codes,
        rearranged at load time, straight into registers; False: they stage
        the row-major codes through LDS."""
        _check(lib().i6g_set_option(self._h, 3, int(bool(on))))

    def set_fused_tail(self, on):
        """True (default): output projection, norm and MLP of each block as
        one kernel (d_model 512); False: three GEMM launches."""
        _check(lib().i6g_set_option(self._h, 4, int(bool(on))))

    def set_qkv_tile(self, on):
        """True (default): the q/k/v projection as one kernel per 128-row
        tile (d_model 512, head size 64, no LoRA), and with the fused block
        tail on, computed for the next layer inside each tail; False: the
        LDS-staged GEMM."""
        _check(lib().i6g_set_option(self._h, 5, int(bool(on))))

    def score(self, tokens, nbytes, window, stride, nats=None, totals=None, check=True):
        """Score a device token stream; returns (nats [N-1] fp32, totals [4] fp64)
        with totals = (sum nats, sum bytes, scored predictions, bits per byte)."""
        import torch
        tokens = _dev(tokens, torch.int32)
        nbytes = _dev(nbytes, torch.int32)
        n = tokens.numel()
        if nbytes.numel() != n:
            raise ValueError("tokens and byte counts differ in length")
        if nats is None:
            nats = torch.empty(max(n - 1, 0), dtype=torch.float32, device=tokens.device)
        if totals is None:
            totals = torch.empty(4, dtype=torch.float64, device=tokens.device)
        _check(lib().i6g_score_tokens(self._h, _ptr(tokens), _ptr(nbytes), n, window, stride,
                                      _ptr(nats), _ptr(totals), _stream()))
        if check:
            self.status()
        return nats, totals

    def status(self):
        """Synchronise and raise on a device-side error (bad token or bytes)."""
        _check(lib().i6g_model_status(self._h, _stream()))

    def set_timing(self, enable, classes=None):
        mask = 0
        for c in (classes or KERNEL_CLASSES):
            mask |= 1 << KERNEL_CLASSES.index(c)
        _check(lib().i6g_set_timing(self._h, int(enable), mask))

    def timing(self, cls):
        """(total_ms, launches, flops, bytes) for one kernel class."""
        ms, n = ctypes.c_double(), ctypes.c_int64()
        fl, by = ctypes.c_double(), ctypes.c_double()
        _check(lib().i6g_get_timing(self._h, KERNEL_CLASSES.index(cls), ctypes.byref(ms),
                                    ctypes.byref(n), ctypes.byref(fl), ctypes.byref(by)))
        return ms.value, n.value, fl.value, by.value


def matrix_bits(arch, name):
    """Bits of one block matrix: ``bits_attn`` for q, k, v, o and ``bits_mlp``
    for fc, proj when the arch gives them (mixed int5 / int6), else ``bits``."""
    key = "bits_attn" if name in ("q", "k", "v", "o") else "bits_mlp"
    return int(arch.get(key) or arch["bits"])


def quantize_model(model, flags=None):
    """Quantise every block matrix of a synthetic model on the GPU; returns
    a list of dicts name -> (codes, scales) of device tensors.  Without a
    ``flags`` tensor a NaN / Inf weight raises I6GError (I6G_ENONFINITE)."""
    import torch
    arch = model["arch"]
    out = []
    for blk in model["blocks"]:
        qb = {}
        for name, w in blk.items():
            wt = _dev(w, torch.float32)
            qb[name] = quantize_rows(wt, matrix_bits(arch, name), arch["clip_q"], flags, check=False)
        out.append(qb)
    if flags is None:
        weights_status()
    return out


def load(model, qblocks):
    """Load a synthetic model dict with the given quantised blocks."""
    return Model(model["arch"], qblocks, model["embed"], model.get("skip_w"),
                 model.get("lora"), model.get("bigram"))


# ---------------------------------------------------------------------------
# Export side: bit packing, dequantisation and code statistics.

def packed_size(n, bits=6):
    """Bytes of n packed codes: 3 per 4 int6 codes, 5 per 8 int5 codes (the
    last word padded)."""
    if bits == 6:
        return 3 * ((n + 3) // 4)
    if bits == 5:
        return 5 * ((n + 7) // 8)
    raise ValueError("bits must be 5 or 6")


def pack_codes(codes, bits=6, flags=None, out=None):
    """Pack a device int8 tensor of int6 or int5 codes (flattened) into a
    uint8 tensor of packed_size(numel, bits) bytes."""
    import torch
    if not (codes.is_cuda and codes.dtype == torch.int8 and codes.is_contiguous()):
        raise ValueError("codes must be a contiguous int8 CUDA tensor")
    n = codes.numel()
    size = packed_size(n, bits)
    if out is None:
        out = torch.empty(size, dtype=torch.uint8, device=codes.device)
    if out.numel() < size:
        raise ValueError("out is too small")
    _check(lib().i6g_pack_codes(_ptr(codes), n, bits, _ptr(out), _ptr(flags), _stream()))
    return out


def unpack_codes(packed, n, bits=6, out=None):
    """The first n codes held in a packed uint8 device tensor -> int8 [n]."""
    import torch
    if not (packed.is_cuda and packed.dtype == torch.uint8 and packed.is_contiguous()):
        raise ValueError("packed must be a contiguous uint8 CUDA tensor")
    if packed.numel() < packed_size(n, bits):
        raise ValueError("packed holds fewer than n codes")
    if out is None:
        out = torch.empty(n, dtype=torch.int8, device=packed.device)
    _check(lib().i6g_unpack_codes(_ptr(packed), n, bits, _ptr(out), _stream()))
    return out


def _dq_dtype(dtype):
    import torch
    if dtype == torch.float32:
        return DTYPE_F32
    if dtype == torch.bfloat16:
        return DTYPE_BF16
    raise ValueError("dtype must be torch.float32 or torch.bfloat16")


def dequantize(codes, scales, dtype=None):
    """code * scale per row of a device int8 [rows, cols] matrix with binary16
    row scales (int16 bit patterns or float16), as float32 or bfloat16."""
    import torch
    dtype = dtype or torch.float32
    if not (codes.is_cuda and codes.dtype == torch.int8 and codes.dim() == 2 and codes.is_contiguous()):
        raise ValueError("codes must be a contiguous 2-D int8 CUDA tensor")
    rows, cols = codes.shape
    if scales.numel() != rows or scales.element_size() != 2 or not scales.is_contiguous():
        raise ValueError("scales must hold one binary16 value per row")
    out = torch.empty((rows, cols), dtype=dtype, device=codes.device)
    _check(lib().i6g_dequantize_rows(_ptr(codes), _ptr(scales), rows, cols, _dq_dtype(dtype), _ptr(out),
                                     _stream()))
    return out


def dequantize_packed(packed, scales, rows, cols, dtype=None, bits=6):
    """dequantize() of a [rows, cols] int6 or int5 matrix given in packed form."""
    import torch
    dtype = dtype or torch.float32
    if not (packed.is_cuda and packed.dtype == torch.uint8 and packed.is_contiguous()):
        raise ValueError("packed must be a contiguous uint8 CUDA tensor")
    if packed.numel() < packed_size(rows * cols, bits):
        raise ValueError("packed holds fewer than rows * cols codes")
    if scales.numel() != rows or scales.element_size() != 2 or not scales.is_contiguous():
        raise ValueError("scales must hold one binary16 value per row")
    out = torch.empty((rows, cols), dtype=dtype, device=packed.device)
    _check(lib().i6g_dequantize_packed(_ptr(packed), bits, _ptr(scales), rows, cols, _dq_dtype(dtype),
                                       _ptr(out), _stream()))
    return out


def code_histogram(codes, hist=None, accumulate=False):
    """Counts of every int8 value of a device tensor: int64 [256], index v + 128."""
    import torch
    if not (codes.is_cuda and codes.dtype == torch.int8 and codes.is_contiguous()):
        raise ValueError("codes must be a contiguous int8 CUDA tensor")
    if hist is None:
        if accumulate:
            raise ValueError("accumulate needs an existing histogram")
        hist = torch.empty(256, dtype=torch.int64, device=codes.device)
    _check(lib().i6g_code_histogram(_ptr(codes), codes.numel(), int(bool(accumulate)), _ptr(hist),
                                    _stream()))
    return hist


def code_entropy(hist):
    """Entropy in bits per value of a device int64 [256] histogram, as a
    float64 device tensor of one element."""
    import torch
    if not (hist.is_cuda and hist.dtype == torch.int64 and hist.numel() == 256 and hist.is_contiguous()):
        raise ValueError("hist must be a contiguous int64 CUDA tensor of 256 counts")
    out = torch.empty(1, dtype=torch.float64, device=hist.device)
    _check(lib().i6g_code_entropy(_ptr(hist), _ptr(out), _stream()))
    return out


def artifact_bytes(shapes, passthrough_elements=0, bits=None):
    """Bytes of a packed artifact of matrices with the given (rows, cols)
    shapes and bit widths (default int6), each with binary16 row scales,
    plus binary16 passthrough values."""
    arr = np.ascontiguousarray(np.asarray(shapes, dtype=np.int64).reshape(-1, 2))
    b = None if bits is None else np.ascontiguousarray(np.asarray(bits, dtype=np.int32))
    if b is not None and len(b) != len(arr):
        raise ValueError("one bit width per matrix")
    out = ctypes.c_int64(0)
    _check(lib().i6g_artifact_bytes(arr.ctypes.data if len(arr) else None,
                                    b.ctypes.data if b is not None and len(b) else None, len(arr),
                                    int(passthrough_elements), ctypes.byref(out)))
    return out.value


def export_model(qblocks, arch, passthrough_elements=0):
    """Pack every block matrix of a quantised model at its bit width
    (matrix_bits) and measure its codes.  Returns a dict with ``packed``
    (list of dicts name -> (packed, scales, shape, bits)), ``hist`` (int64
    [256] over all codes), ``entropy_bits`` (device float64 [1]) and
    ``bytes`` (the artifact size)."""
    import torch
    packed, shapes, widths, hist, flags = [], [], [], None, None
    for qb in qblocks:
        pb = {}
        for name, (codes, scales) in qb.items():
            b = matrix_bits(arch, name)
            if flags is None:
                flags = torch.zeros(1, dtype=torch.int32, device=codes.device)
            if b == 8:
                pb[name] = (codes.reshape(-1).view(torch.uint8).clone(), scales, tuple(codes.shape), b)
            else:
                pb[name] = (pack_codes(codes, b, flags), scales, tuple(codes.shape), b)
            hist = code_histogram(codes, hist, accumulate=hist is not None)
            shapes.append(codes.shape)
            widths.append(b)
        packed.append(pb)
    if flags is not None and int(flags.item()) & FLAG_CODE:
        raise I6GError(-1, "a block matrix holds a code outside its format")
    return {"packed": packed, "hist": hist, "entropy_bits": code_entropy(hist),
            "bytes": artifact_bytes(shapes, passthrough_elements, widths)}


def import_model(packed):
    """Unpack the codes of export_model()'s ``packed`` list; returns the
    qblocks list (dicts name -> (codes, scales)) that load() takes."""
    import torch
    out = []
    for pb in packed:
        qb = {}
        for name, (p, scales, shape, b) in pb.items():
            n = shape[0] * shape[1]
            codes = p.view(torch.int8).clone() if b == 8 else unpack_codes(p, n, b)
            qb[name] = (codes.view(shape), scales)
        out.append(qb)
    return out


# ---------------------------------------------------------------------------
# Forward-only quantisation-aware weights.

def fake_quantize_rows(w, bits, clip_quantile=1.0, dtype=None, flags=None):
    """The straight-through forward value code * fp32 scale of each row of a
    device fp32 matrix, as float32 or bfloat16."""
    import torch
    dtype = dtype or torch.float32
    if not (w.is_cuda and w.dtype == torch.float32 and w.dim() == 2):
        raise ValueError("w must be a 2-D float32 CUDA tensor")
    w = w.contiguous()
    out = torch.empty(w.shape, dtype=dtype, device=w.device)
    _check(lib().i6g_fake_quantize_rows(_ptr(w), w.shape[0], w.shape[1], bits, float(clip_quantile),
                                        _dq_dtype(dtype), _ptr(out), _ptr(flags), _stream()))
    if flags is None:
        weights_status()
    return out


def noisy_weights(w, levels, seed, dtype=None, flags=None):
    """w + (U - 0.5) * amax / levels per row of a device fp32 matrix (U from
    Philox4x32-10 keyed by ``seed``), as float32 or bfloat16."""
    import torch
    dtype = dtype or torch.float32
    if not (w.is_cuda and w.dtype == torch.float32 and w.dim() == 2):
        raise ValueError("w must be a 2-D float32 CUDA tensor")
    w = w.contiguous()
    out = torch.empty(w.shape, dtype=dtype, device=w.device)
    _check(lib().i6g_noisy_weights(_ptr(w), w.shape[0], w.shape[1], float(levels), int(seed) & (2 ** 64 - 1),
                                   _dq_dtype(dtype), _ptr(out), _ptr(flags), _stream()))
    if flags is None:
        weights_status()
    return out
