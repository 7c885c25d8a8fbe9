// C ABI of the scoring library: argument validation, model loading, the
// block-schedule driver and the sliding-window batch loop.
//
// Block schedule (pwwt.cn "parameter-golf 16MB 极限压缩实战 …", 架构: U-Net
// skips -- encoder outputs pushed on a stack, decoder layers pop them in
// reverse and add skip_weights[i] * skip; kwkr.cn PR #363 write-up:
// Stem -> Core x R -> Tail with stem outputs added to tail inputs with
// learned weights; pigsec.cn README mirror: looped layers and parallel
// attention/MLP lanes): the host walks the effective layers, runs the unique
// block each one names, and fuses every push and pop into the epilogue of the
// GEMM that produces the layer's output.
#include "../../include/i6g.h"
#include "common.h"
#include <cmath>

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <climits>
#include <mutex>
#include <string>
#include <vector>

using namespace i6g;

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

#define HIP_TRY(expr)                                                                 \
  do {                                                                                \
    hipError_t e_ = (expr);                                                           \
    if (e_ != hipSuccess)                                                             \
      return fail(e_ == hipErrorOutOfMemory ? I6G_ENOMEM : I6G_EDEVICE, "%s: %s (%s)", \
                  #expr, hipGetErrorString(e_), __func__);                            \
  } while (0)

struct DevBuf {
  void* p = nullptr;
  size_t bytes = 0;
  ~DevBuf() { release(); }
  void release() {
    if (p) (void)hipFree(p);
    p = nullptr;
    bytes = 0;
  }
  hipError_t ensure(size_t n) {
    if (n <= bytes && p) return hipSuccess;
    release();
    hipError_t e = hipMalloc(&p, n ? n : 1);
    if (e == hipSuccess) bytes = n;
    else p = nullptr;
    return e;
  }
  template <class T> T* as() const { return reinterpret_cast<T*>(p); }
};

struct BlockDev {
  DevBuf qkv_codes, qkv_scales, o_codes, o_scales, fc_codes, fc_scales, proj_codes, proj_scales;
  // fc and proj codes in the fragment order of the register-fed GEMM path
  // (the output projection, K = d, stays LDS-staged there: its short K loop
  // does not repay the register-fed tile's longer residual epilogue); the
  // fused block tail reads o, fc and proj in fragment order (o and proj rows
  // with a zero scale as zero codes)
  DevBuf fc_frag, proj_frag, o_frag;
  // q/k/v codes in per-head fragment order for the one-tile q/k/v kernel
  // (d_model 512, head size 64, no LoRA; empty otherwise)
  DevBuf qkv_frag;
};

struct TimeRec {
  int cls;
  hipEvent_t a, b;
  double flops, bytes;
};

int64_t window_count(int64_t P, int64_t L, int64_t S) {
  return (P <= L) ? 1 : 1 + (P - L + S - 1) / S;
}

int64_t window_end(int64_t k, int64_t P, int64_t L, int64_t S) {
  return std::min(k * S + L, P);
}

// Library-owned non-finite latch, one copy per device: the quantiser and the
// forward-QAT kernels OR I6G_FLAG_NONFINITE into it when the caller passes
// no flag word of its own; i6g_weights_status() reports and clears it.  Host
// code uses the address hipGetSymbolAddress returns for the current device.
__device__ int32_t g_weight_latch;
constexpr int kMaxDevices = 64;
std::mutex g_latch_mu;
int32_t* g_latch_ptr[kMaxDevices] = {};

int latch_address(int32_t** out) {
  int dev = -1;
  HIP_TRY(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return fail(I6G_EDEVICE, "device %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_latch_mu);
  if (!g_latch_ptr[dev]) {
    void* p = nullptr;
    HIP_TRY(hipGetSymbolAddress(&p, HIP_SYMBOL(g_weight_latch)));
    g_latch_ptr[dev] = static_cast<int32_t*>(p);
  }
  *out = g_latch_ptr[dev];
  return I6G_OK;
}

// The caller's flag word, or the current device's latch when it passes none.
int flag_word(int32_t* flags_dev, int32_t** out) {
  if (flags_dev) {
    *out = flags_dev;
    return I6G_OK;
  }
  return latch_address(out);
}

// True when p is plain or pinned host memory (or the HIP runtime cannot
// tell, which means no device memory exists to be confused with): such
// tensors of a model descriptor are checked for NaN / Inf on the host before
// anything is allocated; device tensors are checked on the device after the
// copy.
bool host_readable(const void* p) {
  hipPointerAttribute_t at{};
  if (hipPointerGetAttributes(&at, p) != hipSuccess) {
    (void)hipGetLastError();
    return true;
  }
  return at.type == hipMemoryTypeHost || at.type == hipMemoryTypeUnregistered;
}

bool host_nonfinite_f16(const uint16_t* p, int64_t n) {
  if (!p || !host_readable(p)) return false;
  for (int64_t i = 0; i < n; ++i)
    if ((p[i] & 0x7c00u) == 0x7c00u) return true;
  return false;
}

bool host_nonfinite_f32(const float* p, int64_t n) {
  if (!p || !host_readable(p)) return false;
  for (int64_t i = 0; i < n; ++i)
    if (!std::isfinite(p[i])) return true;
  return false;
}

}  // namespace

struct i6g_model {
  // architecture
  int V, d, Hq, Hkv, hd, F, kvd, nqkv;
  double rope_base, eps;
  int n_unique, n_eff;
  std::vector<int> schedule, push_after, pop_before, pop_slot, push_slot;
  int max_depth = 0;
  int skip_kind, n_skip, parallel, lora_r, buckets, bigram_dim, embed_f32;
  // evaluation variants
  float inv_temp = 1.0f, leaky = 0.0f;
  int rope_dims = 0, xsa_last_n = 0;
  int device = 0;
  // weights
  std::vector<BlockDev> blocks;
  DevBuf embed, embed16, skip_w, lora_aq, lora_bq, lora_av, lora_bv, bigram;
  // tables and scratch
  DevBuf rope;
  int rope_L = 0;
  // per-batch scratch: a second set is allocated only when consecutive
  // batches of windows run on two streams at once (batches are independent)
  struct Scratch {
    DevBuf x, xb, ss, q, k, vt, o, h, slots, lora_u;
  } sc[2];
  DevBuf flags, part_n, part_b;
  int streams = 1;                 // 1: every batch on the caller's stream
  hipStream_t aux = nullptr;       // the second stream (default priority)
  hipEvent_t ev_fork = nullptr, ev_join = nullptr;
  int batch_windows = 0;
  int prune_last = 1;
  int register_codes = 1;
  int fused_tail = 1;
  int qkv_tile = 1;
  // timing
  bool timing = false;
  uint32_t timing_mask = 0;
  std::vector<hipEvent_t> pool;
  std::vector<TimeRec> recs;
  hipStream_t timed_stream = nullptr;
  double t_ms[I6G_K_COUNT] = {}, t_flops[I6G_K_COUNT] = {}, t_bytes[I6G_K_COUNT] = {};
  int64_t t_n[I6G_K_COUNT] = {};

  hipEvent_t take_event() {
    if (!pool.empty()) {
      hipEvent_t e = pool.back();
      pool.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
  ~i6g_model() {
    for (auto& r : recs) { pool.push_back(r.a); pool.push_back(r.b); }
    for (auto e : pool) (void)hipEventDestroy(e);
    if (aux) {
      (void)hipStreamSynchronize(aux);
      (void)hipStreamDestroy(aux);
    }
    if (ev_fork) (void)hipEventDestroy(ev_fork);
    if (ev_join) (void)hipEventDestroy(ev_join);
  }
};

namespace {

// Wrap a launch with an event pair when timing is on for its class.
template <class F>
int timed(i6g_model* m, int cls, hipStream_t s, double flops, double bytes, F&& launch) {
  hipEvent_t a = nullptr, b = nullptr;
  const bool on = m->timing && (m->timing_mask >> cls & 1u);
  if (on) {
    a = m->take_event();
    b = m->take_event();
    if (!a || !b) return fail(I6G_EDEVICE, "hipEventCreate failed");
    HIP_TRY(hipEventRecord(a, s));
  }
  hipError_t e = launch();
  if (e != hipSuccess) return fail(I6G_EDEVICE, "kernel launch (class %d): %s", cls, hipGetErrorString(e));
  if (on) {
    HIP_TRY(hipEventRecord(b, s));
    m->recs.push_back(TimeRec{cls, a, b, flops, bytes});
    m->timed_stream = s;
  }
  return I6G_OK;
}

int copy_in(DevBuf& dst, const void* src, size_t bytes, hipStream_t s) {
  HIP_TRY(dst.ensure(bytes));
  HIP_TRY(hipMemcpyAsync(dst.p, src, bytes, hipMemcpyDefault, s));
  return I6G_OK;
}

int build_plan(i6g_model* m) {
  const int ne = m->n_eff;
  m->push_after.assign(ne, 0);
  m->pop_before.assign(ne, -1);
  if (m->skip_kind == I6G_SKIP_UNET) {
    const int n_enc = ne / 2;
    if (m->n_skip != n_enc)
      return fail(I6G_EINVAL, "U-Net with %d effective layers needs %d skip weights, got %d", ne, n_enc,
                  m->n_skip);
    for (int e = 0; e < n_enc; ++e) m->push_after[e] = 1;
    for (int i = 0; i < n_enc; ++i) m->pop_before[n_enc + i] = i;
  } else if (m->skip_kind == I6G_SKIP_STEM_TAIL) {
    const int n = m->n_skip;
    if (n < 1 || 2 * n > ne) return fail(I6G_EINVAL, "stem/tail skips: n_skip=%d with n_eff=%d", n, ne);
    for (int e = 0; e < n; ++e) m->push_after[e] = 1;
    for (int j = 0; j < n; ++j) m->pop_before[ne - n + j] = j;
  } else if (m->skip_kind != I6G_SKIP_NONE) {
    return fail(I6G_EINVAL, "unknown skip_kind %d", m->skip_kind);
  }
  // Resolve the LIFO stack into slot indices.
  m->push_slot.assign(ne, -1);
  m->pop_slot.assign(ne, -1);
  int depth = 0;
  m->max_depth = 0;
  for (int e = 0; e < ne; ++e) {
    if (m->pop_before[e] >= 0) {
      if (depth == 0) return fail(I6G_EINVAL, "skip pop before layer %d with an empty stack", e);
      m->pop_slot[e] = --depth;
    }
    if (m->push_after[e]) {
      m->push_slot[e] = depth++;
      m->max_depth = std::max(m->max_depth, depth);
    }
  }
  if (m->pop_before[0] >= 0) return fail(I6G_EINVAL, "pop before the first layer");
  return I6G_OK;
}

// Scratch for batches of W windows of Lp rows: the second set only when
// batches alternate over two streams, and the hidden activations only when
// the MLP runs as two GEMMs (the fused block tail keeps them on the chip).
// Buffers only grow; hipFree of a smaller one waits for the device first.
int ensure_scratch(i6g_model* m, int W, int Lp, hipStream_t s, int n_sets, bool need_h) {
  const int64_t M = (int64_t)W * Lp;
  const int nt = m->d / 128;
  for (int i = 0; i < n_sets; ++i) {
    auto& c = m->sc[i];
    HIP_TRY(c.x.ensure(M * m->d * 4));
    HIP_TRY(c.xb.ensure(M * m->d * 2));
    HIP_TRY(c.ss.ensure(M * nt * 4));
    HIP_TRY(c.q.ensure(M * m->d * 2));
    HIP_TRY(c.k.ensure(M * m->kvd * 2));
    HIP_TRY(c.vt.ensure(M * m->kvd * 2));
    HIP_TRY(c.o.ensure(M * m->d * 2));
    if (need_h) HIP_TRY(c.h.ensure(M * m->F * 2));
    if (m->max_depth > 0) HIP_TRY(c.slots.ensure((size_t)m->max_depth * M * m->d * 4));
    if (m->lora_r > 0) HIP_TRY(c.lora_u.ensure(M * 2 * m->lora_r * 4));
  }
  if (!m->aux) {
    HIP_TRY(hipStreamCreateWithFlags(&m->aux, hipStreamNonBlocking));
    HIP_TRY(hipEventCreateWithFlags(&m->ev_fork, hipEventDisableTiming));
    HIP_TRY(hipEventCreateWithFlags(&m->ev_join, hipEventDisableTiming));
  }
  if (Lp > m->rope_L) {
    HIP_TRY(m->rope.ensure((size_t)Lp * (m->hd / 2) * sizeof(float2)));
    HIP_TRY(launch_rope_table(m->rope.as<float2>(), Lp, m->hd, m->rope_dims, m->rope_base, s));
    m->rope_L = Lp;
  }
  return I6G_OK;
}

}  // namespace

extern "C" {

const char* i6g_last_error(void) { return g_err.c_str(); }

int i6g_plan_windows(int64_t n_tokens, int32_t window, int32_t stride, int64_t* n_windows,
                     int64_t* starts, int64_t* ends, int64_t* score_from, int64_t capacity) {
  if (n_tokens < 2 || window < 1 || stride < 1 || stride > window || !n_windows)
    return fail(I6G_EINVAL, "plan_windows: need n_tokens >= 2, 1 <= stride <= window");
  const int64_t P = n_tokens - 1;
  const int64_t K = window_count(P, window, stride);
  *n_windows = K;
  int64_t e_prev = 0;
  for (int64_t k = 0; k < K && k < capacity; ++k) {
    const int64_t s = k * stride, e = window_end(k, P, window, stride);
    if (starts) starts[k] = s;
    if (ends) ends[k] = e;
    if (score_from) score_from[k] = std::max(s, e_prev);
    e_prev = e;
  }
  return I6G_OK;
}

// Validation and the host-side quantile split shared by both quantiser
// entry points: pos = q * (cols - 1) in binary64, lo = floor(pos), the
// kernel keeps the cols - lo largest |w| and interpolates with f = pos - lo.
static bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

static int quant_plan(const char* who, int job, const void* w, const void* codes, const void* scales,
                      int64_t rows, int64_t cols, int bits, double clip_quantile, int32_t* topk,
                      float* frac) {
  // the caller's name (and job number), formatted only for an error
  char name[64];
  auto id = [&]() -> const char* {
    if (job < 0) return who;
    snprintf(name, sizeof name, "%s job %d", who, job);
    return name;
  };
  if (!w || !codes || !scales) return fail(I6G_EINVAL, "%s: NULL array", id());
  if (rows < 1 || cols < 1) return fail(I6G_EINVAL, "%s: rows and cols must be >= 1", id());
  if (bits != 5 && bits != 6 && bits != 8) return fail(I6G_EINVAL, "%s: bits must be 5, 6 or 8", id());
  if (!(clip_quantile > 0.0 && clip_quantile <= 1.0))
    return fail(I6G_EINVAL, "%s: clip_quantile must be in (0, 1]", id());
  if (cols > 65536) return fail(I6G_EUNSUPPORTED, "%s: cols > 65536", id());
  const double pos = clip_quantile * (double)(cols - 1);
  const int64_t lo = (int64_t)floor(pos);
  if (cols - lo > 8)
    return fail(I6G_EUNSUPPORTED, "%s: quantile needs the %lld largest values (max 8)", id(),
                (long long)(cols - lo));
  *topk = (int32_t)(cols - lo);
  *frac = (float)(pos - (double)lo);
  return I6G_OK;
}

int i6g_quantize_rows(const float* w_dev, int64_t rows, int64_t cols, int bits, double clip_quantile,
                      int8_t* codes_dev, uint16_t* scales_dev, int32_t* flags_dev, void* stream) {
  int32_t topk = 0;
  float frac = 0.0f;
  int rc = quant_plan("quantize_rows", -1, w_dev, codes_dev, scales_dev, rows, cols, bits, clip_quantile,
                      &topk, &frac);
  if (rc) return rc;
  int32_t* flags = nullptr;
  if ((rc = flag_word(flags_dev, &flags))) return rc;
  QuantArgs a{};
  a.w = w_dev;
  a.codes = codes_dev;
  a.scales = scales_dev;
  a.flags = flags;
  a.rows = rows;
  a.cols = (int32_t)cols;
  a.bits = bits;
  a.topk = topk;
  a.frac = frac;
  a.shape = quant_unit_shape(cols, cols % 4 == 0 && aligned(w_dev, 16) && aligned(codes_dev, 4), topk);
  HIP_TRY(launch_quantize(a, (hipStream_t)stream));
  return I6G_OK;
}

int i6g_quantize_rows_many(const i6g_quant_job* jobs, int32_t n_jobs, int bits, double clip_quantile,
                           int32_t* flags_dev, void* stream) {
  if (!jobs || n_jobs < 1) return fail(I6G_EINVAL, "quantize_rows_many: need n_jobs >= 1 jobs");
  std::vector<QuantJob> plan(n_jobs);
  std::vector<int64_t> units(n_jobs);
  for (int j = 0; j < n_jobs; ++j) {
    const i6g_quant_job& J = jobs[j];
    int32_t topk = 0;
    float frac = 0.0f;
    int rc = quant_plan("quantize_rows_many", j, J.w, J.codes, J.scales, J.rows, J.cols, bits, clip_quantile, &topk, &frac);
    if (rc) return rc;
    plan[j].w = J.w; plan[j].codes = J.codes; plan[j].scales = J.scales;
    plan[j].cols = (int32_t)J.cols;
    plan[j].topk = (int16_t)topk;
    plan[j].frac = frac;
    const bool vec = J.cols % 4 == 0 && aligned(J.w, 16) && aligned(J.codes, 4);
    const int shape = quant_unit_shape(J.cols, vec, topk);
    const int per = quant_unit_rows(shape);
    plan[j].shape = (uint8_t)shape;
    plan[j].last = (uint8_t)(J.rows - (J.rows - 1) / per * per);
    units[j] = (J.rows + per - 1) / per;
  }
  int32_t* flags = nullptr;
  if (int rc = flag_word(flags_dev, &flags)) return rc;
  for (int j0 = 0; j0 < n_jobs; j0 += kQuantJobs) {
    QuantManyArgs a{};
    a.n = std::min(kQuantJobs, n_jobs - j0);
    a.bits = bits;
    a.flags = flags;
    a.unit0[0] = 0;
    for (int j = 0; j < a.n; ++j) {
      a.job[j] = plan[j0 + j];
      a.unit0[j + 1] = a.unit0[j] + units[j0 + j];
    }
    HIP_TRY(launch_quantize_many(a, (hipStream_t)stream));
  }
  return I6G_OK;
}

int i6g_fake_quantize_rows(const float* w_dev, int64_t rows, int64_t cols, int bits, double clip_quantile,
                           int out_dtype, void* out_dev, int32_t* flags_dev, void* stream) {
  int32_t topk = 0;
  float frac = 0.0f;
  int rc = quant_plan("fake_quantize_rows", -1, w_dev, out_dev, out_dev, rows, cols, bits, clip_quantile, &topk,
                      &frac);
  if (rc) return rc;
  if (out_dtype != I6G_DTYPE_F32 && out_dtype != I6G_DTYPE_BF16)
    return fail(I6G_EINVAL, "fake_quantize_rows: out_dtype must be I6G_DTYPE_F32 or I6G_DTYPE_BF16");
  int32_t* flags = nullptr;
  if ((rc = flag_word(flags_dev, &flags))) return rc;
  QuantArgs a{};
  a.w = w_dev;
  a.flags = flags;
  a.rows = rows;
  a.cols = (int32_t)cols;
  a.bits = bits;
  a.topk = topk;
  a.frac = frac;
  a.fq = out_dev;
  a.fq_bf16 = out_dtype == I6G_DTYPE_BF16;
  a.shape = quant_unit_shape(cols, cols % 4 == 0 && aligned(w_dev, 16) && aligned(out_dev, a.fq_bf16 ? 8 : 16),
                             topk);
  HIP_TRY(launch_fake_quantize(a, (hipStream_t)stream));
  return I6G_OK;
}

int i6g_noisy_weights(const float* w_dev, int64_t rows, int64_t cols, double levels, uint64_t seed, int out_dtype,
                      void* out_dev, int32_t* flags_dev, void* stream) {
  if (!w_dev || !out_dev) return fail(I6G_EINVAL, "noisy_weights: NULL array");
  if (rows < 1 || cols < 1 || cols > INT32_MAX) return fail(I6G_EINVAL, "noisy_weights: need rows, cols >= 1");
  if (!(levels > 0.0) || !std::isfinite(levels) || !std::isfinite((float)levels))
    return fail(I6G_EINVAL, "noisy_weights: levels must be positive and finite");
  if (out_dtype != I6G_DTYPE_F32 && out_dtype != I6G_DTYPE_BF16)
    return fail(I6G_EINVAL, "noisy_weights: out_dtype must be I6G_DTYPE_F32 or I6G_DTYPE_BF16");
  if (!aligned(w_dev, 16) || !aligned(out_dev, 16))
    return fail(I6G_EUNSUPPORTED, "noisy_weights: w and out must be 16-byte aligned");
  int32_t* flags = nullptr;
  if (int rc = flag_word(flags_dev, &flags)) return rc;
  NoisyArgs a{};
  a.w = w_dev;
  a.out = out_dev;
  a.flags = flags;
  a.rows = rows;
  a.cols = (int32_t)cols;
  a.out_bf16 = out_dtype == I6G_DTYPE_BF16;
  a.levels = (float)levels;
  a.key0 = (uint32_t)seed;
  a.key1 = (uint32_t)(seed >> 32);
  HIP_TRY(launch_noisy_weights(a, (hipStream_t)stream));
  return I6G_OK;
}

int i6g_weights_status(void* stream) {
  int32_t* latch = nullptr;
  if (int rc = latch_address(&latch)) return rc;
  HIP_TRY(hipStreamSynchronize((hipStream_t)stream));
  int32_t f = 0;
  HIP_TRY(hipMemcpy(&f, latch, 4, hipMemcpyDeviceToHost));
  if (f) HIP_TRY(hipMemset(latch, 0, 4));
  if (f & I6G_FLAG_NONFINITE) return fail(I6G_ENONFINITE, "a weight row held NaN or Inf");
  return I6G_OK;
}

static int64_t packed_bytes(int64_t n, int bits) {
  return bits == 6 ? 3 * ((n + 3) / 4) : bits == 5 ? 5 * ((n + 7) / 8) : n;
}

int i6g_pack_codes(const int8_t* codes_dev, int64_t n, int bits, uint8_t* packed_dev, int32_t* flags_dev,
                   void* stream) {
  if (bits != 5 && bits != 6) return fail(I6G_EINVAL, "pack_codes: bits must be 5 or 6");
  if (n < 0 || (n > 0 && (!codes_dev || !packed_dev))) return fail(I6G_EINVAL, "pack_codes: n < 0 or NULL buffer");
  if (n == 0) return I6G_OK;
  if (!aligned(codes_dev, 16) || !aligned(packed_dev, 4))
    return fail(I6G_EUNSUPPORTED, "pack_codes: codes must be 16-byte and packed 4-byte aligned");
  HIP_TRY(launch_pack_codes(codes_dev, n, bits, packed_dev, flags_dev, (hipStream_t)stream));
  return I6G_OK;
}

int i6g_unpack_codes(const uint8_t* packed_dev, int64_t n, int bits, int8_t* codes_dev, void* stream) {
  if (bits != 5 && bits != 6) return fail(I6G_EINVAL, "unpack_codes: bits must be 5 or 6");
  if (n < 0 || (n > 0 && (!codes_dev || !packed_dev))) return fail(I6G_EINVAL, "unpack_codes: n < 0 or NULL buffer");
  if (n == 0) return I6G_OK;
  if (!aligned(codes_dev, 16) || !aligned(packed_dev, 4))
    return fail(I6G_EUNSUPPORTED, "unpack_codes: codes must be 16-byte and packed 4-byte aligned");
  HIP_TRY(launch_unpack_codes(packed_dev, n, bits, codes_dev, (hipStream_t)stream));
  return I6G_OK;
}

static int dequant(const char* who, const void* src, int bits, const uint16_t* scales_dev, int64_t rows,
                   int64_t cols, int out_dtype, void* out_dev, void* stream) {
  if (rows < 0 || cols < 0) return fail(I6G_EINVAL, "%s: rows and cols must be >= 0", who);
  if (out_dtype != I6G_DTYPE_F32 && out_dtype != I6G_DTYPE_BF16)
    return fail(I6G_EINVAL, "%s: out_dtype must be I6G_DTYPE_F32 or I6G_DTYPE_BF16", who);
  if (rows == 0 || cols == 0) return I6G_OK;
  if (!src || !scales_dev || !out_dev) return fail(I6G_EINVAL, "%s: NULL buffer", who);
  if (!aligned(src, bits == 8 ? 16 : 4) || !aligned(out_dev, 16) || !aligned(scales_dev, 2))
    return fail(I6G_EUNSUPPORTED, "%s: misaligned buffer", who);
  HIP_TRY(launch_dequantize(src, bits, scales_dev, rows, cols, out_dtype == I6G_DTYPE_BF16, out_dev,
                            (hipStream_t)stream));
  return I6G_OK;
}

int i6g_dequantize_rows(const int8_t* codes_dev, const uint16_t* scales_dev, int64_t rows, int64_t cols,
                        int out_dtype, void* out_dev, void* stream) {
  return dequant("dequantize_rows", codes_dev, 8, scales_dev, rows, cols, out_dtype, out_dev, stream);
}

int i6g_dequantize_packed(const uint8_t* packed_dev, int bits, const uint16_t* scales_dev, int64_t rows,
                          int64_t cols, int out_dtype, void* out_dev, void* stream) {
  if (bits != 5 && bits != 6) return fail(I6G_EINVAL, "dequantize_packed: bits must be 5 or 6");
  return dequant("dequantize_packed", packed_dev, bits, scales_dev, rows, cols, out_dtype, out_dev, stream);
}

int i6g_code_histogram(const int8_t* codes_dev, int64_t n, int accumulate, int64_t* hist_dev, void* stream) {
  if (n < 0 || !hist_dev || (n > 0 && !codes_dev)) return fail(I6G_EINVAL, "code_histogram: n < 0 or NULL buffer");
  if (n > 0 && !aligned(codes_dev, 16)) return fail(I6G_EUNSUPPORTED, "code_histogram: codes must be 16-byte aligned");
  if (n > code_histogram_max_codes())
    return fail(I6G_EUNSUPPORTED, "code_histogram: n = %lld is beyond the %lld codes one call covers", (long long)n,
                (long long)code_histogram_max_codes());
  HIP_TRY(launch_code_histogram(codes_dev, n, accumulate != 0, hist_dev, (hipStream_t)stream));
  return I6G_OK;
}

int i6g_code_histogram_noalloc(const int8_t* codes_dev, int64_t n, int accumulate, int64_t* hist_dev,
                               void* stream) {
  if (n < 0 || !hist_dev || (n > 0 && !codes_dev))
    return fail(I6G_EINVAL, "code_histogram_noalloc: n < 0 or NULL buffer");
  if (n > 0 && !aligned(codes_dev, 16))
    return fail(I6G_EUNSUPPORTED, "code_histogram_noalloc: codes must be 16-byte aligned");
  if (n > code_histogram_max_codes())
    return fail(I6G_EUNSUPPORTED, "code_histogram_noalloc: n = %lld is beyond the %lld codes one call covers",
                (long long)n, (long long)code_histogram_max_codes());
  HIP_TRY(launch_code_histogram_noalloc(codes_dev, n, accumulate != 0, hist_dev, (hipStream_t)stream));
  return I6G_OK;
}

int i6g_code_entropy(const int64_t* hist_dev, double* bits_dev, void* stream) {
  if (!hist_dev || !bits_dev) return fail(I6G_EINVAL, "code_entropy: NULL buffer");
  HIP_TRY(launch_code_entropy(hist_dev, bits_dev, (hipStream_t)stream));
  return I6G_OK;
}

int i6g_artifact_bytes(const int64_t* shapes, const int32_t* bits, int32_t n_mats, int64_t passthrough_elements,
                       int64_t* bytes) {
  if (!bytes || n_mats < 0 || passthrough_elements < 0 || (n_mats > 0 && !shapes))
    return fail(I6G_EINVAL, "artifact_bytes: negative count or NULL array");
  int64_t total = 2 * passthrough_elements;
  for (int32_t i = 0; i < n_mats; ++i) {
    const int64_t r = shapes[2 * i], c = shapes[2 * i + 1];
    const int b = bits ? bits[i] : 6;
    if (r < 0 || c < 0) return fail(I6G_EINVAL, "artifact_bytes: matrix %d has a negative size", i);
    if (b != 5 && b != 6 && b != 8) return fail(I6G_EINVAL, "artifact_bytes: matrix %d: bits must be 5, 6 or 8", i);
    total += packed_bytes(r * c, b) + 2 * r;
  }
  *bytes = total;
  return I6G_OK;
}

int i6g_load_model(const i6g_model_desc* desc, void* stream, i6g_model** out) {
  if (!out) return fail(I6G_EINVAL, "load_model: out is NULL");
  *out = nullptr;
  if (!desc) return fail(I6G_EINVAL, "load_model: desc is NULL");
  const i6g_model_desc& D = *desc;
  hipStream_t s = (hipStream_t)stream;
  if (D.vocab < 64 || D.vocab % 64 || D.d_model < 128 || D.n_heads < 1 || D.n_kv_heads < 1 ||
      D.head_dim < 1 || D.d_ff < 128 || D.n_unique < 1 || D.n_eff < 1 || !D.schedule || !D.blocks ||
      !D.embed)
    return fail(I6G_EINVAL, "load_model: bad sizes or NULL tensors");
  if (D.n_heads * D.head_dim != D.d_model)
    return fail(I6G_EINVAL, "load_model: n_heads * head_dim != d_model");
  if (D.head_dim != 32 && D.head_dim != 64 && D.head_dim != 80)
    return fail(I6G_EUNSUPPORTED, "load_model: head_dim %d (supported: 32, 64, 80)", D.head_dim);
  if (D.n_heads != 2 * D.n_kv_heads)
    return fail(I6G_EUNSUPPORTED, "load_model: needs n_heads == 2 * n_kv_heads");
  if (D.n_kv_heads % 2)
    return fail(I6G_EUNSUPPORTED, "load_model: needs an even number of kv heads (the v block of the "
                                  "q/k/v projection starts on a two-head tile boundary)");
  if (D.d_model % 128 || D.d_ff % 128 || D.d_model > 640)
    return fail(I6G_EUNSUPPORTED, "load_model: d_model and d_ff must be multiples of 128, d_model <= 640");
  if (D.embed_dtype != I6G_DTYPE_F16 && D.embed_dtype != I6G_DTYPE_F32)
    return fail(I6G_EINVAL, "load_model: embed_dtype");
  if (D.lora_rank < 0 || D.lora_rank > 8) return fail(I6G_EINVAL, "load_model: lora_rank must be 0..8");
  if (D.lora_rank > 0 && (!D.lora_aq || !D.lora_bq || !D.lora_av || !D.lora_bv))
    return fail(I6G_EINVAL, "load_model: LoRA factors missing");
  if (D.bigram_buckets < 0 || (D.bigram_buckets > 0 && (D.bigram_dim < 1 || !D.bigram_table || !D.bigram_proj)))
    return fail(I6G_EINVAL, "load_model: bigram tensors");
  if (D.skip_kind != I6G_SKIP_NONE && (D.n_skip < 1 || !D.skip_weights))
    return fail(I6G_EINVAL, "load_model: skip weights missing");
  for (int e = 0; e < D.n_eff; ++e)
    if (D.schedule[e] < 0 || D.schedule[e] >= D.n_unique)
      return fail(I6G_EINVAL, "load_model: schedule[%d] = %d out of range", e, D.schedule[e]);
  if (!(D.logit_temperature >= 0.0) || !std::isfinite(D.logit_temperature))
    return fail(I6G_EINVAL, "load_model: logit_temperature must be finite and >= 0 (0 = off)");
  // The head scales each normed row (elements up to sqrt(d_model) <= 25.3)
  // by log2(e) / temperature and holds it in binary16 (largest finite 65504):
  // temperatures of at least 0.01 keep that product below 3,700.
  if (D.logit_temperature != 0.0 && D.logit_temperature < 0.01)
    return fail(I6G_EUNSUPPORTED, "load_model: logit_temperature below 0.01 is not supported");
  if (!std::isfinite(D.leaky_slope)) return fail(I6G_EINVAL, "load_model: leaky_slope must be finite");
  if (D.xsa_last_n < 0 || D.xsa_last_n > D.n_eff)
    return fail(I6G_EINVAL, "load_model: xsa_last_n must be in 0..n_eff");
  if (D.rope_dims < 0 || D.rope_dims > D.head_dim)
    return fail(I6G_EINVAL, "load_model: rope_dims must be in 0..head_dim");
  if (D.rope_dims != 0 && D.rope_dims % (D.head_dim / 4))
    return fail(I6G_EUNSUPPORTED, "load_model: rope_dims %d is not a multiple of head_dim/4", D.rope_dims);

  // NaN / Inf in a tensor held in host memory: refused before anything is
  // allocated (device tensors are checked on the device after their copy)
  {
    const int kvd = D.n_kv_heads * D.head_dim;
    for (int b = 0; b < D.n_unique; ++b) {
      const i6g_block& B = D.blocks[b];
      const i6g_matrix* mats[6] = {&B.q, &B.k, &B.v, &B.o, &B.fc, &B.proj};
      const int rows[6] = {D.d_model, kvd, kvd, D.d_model, D.d_ff, D.d_model};
      for (int i = 0; i < 6; ++i)
        if (host_nonfinite_f16(mats[i]->scales, rows[i]))
          return fail(I6G_ENONFINITE, "load_model: block %d matrix %d has a NaN or Inf scale", b, i);
    }
    const int64_t nE = (int64_t)D.vocab * D.d_model;
    if (D.embed_dtype == I6G_DTYPE_F32 ? host_nonfinite_f32((const float*)D.embed, nE)
                                       : host_nonfinite_f16((const uint16_t*)D.embed, nE))
      return fail(I6G_ENONFINITE, "load_model: the embedding holds NaN or Inf");
    const int64_t ne = D.n_eff, r = D.lora_rank;
    if ((D.skip_kind != I6G_SKIP_NONE && host_nonfinite_f16(D.skip_weights, (int64_t)D.n_skip * D.d_model)) ||
        (r > 0 && (host_nonfinite_f16(D.lora_aq, ne * r * D.d_model) ||
                   host_nonfinite_f16(D.lora_bq, ne * D.d_model * r) ||
                   host_nonfinite_f16(D.lora_av, ne * r * D.d_model) || host_nonfinite_f16(D.lora_bv, ne * kvd * r))) ||
        (D.bigram_buckets > 0 &&
         (host_nonfinite_f16(D.bigram_table, (int64_t)D.bigram_buckets * D.bigram_dim) ||
          host_nonfinite_f16(D.bigram_proj, (int64_t)D.d_model * D.bigram_dim))))
      return fail(I6G_ENONFINITE, "load_model: a skip, LoRA or bigram tensor holds NaN or Inf");
  }

  i6g_model* m = new i6g_model();
  m->V = D.vocab; m->d = D.d_model; m->Hq = D.n_heads; m->Hkv = D.n_kv_heads; m->hd = D.head_dim;
  m->F = D.d_ff; m->kvd = D.n_kv_heads * D.head_dim; m->nqkv = m->d + 2 * m->kvd;
  m->rope_base = D.rope_base; m->eps = D.norm_eps;
  m->n_unique = D.n_unique; m->n_eff = D.n_eff;
  m->schedule.assign(D.schedule, D.schedule + D.n_eff);
  m->skip_kind = D.skip_kind; m->n_skip = D.skip_kind == I6G_SKIP_NONE ? 0 : D.n_skip;
  m->parallel = D.parallel_residual != 0; m->lora_r = D.lora_rank;
  m->buckets = D.bigram_buckets; m->bigram_dim = D.bigram_dim;
  m->embed_f32 = D.embed_dtype == I6G_DTYPE_F32;
  m->inv_temp = (D.logit_temperature == 0.0 || D.logit_temperature == 1.0)
                    ? 1.0f : (float)(1.0 / D.logit_temperature);
  m->leaky = (float)D.leaky_slope;
  m->rope_dims = D.rope_dims == 0 ? D.head_dim : D.rope_dims;
  m->xsa_last_n = D.xsa_last_n;
  (void)hipGetDevice(&m->device);

  int rc = build_plan(m);
  if (rc != I6G_OK) { delete m; return rc; }

  auto cleanup = [&](int code) { delete m; return code; };
  const int d = m->d, F = m->F, kvd = m->kvd;
  if (m->flags.ensure(4) != hipSuccess || m->part_n.ensure(256 * 8) != hipSuccess ||
      m->part_b.ensure(256 * 8) != hipSuccess)
    return cleanup(fail(I6G_ENOMEM, "out of device memory"));
  if (hipMemsetAsync(m->flags.p, 0, 4, s) != hipSuccess) return cleanup(fail(I6G_EDEVICE, "memset"));
  int32_t* fl = m->flags.as<int32_t>();
  // the device copies of every floating-point tensor are checked for NaN /
  // Inf (bit 1 of the model's flag word), read back at the end of the load
  auto check = [&](const DevBuf& b, int64_t n, bool f32) -> int {
    if (launch_check_finite(b.p, n, f32, fl, s) != hipSuccess) return fail(I6G_EDEVICE, "finite check failed");
    return I6G_OK;
  };
  m->blocks.resize(m->n_unique);
  for (int b = 0; b < m->n_unique; ++b) {
    const i6g_block& B = D.blocks[b];
    const i6g_matrix* mats[6] = {&B.q, &B.k, &B.v, &B.o, &B.fc, &B.proj};
    for (auto* mt : mats)
      if (!mt->codes || !mt->scales) return cleanup(fail(I6G_EINVAL, "load_model: block %d has a NULL matrix", b));
    BlockDev& bd = m->blocks[b];
    if (bd.qkv_codes.ensure((size_t)m->nqkv * d) != hipSuccess ||
        bd.qkv_scales.ensure((size_t)m->nqkv * 2) != hipSuccess)
      return cleanup(fail(I6G_ENOMEM, "load_model: out of device memory"));
    int8_t* qc = bd.qkv_codes.as<int8_t>();
    uint16_t* qs = bd.qkv_scales.as<uint16_t>();
    if (hipMemcpyAsync(qc, B.q.codes, (size_t)d * d, hipMemcpyDefault, s) != hipSuccess ||
        hipMemcpyAsync(qc + (size_t)d * d, B.k.codes, (size_t)kvd * d, hipMemcpyDefault, s) != hipSuccess ||
        hipMemcpyAsync(qc + (size_t)(d + kvd) * d, B.v.codes, (size_t)kvd * d, hipMemcpyDefault, s) != hipSuccess ||
        hipMemcpyAsync(qs, B.q.scales, (size_t)d * 2, hipMemcpyDefault, s) != hipSuccess ||
        hipMemcpyAsync(qs + d, B.k.scales, (size_t)kvd * 2, hipMemcpyDefault, s) != hipSuccess ||
        hipMemcpyAsync(qs + d + kvd, B.v.scales, (size_t)kvd * 2, hipMemcpyDefault, s) != hipSuccess)
      return cleanup(fail(I6G_EDEVICE, "load_model: copy of q/k/v failed"));
    if ((rc = copy_in(bd.o_codes, B.o.codes, (size_t)d * d, s)) ||
        (rc = copy_in(bd.o_scales, B.o.scales, (size_t)d * 2, s)) ||
        (rc = copy_in(bd.fc_codes, B.fc.codes, (size_t)F * d, s)) ||
        (rc = copy_in(bd.fc_scales, B.fc.scales, (size_t)F * 2, s)) ||
        (rc = copy_in(bd.proj_codes, B.proj.codes, (size_t)d * F, s)) ||
        (rc = copy_in(bd.proj_scales, B.proj.scales, (size_t)d * 2, s)))
      return cleanup(rc);
    if (bd.fc_frag.ensure((size_t)F * d) != hipSuccess || bd.proj_frag.ensure((size_t)d * F) != hipSuccess ||
        bd.o_frag.ensure((size_t)d * d) != hipSuccess)
      return cleanup(fail(I6G_ENOMEM, "load_model: out of device memory"));
    if (launch_shuffle_codes(bd.fc_codes.as<int8_t>(), F, d, nullptr, bd.fc_frag.as<int8_t>(), s) != hipSuccess ||
        launch_shuffle_codes(bd.proj_codes.as<int8_t>(), d, F, bd.proj_scales.as<uint16_t>(),
                             bd.proj_frag.as<int8_t>(), s) != hipSuccess ||
        launch_shuffle_codes(bd.o_codes.as<int8_t>(), d, d, bd.o_scales.as<uint16_t>(), bd.o_frag.as<int8_t>(),
                             s) != hipSuccess)
      return cleanup(fail(I6G_EDEVICE, "load_model: rearranging the codes failed"));
    if (qkv_tile_supported(d, m->hd, m->Hq, m->Hkv, m->rope_dims, m->lora_r)) {
      if (bd.qkv_frag.ensure((size_t)m->nqkv * d) != hipSuccess)
        return cleanup(fail(I6G_ENOMEM, "load_model: out of device memory"));
      if (launch_shuffle_qkv_codes(bd.qkv_codes.as<int8_t>(), m->Hq, m->Hkv, d, m->rope_dims,
                                   bd.qkv_frag.as<int8_t>(), s) != hipSuccess)
        return cleanup(fail(I6G_EDEVICE, "load_model: rearranging the q/k/v codes failed"));
    }
    if ((rc = check(bd.qkv_scales, m->nqkv, false)) || (rc = check(bd.o_scales, d, false)) ||
        (rc = check(bd.fc_scales, F, false)) || (rc = check(bd.proj_scales, d, false)))
      return cleanup(rc);
  }
  const size_t esz = m->embed_f32 ? 4 : 2;
  if ((rc = copy_in(m->embed, D.embed, (size_t)m->V * d * esz, s))) return cleanup(rc);
  if ((rc = check(m->embed, (int64_t)m->V * d, m->embed_f32 != 0))) return cleanup(rc);
  if (m->embed_f32) {
    if (m->embed16.ensure((size_t)m->V * d * 2) != hipSuccess) return cleanup(fail(I6G_ENOMEM, "embed16"));
    if (launch_f32_to_f16(m->embed.as<float>(), m->embed16.as<_Float16>(), (int64_t)m->V * d, s) != hipSuccess)
      return cleanup(fail(I6G_EDEVICE, "embedding conversion failed"));
  }
  DevBuf tmp;
  auto f16_in = [&](DevBuf& dst, const uint16_t* src, int64_t n) -> int {
    int r = copy_in(tmp, src, (size_t)n * 2, s);
    if (r) return r;
    if (dst.ensure((size_t)n * 4) != hipSuccess) return fail(I6G_ENOMEM, "out of device memory");
    if (launch_f16_to_f32(tmp.as<uint16_t>(), dst.as<float>(), n, s) != hipSuccess)
      return fail(I6G_EDEVICE, "f16 conversion failed");
    if (int r2 = check(dst, n, true)) return r2;
    if (hipStreamSynchronize(s) != hipSuccess) return fail(I6G_EDEVICE, "sync failed");
    return I6G_OK;
  };
  if (m->n_skip > 0 && (rc = f16_in(m->skip_w, D.skip_weights, (int64_t)m->n_skip * d))) return cleanup(rc);
  if (m->lora_r > 0) {
    const int64_t ne = m->n_eff, r = m->lora_r;
    if ((rc = f16_in(m->lora_aq, D.lora_aq, ne * r * d)) || (rc = f16_in(m->lora_bq, D.lora_bq, ne * d * r)) ||
        (rc = f16_in(m->lora_av, D.lora_av, ne * r * d)) || (rc = f16_in(m->lora_bv, D.lora_bv, ne * kvd * r)))
      return cleanup(rc);
  }
  if (m->buckets > 0) {
    DevBuf t2;
    if ((rc = copy_in(tmp, D.bigram_table, (size_t)m->buckets * m->bigram_dim * 2, s)) ||
        (rc = copy_in(t2, D.bigram_proj, (size_t)d * m->bigram_dim * 2, s)))
      return cleanup(rc);
    if (m->bigram.ensure((size_t)m->buckets * d * 4) != hipSuccess) return cleanup(fail(I6G_ENOMEM, "bigram"));
    if (launch_bigram_table(tmp.as<uint16_t>(), t2.as<uint16_t>(), m->bigram.as<float>(), m->buckets,
                            m->bigram_dim, d, s) != hipSuccess)
      return cleanup(fail(I6G_EDEVICE, "bigram table kernel failed"));
    // a NaN or Inf in the table or the projection reaches the product table
    if ((rc = check(m->bigram, (int64_t)m->buckets * d, true))) return cleanup(rc);
    if (hipStreamSynchronize(s) != hipSuccess) return cleanup(fail(I6G_EDEVICE, "sync failed"));
  }
  if (hipStreamSynchronize(s) != hipSuccess) return cleanup(fail(I6G_EDEVICE, "sync failed"));
  {
    int32_t f = 0;
    if (hipMemcpy(&f, fl, 4, hipMemcpyDeviceToHost) != hipSuccess) return cleanup(fail(I6G_EDEVICE, "flag read"));
    if (f & I6G_FLAG_NONFINITE)
      return cleanup(fail(I6G_ENONFINITE, "load_model: a scale, the embedding or a skip, LoRA or bigram tensor "
                                          "holds NaN or Inf"));
  }
  *out = m;
  return I6G_OK;
}

void i6g_free_model(i6g_model* m) { delete m; }

int i6g_set_option(i6g_model* m, int option, int64_t value) {
  if (!m) return fail(I6G_EINVAL, "set_option: NULL model");
  switch (option) {
    case I6G_OPT_BATCH_WINDOWS:
      if (value < 0 || value > (1 << 20)) return fail(I6G_EINVAL, "set_option: batch windows %lld", (long long)value);
      m->batch_windows = (int)value;
      return I6G_OK;
    case I6G_OPT_PRUNE_LAST:
      m->prune_last = value != 0;
      return I6G_OK;
    case I6G_OPT_STREAMS:
      if (value != 1 && value != 2) return fail(I6G_EINVAL, "set_option: streams must be 1 or 2");
      m->streams = (int)value;
      return I6G_OK;
    case I6G_OPT_REGISTER_CODES:
      m->register_codes = value != 0;
      return I6G_OK;
    case I6G_OPT_FUSED_TAIL:
      m->fused_tail = value != 0;
      return I6G_OK;
    case I6G_OPT_QKV_TILE:
      m->qkv_tile = value != 0;
      return I6G_OK;
  }
  return fail(I6G_EINVAL, "set_option: unknown option %d", option);
}

int i6g_model_status(i6g_model* m, void* stream) {
  if (!m) return fail(I6G_EINVAL, "model_status: NULL model");
  HIP_TRY(hipStreamSynchronize((hipStream_t)stream));
  int32_t f = 0;
  HIP_TRY(hipMemcpy(&f, m->flags.p, 4, hipMemcpyDeviceToHost));
  HIP_TRY(hipMemset(m->flags.p, 0, 4));
  if (f & I6G_FLAG_TOKEN) return fail(I6G_ETOKEN, "a token id was outside [0, vocab)");
  if (f & I6G_FLAG_BYTES) return fail(I6G_EBYTES, "negative byte count or zero total bytes");
  if (f & I6G_FLAG_RANGE)
    return fail(I6G_EUNSUPPORTED, "an activation left the binary16 range (a residual row with a sum of squares "
                                  "of at least 65504^2, or an MLP hidden value of at least 65504)");
  return I6G_OK;
}

int i6g_score_tokens(i6g_model* m, const int32_t* tokens_dev, const int32_t* bytes_dev, int64_t n_tokens,
                     int32_t window, int32_t stride, float* nats_dev, double* totals_dev, void* stream) {
  if (!m) return fail(I6G_EINVAL, "score_tokens: NULL model");
  if (!tokens_dev || !bytes_dev || !nats_dev || !totals_dev) return fail(I6G_EINVAL, "score_tokens: NULL array");
  if (n_tokens < 2 || window < 1 || stride < 1 || stride > window)
    return fail(I6G_EINVAL, "score_tokens: need n_tokens >= 2 and 1 <= stride <= window");
  {
    int dev = -1;
    HIP_TRY(hipGetDevice(&dev));
    if (dev != m->device)
      return fail(I6G_EINVAL, "score_tokens: the model was loaded on device %d but device %d is current", m->device,
                  dev);
  }
  hipStream_t s = (hipStream_t)stream;
  const int64_t P = n_tokens - 1;
  const int64_t L = window, S = stride;
  const int64_t K = window_count(P, L, S);
  const int64_t Lp64 = (std::min<int64_t>(L, P) + 63) / 64 * 64;
  // Element offsets are 64-bit in the kernels, but row indices, a window's
  // position x head_dim offsets (head_dim <= 80) and GEMM tile indices
  // (rows / 128 down, tiles at least 64 columns wide across) are 32-bit: a
  // batch holds fewer than 2^24 rows and fewer than 2^31 tiles of its widest
  // GEMM.
  const int64_t widest = std::max<int64_t>((int64_t)m->d + 2 * m->kvd, m->F);
  const int64_t max_rows = std::min<int64_t>(INT32_MAX / 128, 128 * (INT32_MAX / ((widest + 63) / 64)));
  if (Lp64 > max_rows)
    return fail(I6G_EUNSUPPORTED, "score_tokens: a window of %lld positions exceeds the %lld rows a batch can hold "
                "for this model", (long long)Lp64, (long long)max_rows);
  const int Lp = (int)Lp64;
  // The fused block tail (d_model 512) runs one 128-row tile per CU: a
  // batch of 131072 rows (64 windows of 2048) is four full waves of 256
  // tiles (measured 4 % more scored tokens/s than two waves: each tile's
  // load and store bursts overlap other tiles' arithmetic more often).
  // Without it, 49152 rows (24 windows) split the separate GEMMs' tiles
  // evenly over the workgroups the device holds at once.
  const bool tail = m->fused_tail && m->d == 512 && m->F % 128 == 0 && P < INT32_MAX;
  // the one-tile q/k/v kernel needs a row block of a tile to span at most
  // two windows
  const bool qkv_tile = m->qkv_tile && Lp >= 128;
  int Wb = m->batch_windows > 0 ? m->batch_windows : std::max(1, (tail ? 131072 : 49152) / Lp);
  Wb = (int)std::min<int64_t>({(int64_t)Wb, K, max_rows / Lp});
  const bool two = m->streams == 2 && K > Wb;
  int rc = ensure_scratch(m, Wb, Lp, s, two ? 2 : 1, !tail);
  if (rc) return rc;

  const int d = m->d, F = m->F, kvd = m->kvd, nt = d / 128;
  const float eps = (float)m->eps;
  const float scale_log2 = (float)(1.4426950408889634 / sqrt((double)m->hd));
  const int64_t e0 = window_end(0, P, L, S);

  // Batches alternate between the caller's stream and the model's second
  // stream (each with its own scratch set), so that one batch's memory-bound
  // kernels can overlap the other's compute-bound ones; the second stream
  // starts after the caller's prior work and the caller's stream waits for
  // it before the final reduction.
  const hipStream_t s_caller = s;
  if (two) {
    HIP_TRY(hipEventRecord(m->ev_fork, s_caller));
    HIP_TRY(hipStreamWaitEvent(m->aux, m->ev_fork, 0));
  }
  int64_t batch = 0;
  for (int64_t k0 = 0; k0 < K; k0 += Wb, ++batch) {
    const bool odd = two && (batch & 1);
    s = odd ? m->aux : s_caller;
    auto& sc = m->sc[odd ? 1 : 0];
    const int W = (int)std::min<int64_t>(Wb, K - k0);
    const int M = W * Lp;
    // predictions scored by this batch
    const int64_t p0 = (k0 == 0) ? 0 : window_end(k0 - 1, P, L, S);
    const int64_t p1 = window_end(k0 + W - 1, P, L, S);
    const int R = (int)(p1 - p0);
    // In the final layer only scored rows need queries, the output
    // projection and the MLP (K and V still come from every row): exact.
    const bool prune = m->prune_last && R < M;
    // real rows of this batch (for algorithmic FLOP counts)
    double real_rows = 0, attn_pairs = 0, attn_pairs_scored = 0;
    for (int64_t k = k0; k < k0 + W; ++k) {
      const double T = (double)(window_end(k, P, L, S) - k * S);
      const double j0 = (double)(std::max(k * S, k == 0 ? (int64_t)0 : window_end(k - 1, P, L, S)) - k * S);
      real_rows += T;
      attn_pairs += T * (T + 1) / 2;
      attn_pairs_scored += (T * (T + 1) - j0 * (j0 + 1)) / 2;
    }

    EmbedArgs ea{};
    ea.tokens = tokens_dev; ea.n_tokens = n_tokens; ea.P = P; ea.k0 = k0;
    ea.W = W; ea.Lp = Lp; ea.L = (int32_t)L; ea.S = (int32_t)S;
    ea.embed = m->embed.p; ea.embed_f32 = m->embed_f32;
    ea.bigram = m->buckets > 0 ? m->bigram.as<float>() : nullptr; ea.buckets = m->buckets;
    ea.vocab = m->V; ea.d = d; ea.nt = nt;
    ea.x = sc.x.as<float>(); ea.xb = sc.xb.as<act>(); ea.ss = sc.ss.as<float>();
    ea.flags = m->flags.as<int32_t>();
    if ((rc = timed(m, I6G_K_EMBED, s, 0.0, real_rows * d * 6.0, [&] { return launch_embed(ea, s); })))
      return rc;

    // set when the previous block tail computed this layer's q, k and v
    bool qkv_done = false;
    // where the residual stream is: x, or the skip slot the previous block
    // tail pushed it into without also writing x
    const float* resid = sc.x.as<float>();
    for (int e = 0; e < m->n_eff; ++e) {
      const BlockDev& B = m->blocks[m->schedule[e]];
      const bool last = (e + 1 == m->n_eff);
      if (m->lora_r > 0) {
        LoraArgs la{};
        la.x = resid; la.M = M; la.d = d; la.r = m->lora_r; la.eps = eps;
        la.aq = m->lora_aq.as<float>() + (size_t)e * m->lora_r * d;
        la.av = m->lora_av.as<float>() + (size_t)e * m->lora_r * d;
        la.u = sc.lora_u.as<float>();
        if ((rc = timed(m, I6G_K_LORA, s, 4.0 * real_rows * m->lora_r * d, real_rows * d * 4.0,
                        [&] { return launch_lora_down(la, s); })))
          return rc;
      }
      GemmArgs g{};
      g.A = sc.xb.as<act>(); g.B = B.qkv_codes.as<int8_t>(); g.scale = B.qkv_scales.as<uint16_t>();
      g.M = M; g.N = m->nqkv; g.K = d; g.ss_in = sc.ss.as<float>(); g.nt_in = nt; g.eps = eps;
      g.q = sc.q.as<act>(); g.k = sc.k.as<act>(); g.vt = sc.vt.as<act>();
      g.n_heads = m->Hq; g.n_kv = m->Hkv; g.hd = m->hd; g.Lp = Lp; g.rope = m->rope.as<float2>();
      g.rope_dims = m->rope_dims;
      if (m->lora_r > 0) {
        g.lora_u = sc.lora_u.as<float>(); g.lora_r = m->lora_r;
        g.lora_bq = m->lora_bq.as<float>() + (size_t)e * d * m->lora_r;
        g.lora_bv = m->lora_bv.as<float>() + (size_t)e * kvd * m->lora_r;
      }
      const double fl_qkv = 2.0 * real_rows * m->nqkv * d;
      const bool one_tile = qkv_tile && B.qkv_frag.p;
      if (one_tile) g.Bp = B.qkv_frag.as<int8_t>();
      if (!qkv_done &&
          (rc = timed(m, I6G_K_QKV, s, fl_qkv, real_rows * (2.0 * d + 2.0 * m->nqkv) + (double)m->nqkv * d,
                      [&] { return one_tile ? launch_qkv_tile(g, s) : launch_gemm(EPI_QKV, g, s); })))
        return rc;
      qkv_done = false;

      const bool pr = last && prune;
      AttnArgs at{};
      at.q = sc.q.as<act>(); at.k = sc.k.as<act>(); at.vt = sc.vt.as<act>(); at.o = sc.o.as<act>();
      at.W = W; at.n_heads = m->Hq; at.n_kv = m->Hkv; at.hd = m->hd; at.Lp = Lp; at.scale_log2 = scale_log2;
      at.prune = pr; at.k0 = k0; at.P = P; at.L = (int32_t)L; at.S = (int32_t)S;
      at.xsa = e >= m->n_eff - m->xsa_last_n;
      if ((rc = timed(m, I6G_K_ATTN, s, 4.0 * m->hd * m->Hq * (pr ? attn_pairs_scored : attn_pairs),
                      real_rows * (2.0 * d + 4.0 * kvd),
                      [&] { return launch_attention(at, s); })))
        return rc;

      // attention output projection, residual add
      GemmArgs go{};
      go.flags = m->flags.as<int32_t>();
      go.A = sc.o.as<act>(); go.B = B.o_codes.as<int8_t>(); go.scale = B.o_scales.as<uint16_t>();
      go.M = M; go.N = d; go.K = d; go.x = sc.x.as<float>();
      if (!m->parallel) { go.xb = sc.xb.as<act>(); go.ss_out = sc.ss.as<float>(); }

      GemmArgs gf{};
      gf.flags = m->flags.as<int32_t>();
      gf.A = sc.xb.as<act>(); gf.B = B.fc_codes.as<int8_t>(); gf.scale = B.fc_scales.as<uint16_t>();
      if (m->register_codes) gf.Bp = B.fc_frag.as<int8_t>();
      gf.M = M; gf.N = F; gf.K = d; gf.ss_in = sc.ss.as<float>(); gf.nt_in = nt; gf.eps = eps;
      gf.h = sc.h.as<act>(); gf.leaky = m->leaky;

      GemmArgs gp{};
      gp.flags = m->flags.as<int32_t>();
      gp.A = sc.h.as<act>(); gp.B = B.proj_codes.as<int8_t>(); gp.scale = B.proj_scales.as<uint16_t>();
      if (m->register_codes) gp.Bp = B.proj_frag.as<int8_t>();
      gp.M = M; gp.N = d; gp.K = F; gp.x = sc.x.as<float>();
      if (!last) { gp.xb = sc.xb.as<act>(); gp.ss_out = sc.ss.as<float>(); }
      if (m->push_after[e]) gp.push_dst = sc.slots.as<float>() + (size_t)m->push_slot[e] * M * d;
      if (!last && m->pop_before[e + 1] >= 0) {
        gp.pop_src = sc.slots.as<float>() + (size_t)m->pop_slot[e + 1] * M * d;
        gp.pop_w = m->skip_w.as<float>() + (size_t)m->pop_before[e + 1] * d;
      }
      if (pr) {
        // GEMM row r = prediction p0 + r; o, xb, ss and x are read and
        // written at the row the prediction occupies in the batch, h is
        // compact
        for (GemmArgs* g2 : {&go, &gf, &gp}) {
          g2->M = R;
          g2->p0 = p0; g2->k0 = k0; g2->n_win = K; g2->e0 = e0;
          g2->L = (int32_t)L; g2->S = (int32_t)S; g2->Lp = Lp;
        }
        go.a_map = 1; go.e_map = 1;
        gf.a_map = 1;
        gp.e_map = 1;
      }

      const double rows_mlp = pr ? (double)R : real_rows;
      const double fl_o = 2.0 * rows_mlp * d * d, fl_fc = 2.0 * rows_mlp * F * d;
      if (tail) {
        // output projection, norm and MLP in one kernel: algorithmic bytes
        // per row are the attention output, the residual read and written,
        // its binary16 copy, skip slots, plus the codes once per launch
        TailArgs ta{};
        ta.flags = m->flags.as<int32_t>();
        ta.o = sc.o.as<act>();
        ta.o_frag = B.o_frag.as<int8_t>(); ta.o_scale = B.o_scales.as<uint16_t>();
        ta.fc_frag = B.fc_frag.as<int8_t>(); ta.fc_scale = B.fc_scales.as<uint16_t>();
        ta.proj_frag = B.proj_frag.as<int8_t>(); ta.proj_scale = B.proj_scales.as<uint16_t>();
        ta.M = pr ? R : M; ta.F = F; ta.eps = eps; ta.leaky = m->leaky;
        ta.x_in = resid;
        ta.x = sc.x.as<float>();
        if (!last) { ta.xb = sc.xb.as<act>(); ta.ss_out = sc.ss.as<float>(); }
        if (m->push_after[e]) ta.push_dst = sc.slots.as<float>() + (size_t)m->push_slot[e] * M * d;
        if (!last && m->pop_before[e + 1] >= 0) {
          ta.pop_src = sc.slots.as<float>() + (size_t)m->pop_slot[e + 1] * M * d;
          ta.pop_w = m->skip_w.as<float>() + (size_t)m->pop_before[e + 1] * d;
        }
        ta.parallel = m->parallel;
        ta.xb_in = sc.xb.as<act>(); ta.ss_in = sc.ss.as<float>(); ta.nt_in = nt;
        if (pr) {
          ta.row_map = 1;
          ta.p0 = p0; ta.k0 = k0; ta.n_win = K; ta.e0 = e0;
          ta.L = (int32_t)L; ta.S = (int32_t)S; ta.Lp = Lp;
        }
        // the next layer's q, k and v from this tail's output rows (its
        // binary16 copy and sums of squares then stay on the chip unless
        // the parallel lanes read them)
        const BlockDev* Bn = last ? nullptr : &m->blocks[m->schedule[e + 1]];
        const bool fuse = qkv_tile && !pr && Bn && Bn->qkv_frag.p;
        if (fuse) {
          ta.qkv.frag = Bn->qkv_frag.as<int8_t>(); ta.qkv.scale = Bn->qkv_scales.as<uint16_t>();
          ta.qkv.q = sc.q.as<act>(); ta.qkv.k = sc.k.as<act>(); ta.qkv.vt = sc.vt.as<act>();
          ta.qkv.rope = m->rope.as<float2>();
          ta.qkv.n_heads = m->Hq; ta.qkv.n_kv = m->Hkv; ta.qkv.rope_dims = m->rope_dims;
          ta.Lp = Lp;
          if (!m->parallel) { ta.xb = nullptr; ta.ss_out = nullptr; }
        }
        // a tail that pushes its result and pops nothing stores it only into
        // the skip slot, and the next tail reads its residual from there
        // (the final layer's result goes to x for the head)
        if (!last && ta.push_dst && !ta.pop_src) ta.x = nullptr;
        resid = ta.x ? sc.x.as<float>() : ta.push_dst;
        double per_row = 2.0 * d + (ta.x ? 8.0 * d : 4.0 * d) + (ta.xb ? 2.0 * d : 0.0) + (ta.push_dst ? 4.0 * d : 0.0) +
                         (ta.pop_src && ta.pop_src != ta.push_dst ? 4.0 * d : 0.0) + (m->parallel ? 2.0 * d : 0.0) +
                         (fuse ? 2.0 * m->nqkv : 0.0);
        const double by_t =
            rows_mlp * per_row + (double)d * d + 2.0 * (double)F * d + (fuse ? (double)m->nqkv * d : 0.0);
        const double fl_t = fl_o + 2.0 * fl_fc + (fuse ? 2.0 * real_rows * m->nqkv * d : 0.0);
        // residual rows spread over the output projection's K steps where a
        // row's place in its tile does not depend on the batching: not in
        // the final layer (whether its rows are pruned, and so remapped,
        // depends on the batch), and only for windows padded to a multiple
        // of the 128-row tile
        ta.spread_residual = !last && Lp % 128 == 0;
        if ((rc = timed(m, I6G_K_TAIL, s, fl_t, by_t, [&] { return launch_tail(ta, s); })))
          return rc;
        qkv_done = fuse;
        continue;
      }
      // algorithmic HBM bytes: A read, fp32 residual read + write, bf16 copy,
      // skip slot written / read, codes (scales and sums of squares are small)
      auto res_bytes = [&](const GemmArgs& g, double a_cols) {
        double per_row = 2.0 * a_cols + 8.0 * d;
        if (g.xb) per_row += 2.0 * d;
        if (g.push_dst) per_row += 4.0 * d;
        if (g.pop_src && g.pop_src != g.push_dst) per_row += 4.0 * d;
        return rows_mlp * per_row + a_cols * d;
      };
      const double by_o = res_bytes(go, d);
      const double by_fc = rows_mlp * (2.0 * d + 2.0 * F) + (double)F * d;
      const double by_p = res_bytes(gp, F);
      auto run_o = [&] {
        return timed(m, I6G_K_OPROJ, s, fl_o, by_o, [&] { return launch_gemm(EPI_RES, go, s); });
      };
      auto run_fc = [&] {
        return timed(m, I6G_K_FC, s, fl_fc, by_fc, [&] { return launch_gemm(EPI_RELU2, gf, s); });
      };
      if (m->parallel) {
        if ((rc = run_fc()) || (rc = run_o())) return rc;
      } else {
        if ((rc = run_o()) || (rc = run_fc())) return rc;
      }
      if ((rc = timed(m, I6G_K_PROJ, s, fl_fc, by_p, [&] { return launch_gemm(EPI_RES, gp, s); })))
        return rc;
    }

    HeadArgs ha{};
    ha.x = sc.x.as<float>();
    ha.E = m->embed_f32 ? m->embed16.as<_Float16>() : m->embed.as<_Float16>();
    ha.tokens = tokens_dev; ha.nats = nats_dev;
    ha.p0 = p0;
    ha.p1 = p1;
    ha.k0 = k0; ha.K = K; ha.e0 = e0; ha.L = (int32_t)L; ha.S = (int32_t)S; ha.Lp = Lp; ha.d = d;
    ha.vocab = m->V; ha.eps = eps; ha.flags = m->flags.as<int32_t>(); ha.inv_temp = m->inv_temp;
    const double Rd = (double)R;
    if ((rc = timed(m, I6G_K_HEAD, s, 2.0 * Rd * m->V * d, Rd * d * 4.0 + (double)m->V * d * 2,
                    [&] { return launch_head(ha, s); })))
      return rc;
  }

  s = s_caller;
  if (two) {
    HIP_TRY(hipEventRecord(m->ev_join, m->aux));
    HIP_TRY(hipStreamWaitEvent(s_caller, m->ev_join, 0));
  }
  ReduceArgs ra{};
  ra.nats = nats_dev; ra.bytes = bytes_dev; ra.P = P;
  ra.part_nats = m->part_n.as<double>(); ra.part_bytes = m->part_b.as<long long>();
  ra.n_parts = (int32_t)std::min<int64_t>(256, (P + 255) / 256);
  ra.totals = totals_dev; ra.flags = m->flags.as<int32_t>();
  if ((rc = timed(m, I6G_K_REDUCE, s, (double)P, (double)P * 8.0, [&] { return launch_reduce(ra, s); })))
    return rc;
  return I6G_OK;
}

int i6g_set_timing(i6g_model* m, int enable, uint32_t class_mask) {
  if (!m) return fail(I6G_EINVAL, "set_timing: NULL model");
  if (m->timed_stream) (void)hipStreamSynchronize(m->timed_stream);
  for (auto& r : m->recs) { m->pool.push_back(r.a); m->pool.push_back(r.b); }
  m->recs.clear();
  m->timing = enable != 0;
  m->timing_mask = class_mask;
  for (int c = 0; c < I6G_K_COUNT; ++c) { m->t_ms[c] = m->t_flops[c] = m->t_bytes[c] = 0; m->t_n[c] = 0; }
  return I6G_OK;
}

int i6g_get_timing(i6g_model* m, int kernel_class, double* total_ms, int64_t* launches, double* flops,
                   double* bytes) {
  if (!m || kernel_class < 0 || kernel_class >= I6G_K_COUNT) return fail(I6G_EINVAL, "get_timing");
  if (!m->recs.empty()) {
    HIP_TRY(hipStreamSynchronize(m->timed_stream));
    if (m->aux) HIP_TRY(hipStreamSynchronize(m->aux));
    for (auto& r : m->recs) {
      float ms = 0.f;
      HIP_TRY(hipEventElapsedTime(&ms, r.a, r.b));
      m->t_ms[r.cls] += ms;
      m->t_flops[r.cls] += r.flops;
      m->t_bytes[r.cls] += r.bytes;
      m->t_n[r.cls] += 1;
      m->pool.push_back(r.a);
      m->pool.push_back(r.b);
    }
    m->recs.clear();
  }
  if (total_ms) *total_ms = m->t_ms[kernel_class];
  if (launches) *launches = m->t_n[kernel_class];
  if (flops) *flops = m->t_flops[kernel_class];
  if (bytes) *bytes = m->t_bytes[kernel_class];
  return I6G_OK;
}

}  // extern "C"
