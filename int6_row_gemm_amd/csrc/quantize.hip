// Per-row int8 / int6 / int5 quantiser: one wavefront per row.
//
// pwwt.cn "parameter-golf 16MB 极限压缩实战 …", sections 训练时的模拟量化 and
// 后训练量化导出: scale = clipped |w| maximum / 127 per row, stored binary16;
// codes round(w/scale), in int6 mode round(code/4)*4 clamped to [-128, 124].
// The clip value is the linear-interpolation quantile of |w| over the row
// (at q = 0.99999 84 only the top two order statistics matter for rows up to
// 625,000 long); kwkr.cn PR #363 Noisy-QAT block: floor 1e-12.  int5 (the
// same write-up's MLP_INT5 / ATTN_INT5 export, step amax / 15): scale = c/15,
// codes round(w/scale) clamped to [-16, 15].
//
// Every fp32 operation is rounded on its own: contraction into FMA is off in
// this file and division is IEEE correctly rounded (the HIP default), so the
// codes and scales are bit-identical to a plain binary32 evaluation.
#include "common.h"

#pragma clang fp contract(off)

namespace i6g {
namespace {

constexpr int kTop = 8;  // most largest |w| a row's quantile may need

template <int KT>
__device__ inline void insert_top(float (&t)[KT], float a) {
  // t is sorted descending; insert a and drop the smallest.
#pragma unroll
  for (int i = 0; i < KT; ++i) {
    float hi = fmaxf(t[i], a);
    float lo = fminf(t[i], a);
    t[i] = hi;
    a = lo;
  }
}

// One row of `cols` fp32 weights -> codes and a binary16 scale, on one
// wavefront (every lane must call it).  Each lane keeps its KT >= topk
// largest |w|; the quantile of every row length these models use needs the
// top two (q < 1) or one (q = 1), so KT = 2 covers them with a quarter of
// the compare work of the general KT = 8.
// FQ: instead of codes and the binary16 scale, write the fake-quantised
// row code * scale (fp32 scale, one rounding) to fq as fp32 or bfloat16.
template <int KT, bool FQ>
__device__ void quantize_row_k(const float* w, int cols, int topk, float frac, int bits, int8_t* codes,
                               uint16_t* scale_out, int32_t* flags, int lane, void* fq, int fq_bf16) {
  // The row is read in chunks of kU elements per lane whose loads are all
  // issued before any is used, so their latencies overlap.
  constexpr int kU = 8;
  float top[KT];
#pragma unroll
  for (int i = 0; i < KT; ++i) top[i] = -1.0f;
  int bad = 0;
  for (int c0 = 0; c0 < cols; c0 += kU * kWave) {
    float v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int c = c0 + u * kWave + lane;
      v[u] = c < cols ? w[c] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      bad |= !isfinite(v[u]);
      insert_top<KT>(top, fabsf(v[u]));   // a 0 past the row end never displaces a |w|
    }
  }
  bad = __any(bad);
  if (bad) {
    for (int c = lane; c < cols; c += kWave) {
      if (FQ) {
        if (fq_bf16) static_cast<uint16_t*>(fq)[c] = 0x7FC0;
        else static_cast<float*>(fq)[c] = __builtin_nanf("");
      } else {
        codes[c] = 0;
      }
    }
    if (lane == 0) {
      if (!FQ) *scale_out = 0x7e00;
      if (flags) atomicOr(flags, 1);
    }
    return;
  }

  // Extract the topk largest values of the row in descending order; the
  // last two extracted are s[lo] and s[lo + 1].
  float s_lo = 0.0f, s_prev = 0.0f;
  for (int r = 0; r < topk; ++r) {
    float best = top[0];
    int who = lane;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      float ob = __shfl_xor(best, off);
      int ow = __shfl_xor(who, off);
      if (ob > best || (ob == best && ow < who)) { best = ob; who = ow; }
    }
    if (lane == who) {
#pragma unroll
      for (int i = 0; i < KT - 1; ++i) top[i] = top[i + 1];
      top[KT - 1] = -1.0f;
    }
    s_prev = s_lo;
    s_lo = best;
  }
  const float s_hi = (topk >= 2) ? s_prev : s_lo;

  float diff = s_hi - s_lo;
  float step = frac * diff;
  float c = s_lo + step;
  c = fmaxf(c, 1e-12f);
  const float scale = c / (bits == 5 ? 15.0f : 127.0f);

  for (int c0 = 0; c0 < cols; c0 += kU * kWave) {
    float wv[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int col = c0 + u * kWave + lane;
      wv[u] = col < cols ? w[col] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int col = c0 + u * kWave + lane;
      float v = fminf(fmaxf(wv[u], -c), c);
      float r = v / scale;
      float k = rintf(r);
      float code;
      if (bits == 8) {
        code = fminf(fmaxf(k, -127.0f), 127.0f);
      } else if (bits == 5) {
        code = fminf(fmaxf(k, -16.0f), 15.0f);
      } else {
        float k4 = rintf(k * 0.25f);
        code = fminf(fmaxf(k4 * 4.0f, -128.0f), 124.0f);
      }
      if (col < cols) {
        if (FQ) {
          // the code as an integer: a zero code gives +0, as the
          // straight-through sum w + (w_q - w) does
          const float q = (float)(int)code * scale;
          if (fq_bf16) static_cast<__bf16*>(fq)[col] = (__bf16)q;   // v_cvt_pk_bf16_f32: nearest even
          else static_cast<float*>(fq)[col] = q;
        } else {
          codes[col] = (int8_t)(int)code;
        }
      }
    }
  }
  if (!FQ && lane == 0) {
    _Float16 h = (_Float16)scale;   // v_cvt_f16_f32: round to nearest even
    *scale_out = __builtin_bit_cast(uint16_t, h);
  }
}

__device__ inline void quantize_row(const float* w, int cols, int topk, float frac, int bits,
                                    int8_t* codes, uint16_t* scale_out, int32_t* flags, int lane) {
  if (topk <= 2)
    quantize_row_k<2, false>(w, cols, topk, frac, bits, codes, scale_out, flags, lane, nullptr, 0);
  else
    quantize_row_k<kTop, false>(w, cols, topk, frac, bits, codes, scale_out, flags, lane, nullptr, 0);
}

__global__ __launch_bounds__(256) void quantize_rows_kernel(QuantArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t row = (int64_t)blockIdx.x * (blockDim.x / kWave) + (threadIdx.x / kWave);
  if (row >= a.rows) return;
  quantize_row(a.w + row * a.cols, a.cols, a.topk, a.frac, a.bits, a.codes + row * a.cols,
               a.scales + row, a.flags, lane);
}

// The straight-through forward value of each row (fake quantisation).
__global__ __launch_bounds__(256) void fake_quant_kernel(QuantArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t row = (int64_t)blockIdx.x * (blockDim.x / kWave) + (threadIdx.x / kWave);
  if (row >= a.rows) return;
  void* out = a.fq_bf16 ? (void*)(static_cast<uint16_t*>(a.fq) + row * a.cols)
                        : (void*)(static_cast<float*>(a.fq) + row * a.cols);
  if (a.topk <= 2)
    quantize_row_k<2, true>(a.w + row * a.cols, a.cols, a.topk, a.frac, a.bits, nullptr, nullptr, a.flags, lane,
                            out, a.fq_bf16);
  else
    quantize_row_k<kTop, true>(a.w + row * a.cols, a.cols, a.topk, a.frac, a.bits, nullptr, nullptr, a.flags,
                               lane, out, a.fq_bf16);
}

// Rows of several matrices in one grid; the job of a row is found by a
// scan of the (at most 64) row offsets, which are in the kernel arguments.
__global__ __launch_bounds__(256) void quantize_many_kernel(QuantManyArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t row = (int64_t)blockIdx.x * (blockDim.x / kWave) + (threadIdx.x / kWave);
  if (row >= a.row0[a.n]) return;
  int j = 0;
  while (j + 1 < a.n && a.row0[j + 1] <= row) ++j;
  const QuantJob& q = a.job[j];
  const int64_t r = row - a.row0[j];
  quantize_row(q.w + r * q.cols, q.cols, q.topk, q.frac, a.bits, q.codes + r * q.cols, q.scales + r,
               a.flags, lane);
}

}  // namespace

hipError_t launch_quantize(const QuantArgs& a, hipStream_t s) {
  const int rows_per_block = 4;
  int64_t blocks = (a.rows + rows_per_block - 1) / rows_per_block;
  hipLaunchKernelGGL(quantize_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_fake_quantize(const QuantArgs& a, hipStream_t s) {
  const int rows_per_block = 4;
  int64_t blocks = (a.rows + rows_per_block - 1) / rows_per_block;
  hipLaunchKernelGGL(fake_quant_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_quantize_many(const QuantManyArgs& a, hipStream_t s) {
  const int rows_per_block = 4;
  int64_t blocks = (a.row0[a.n] + rows_per_block - 1) / rows_per_block;
  hipLaunchKernelGGL(quantize_many_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace i6g
