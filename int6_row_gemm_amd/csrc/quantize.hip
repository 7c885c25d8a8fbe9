// Per-row int8 / int6 quantiser: one wavefront per row.
//
// pwwt.cn "parameter-golf 16MB 极限压缩实战 …", sections 训练时的模拟量化 and
// 后训练量化导出: scale = clipped |w| maximum / 127 per row, stored binary16;
// codes round(w/scale), in int6 mode round(code/4)*4 clamped to [-128, 124].
// The clip value is the linear-interpolation quantile of |w| over the row
// (at q = 0.99999 84 only the top two order statistics matter for rows up to
// 625,000 long); kwkr.cn PR #363 Noisy-QAT block: floor 1e-12.
//
// Every fp32 operation is rounded on its own: contraction into FMA is off in
// this file and division is IEEE correctly rounded (the HIP default), so the
// codes and scales are bit-identical to a plain binary32 evaluation.
#include "common.h"

#pragma clang fp contract(off)

namespace i6g {
namespace {

constexpr int kTop = 8;  // largest |w| kept per lane and per row

__device__ inline void insert_top(float (&t)[kTop], float a) {
  // t is sorted descending; insert a and drop the smallest.
#pragma unroll
  for (int i = 0; i < kTop; ++i) {
    float hi = fmaxf(t[i], a);
    float lo = fminf(t[i], a);
    t[i] = hi;
    a = lo;
  }
}

__global__ __launch_bounds__(256) void quantize_rows_kernel(QuantArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t row = (int64_t)blockIdx.x * (blockDim.x / kWave) + (threadIdx.x / kWave);
  if (row >= a.rows) return;
  const float* w = a.w + row * a.cols;

  float top[kTop];
#pragma unroll
  for (int i = 0; i < kTop; ++i) top[i] = -1.0f;
  int bad = 0;
  for (int c = lane; c < a.cols; c += kWave) {
    float v = w[c];
    bad |= !isfinite(v);
    insert_top(top, fabsf(v));
  }
  bad = __any(bad);
  if (bad) {
    for (int c = lane; c < a.cols; c += kWave) a.codes[row * a.cols + c] = 0;
    if (lane == 0) {
      a.scales[row] = 0x7e00;
      if (a.flags) atomicOr(a.flags, 1);
    }
    return;
  }

  // Extract the topk largest values of the row in descending order; the
  // last two extracted are s[lo] and s[lo + 1].
  float s_lo = 0.0f, s_prev = 0.0f;
  for (int r = 0; r < a.topk; ++r) {
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
      for (int i = 0; i < kTop - 1; ++i) top[i] = top[i + 1];
      top[kTop - 1] = -1.0f;
    }
    s_prev = s_lo;
    s_lo = best;
  }
  const float s_hi = (a.topk >= 2) ? s_prev : s_lo;

  float diff = s_hi - s_lo;
  float step = a.frac * diff;
  float c = s_lo + step;
  c = fmaxf(c, 1e-12f);
  const float scale = c / 127.0f;

  for (int col = lane; col < a.cols; col += kWave) {
    float v = w[col];
    v = fminf(fmaxf(v, -c), c);
    float r = v / scale;
    float k = rintf(r);
    float code;
    if (a.bits == 8) {
      code = fminf(fmaxf(k, -127.0f), 127.0f);
    } else {
      float k4 = rintf(k * 0.25f);
      code = fminf(fmaxf(k4 * 4.0f, -128.0f), 124.0f);
    }
    a.codes[row * a.cols + col] = (int8_t)(int)code;
  }
  if (lane == 0) {
    _Float16 h = (_Float16)scale;   // v_cvt_f16_f32: round to nearest even
    a.scales[row] = __builtin_bit_cast(uint16_t, h);
  }
}

}  // namespace

hipError_t launch_quantize(const QuantArgs& a, hipStream_t s) {
  const int rows_per_block = 4;
  int64_t blocks = (a.rows + rows_per_block - 1) / rows_per_block;
  hipLaunchKernelGGL(quantize_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace i6g
