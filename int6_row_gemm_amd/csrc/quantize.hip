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

// The code of one weight: clip to [-c, c], divide by the scale, round half
// to even; int8 clamps to [-127, 127], int5 to [-16, 15], int6 rounds again
// to a multiple of 4 and clamps to [-128, 124].
__device__ inline float quant_code(float w, float c, float scale, int bits) {
  const float v = fminf(fmaxf(w, -c), c);
  const float r = v / scale;
  const float k = rintf(r);
  if (bits == 8) return fminf(fmaxf(k, -127.0f), 127.0f);
  if (bits == 5) return fminf(fmaxf(k, -16.0f), 15.0f);
  const float k4 = rintf(k * 0.25f);
  return fminf(fmaxf(k4 * 4.0f, -128.0f), 124.0f);
}

// One row of `cols` fp32 weights -> codes and a binary16 scale, on one
// wavefront (every lane must call it).  Each lane keeps its KT >= topk
// largest |w|; the quantile of every row length these models use needs the
// top two (q < 1) or one (q = 1), so KT = 2 covers them with a quarter of
// the compare work of the general KT = 8.
// VEC (cols a multiple of 4, 16-byte aligned rows): a lane handles four
// consecutive columns at a time, so a wavefront moves 1 KiB per load and
// writes four codes per 32-bit store; otherwise one column per lane.
// FQ: instead of codes and the binary16 scale, write the fake-quantised
// row code * scale (fp32 scale, one rounding) to fq as fp32 or bfloat16.
template <int KT, bool FQ, bool VEC>
__device__ void quantize_row_k(const float* w, int cols, int topk, float frac, int bits, int8_t* codes,
                               uint16_t* scale_out, int32_t* flags, int lane, void* fq, int fq_bf16) {
  // The row is read in chunks of kU elements per lane whose loads are all
  // issued before any is used, so their latencies overlap.
  constexpr int kU = 8;
  constexpr int kV = kU / 4;            // float4 loads per lane per chunk (VEC)
  float top[KT];
#pragma unroll
  for (int i = 0; i < KT; ++i) top[i] = -1.0f;
  int bad = 0;
  for (int c0 = 0; c0 < cols; c0 += kU * kWave) {
    float v[kU];
    if (VEC) {
#pragma unroll
      for (int u = 0; u < kV; ++u) {
        const int c = c0 + 4 * (u * kWave + lane);
        const float4 x = c < cols ? *reinterpret_cast<const float4*>(w + c) : make_float4(0.f, 0.f, 0.f, 0.f);
        v[4 * u] = x.x; v[4 * u + 1] = x.y; v[4 * u + 2] = x.z; v[4 * u + 3] = x.w;
      }
    } else {
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int c = c0 + u * kWave + lane;
        v[u] = c < cols ? w[c] : 0.0f;
      }
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
    if (VEC) {
      float4 wv[kV];
#pragma unroll
      for (int u = 0; u < kV; ++u) {
        const int col = c0 + 4 * (u * kWave + lane);
        wv[u] = col < cols ? *reinterpret_cast<const float4*>(w + col) : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int u = 0; u < kV; ++u) {
        const int col = c0 + 4 * (u * kWave + lane);
        if (col >= cols) continue;
        const float k0 = quant_code(wv[u].x, c, scale, bits), k1 = quant_code(wv[u].y, c, scale, bits);
        const float k2 = quant_code(wv[u].z, c, scale, bits), k3 = quant_code(wv[u].w, c, scale, bits);
        if (FQ) {
          // the codes as integers: a zero code gives +0, as the
          // straight-through sum w + (w_q - w) does
          const float q0 = (float)(int)k0 * scale, q1 = (float)(int)k1 * scale;
          const float q2 = (float)(int)k2 * scale, q3 = (float)(int)k3 * scale;
          if (fq_bf16) {
            typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
            typedef float f32x4_t __attribute__((ext_vector_type(4)));
            const f32x4_t f = {q0, q1, q2, q3};
            *reinterpret_cast<bf16x4_t*>(static_cast<__bf16*>(fq) + col) = __builtin_convertvector(f, bf16x4_t);
          } else {
            *reinterpret_cast<float4*>(static_cast<float*>(fq) + col) = make_float4(q0, q1, q2, q3);
          }
        } else {
          const uint32_t packed = ((uint32_t)(uint8_t)(int)k0) | ((uint32_t)(uint8_t)(int)k1 << 8) |
                                  ((uint32_t)(uint8_t)(int)k2 << 16) | ((uint32_t)(uint8_t)(int)k3 << 24);
          *reinterpret_cast<uint32_t*>(codes + col) = packed;
        }
      }
    } else {
      float wv[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int col = c0 + u * kWave + lane;
        wv[u] = col < cols ? w[col] : 0.0f;
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int col = c0 + u * kWave + lane;
        if (col >= cols) continue;
        const float code = quant_code(wv[u], c, scale, bits);
        if (FQ) {
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

// The vector path needs 16-byte aligned weight rows and 4-byte aligned code
// rows (or 16 / 8 bytes for fake-quantised fp32 / bf16 rows).
__device__ inline bool vec_ok(const float* w, const void* out, int cols, int out_align) {
  return (cols & 3) == 0 && ((uintptr_t)w & 15) == 0 && ((uintptr_t)out & (out_align - 1)) == 0;
}

__device__ inline void quantize_row(const float* w, int cols, int topk, float frac, int bits,
                                    int8_t* codes, uint16_t* scale_out, int32_t* flags, int lane) {
  const bool vec = vec_ok(w, codes, cols, 4);
  if (topk <= 2) {
    if (vec) quantize_row_k<2, false, true>(w, cols, topk, frac, bits, codes, scale_out, flags, lane, nullptr, 0);
    else quantize_row_k<2, false, false>(w, cols, topk, frac, bits, codes, scale_out, flags, lane, nullptr, 0);
  } else {
    if (vec) quantize_row_k<kTop, false, true>(w, cols, topk, frac, bits, codes, scale_out, flags, lane, nullptr, 0);
    else quantize_row_k<kTop, false, false>(w, cols, topk, frac, bits, codes, scale_out, flags, lane, nullptr, 0);
  }
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
  const float* w = a.w + row * a.cols;
  const bool vec = vec_ok(w, out, a.cols, a.fq_bf16 ? 8 : 16);
  if (a.topk <= 2) {
    if (vec) quantize_row_k<2, true, true>(w, a.cols, a.topk, a.frac, a.bits, nullptr, nullptr, a.flags, lane, out, a.fq_bf16);
    else quantize_row_k<2, true, false>(w, a.cols, a.topk, a.frac, a.bits, nullptr, nullptr, a.flags, lane, out, a.fq_bf16);
  } else {
    if (vec) quantize_row_k<kTop, true, true>(w, a.cols, a.topk, a.frac, a.bits, nullptr, nullptr, a.flags, lane, out, a.fq_bf16);
    else quantize_row_k<kTop, true, false>(w, a.cols, a.topk, a.frac, a.bits, nullptr, nullptr, a.flags, lane, out, a.fq_bf16);
  }
}

// Rows of several matrices in one grid; the job of a row is found from the
// (at most kQuantJobs) row offsets, which are in the kernel arguments.
__global__ __launch_bounds__(256) void quantize_many_kernel(QuantManyArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t row = (int64_t)blockIdx.x * (blockDim.x / kWave) + (threadIdx.x / kWave);
  if (row >= a.row0[a.n]) return;
  // job of this row = number of jobs j >= 1 with row0[j] <= row: lane l
  // tests row0[l + 1] and row0[l + 65], so two loads and ballots replace a
  // serial scan
  static_assert(kQuantJobs <= 2 * kWave, "two ballots cover the job table");
  const int64_t n1 = lane + 1 < a.n ? a.row0[lane + 1] : INT64_MAX;
  const int64_t n2 = lane + 1 + kWave < a.n ? a.row0[lane + 1 + kWave] : INT64_MAX;
  const int j = __popcll(__ballot(n1 <= row)) + __popcll(__ballot(n2 <= row));
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
