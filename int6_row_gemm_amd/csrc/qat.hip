// Noisy-QAT weights: each row plus uniform noise of one quantisation step.
//
// kwkr.cn write-up of parameter-golf PR #363, Noisy QAT: the forward adds
// (U[0, 1) - 0.5) * step to every weight, step = the row's absolute maximum
// (floored at 1e-12) / 127 -- or / 15 to match an int5 export, as the
// write-up's closing notes suggest.  The uniform numbers come from
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as
// easy as 1, 2, 3", SC 2011): key = the 64-bit seed, counter = (element
// index / 4 as 64 bits, 0, 0), word = element index % 4, U = (word >> 8) *
// 2^-24.  A counter-based generator needs no state and no random array in
// memory: every element's number is a pure function of its index.
//
// One wavefront per row: a first pass over the row finds the absolute
// maximum, a second adds the noise.  Each lane handles four consecutive
// elements, which share one Philox block, when the row length is a multiple
// of 4 (then every four-element group starts at an index divisible by 4);
// otherwise one element per lane.  All fp32 operations are rounded one at a
// time (no contraction into FMA), as the noise definition is written.
#include "common.h"

#pragma clang fp contract(off)

namespace i6g {
namespace {

constexpr uint32_t kM0 = 0xD2511F53u, kM1 = 0xCD9E8D57u;   // Philox4x32 multipliers
constexpr uint32_t kW0 = 0x9E3779B9u, kW1 = 0xBB67AE85u;   // key increments

__device__ inline uint4 philox4x32_10(uint4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += kW0;
      k1 += kW1;
    }
    const uint32_t hi0 = __umulhi(kM0, c.x), lo0 = kM0 * c.x;
    const uint32_t hi1 = __umulhi(kM1, c.z), lo1 = kM1 * c.z;
    c = make_uint4(hi1 ^ c.y ^ k0, lo1, hi0 ^ c.w ^ k1, lo0);
  }
  return c;
}

__device__ inline float uniform24(uint32_t x) { return (float)(x >> 8) * 0x1p-24f; }

__device__ inline float noisy(float w, uint32_t x, float step) {
  const float n = (uniform24(x) - 0.5f) * step;
  return w + n;
}

__device__ inline float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

__global__ __launch_bounds__(256) void noisy_kernel(NoisyArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t row = (int64_t)blockIdx.x * (blockDim.x / kWave) + (threadIdx.x / kWave);
  if (row >= a.rows) return;
  const int cols = a.cols;
  const float* w = a.w + row * cols;
  const bool vec = (cols & 3) == 0;

  float m = 0.0f;
  bool bad = false;
  if (vec) {
    for (int c = 4 * lane; c < cols; c += 4 * kWave) {
      const float4 v = *reinterpret_cast<const float4*>(w + c);
      bad |= !isfinite(v.x) || !isfinite(v.y) || !isfinite(v.z) || !isfinite(v.w);
      m = fmaxf(m, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
    }
  } else {
    for (int c = lane; c < cols; c += kWave) {
      const float v = w[c];
      bad |= !isfinite(v);
      m = fmaxf(m, fabsf(v));
    }
  }
  m = wave_max(m);
  if (__any(bad)) {
    // a row with NaN or Inf: every output of the row is NaN
    for (int c = lane; c < cols; c += kWave) {
      if (a.out_bf16) static_cast<uint16_t*>(a.out)[row * cols + c] = 0x7FC0;
      else static_cast<float*>(a.out)[row * cols + c] = __builtin_nanf("");
    }
    if (lane == 0 && a.flags) atomicOr(a.flags, 1);
    return;
  }
  const float step = fmaxf(m, 1e-12f) / a.levels;   // correctly rounded division

  const uint64_t base = (uint64_t)row * (uint64_t)cols;
  if (vec) {
    for (int c = 4 * lane; c < cols; c += 4 * kWave) {
      const float4 v = *reinterpret_cast<const float4*>(w + c);
      const uint64_t q = (base + c) >> 2;
      const uint4 x = philox4x32_10(make_uint4((uint32_t)q, (uint32_t)(q >> 32), 0u, 0u), a.key0, a.key1);
      const float o0 = noisy(v.x, x.x, step), o1 = noisy(v.y, x.y, step);
      const float o2 = noisy(v.z, x.z, step), o3 = noisy(v.w, x.w, step);
      if (a.out_bf16) {
        typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
        typedef float f32x4_t __attribute__((ext_vector_type(4)));
        const f32x4_t f = {o0, o1, o2, o3};
        *reinterpret_cast<bf16x4_t*>(static_cast<__bf16*>(a.out) + base + c) = __builtin_convertvector(f, bf16x4_t);
      } else {
        *reinterpret_cast<float4*>(static_cast<float*>(a.out) + base + c) = make_float4(o0, o1, o2, o3);
      }
    }
  } else {
    for (int c = lane; c < cols; c += kWave) {
      const uint64_t i = base + c;
      const uint4 x = philox4x32_10(make_uint4((uint32_t)(i >> 2), (uint32_t)(i >> 34), 0u, 0u), a.key0, a.key1);
      const uint32_t word = (i & 3) == 0 ? x.x : (i & 3) == 1 ? x.y : (i & 3) == 2 ? x.z : x.w;
      const float o = noisy(w[c], word, step);
      if (a.out_bf16) static_cast<__bf16*>(a.out)[i] = (__bf16)o;
      else static_cast<float*>(a.out)[i] = o;
    }
  }
}

}  // namespace

hipError_t launch_noisy_weights(const NoisyArgs& a, hipStream_t s) {
  const int rows_per_block = 4;
  const int64_t blocks = (a.rows + rows_per_block - 1) / rows_per_block;
  hipLaunchKernelGGL(noisy_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace i6g
