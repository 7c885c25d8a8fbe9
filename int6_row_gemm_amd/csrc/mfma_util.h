// Device helpers shared by the dequant-fused GEMM and the fused block-tail
// kernels: int8 code widening, binary16 packing, and the row / column
// placements that let a lane of a v_mfma_f32_16x16x32_bf16 accumulator own
// runs of consecutive output columns.
#pragma once

#include "common.h"

namespace i6g {

__device__ inline float h2f(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }

// Four int8 codes (one 32-bit word, byte i = code i) widened exactly to
// binary16, two per 32-bit result: with its top bit flipped a code byte is
// u = c + 128; placed under the exponent byte 0x64 it forms the binary16
// value 1024 + u (unit spacing on [1024, 2048)), and one packed subtraction
// of 1152 leaves c.
__device__ inline void widen4h(uint32_t w, uint32_t& lo, uint32_t& hi) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  const h2 bias = {(_Float16)1152.0f, (_Float16)1152.0f};
  const uint32_t u = w ^ 0x80808080u;
  lo = __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2, __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u)) - bias);
  hi = __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2, __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u)) - bias);
}

// leaky_relu(v, slope); slope 0 gives relu (its square is ReLU^2)
__device__ inline float lrelu(float v, float slope) { return v >= 0.0f ? v : slope * v; }

// binary16 bits of f, rounded to nearest even
__device__ inline uint16_t f2h_bits(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }

// two floats as packed binary16 (a in the low half), rounded to nearest
// even by one v_cvt_pk_f16_f32
__device__ inline uint32_t pack2h(float a, float b) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2{a, b}), h2));
}

// Map the launch index to a logical tile so that each XCD (the hardware
// deals workgroups round-robin over 8 XCDs) gets a contiguous range of
// tiles: neighbouring tiles share A rows, which then stay in one L2.
__device__ inline int xcd_remap(int bid, int nblocks) {
  const int q = nblocks / 8, r = nblocks % 8;
  const int xcd = bid % 8, idx = bid / 8;
  return xcd * q + min(xcd, r) + idx;
}

// Within a 64-row slice, row u is stored at perm16(u), which swaps the two
// 2-bit fields u[5:4] and u[3:2] (so perm16 is its own inverse): the MFMA
// fragment of block b, lane row r (physical row 16b + r) then holds logical
// row 16 * (r >> 2) + 4b + (r & 3).
__device__ inline int perm16(int u) { return ((u & 12) << 2) | ((u >> 4) & 3) << 2 | (u & 3); }

// Placement of the weight rows of a 64-column slice for the row-major
// epilogues: output rows 4g + e of fragment j (lane group g) are columns
// 32*(j>>1) + 8g + 4*(j&1) + e, so a lane holds two runs of 8 consecutive
// columns and the four lanes of a row cover 32 consecutive columns of each
// half (one 128-byte line of fp32, or 64 bytes of bf16, per instruction).
__device__ inline int pair_phys(int u) {
  return 16 * (2 * (u >> 5) + ((u >> 2) & 1)) + 4 * ((u >> 3) & 3) + (u & 3);
}

// Inverse of pair_phys on a 32-column slice (pair_phys keeps each half of a
// 64-column slice in place): the logical column stored at physical row p.
__host__ __device__ inline int pair_logical32(int p) {
  return (p & 3) | (((p >> 4) & 1) << 2) | (((p >> 2) & 3) << 3);
}

// Rotation pairs of one q or k head with R rotated dims (partial RoPE):
// pair p < R/2 is (p, p + R/2); the others pair up the unrotated dims as
// (R + w, R + (hd - R)/2 + w), w = p - R/2, and turn by the identity.  For
// R = hd these are the pairs (p, p + hd/2) of full RoPE.
template <int HD>
__host__ __device__ inline int pair_first(int p, int R) { return p < R / 2 ? p : R + (p - R / 2); }
template <int HD>
__host__ __device__ inline int pair_second(int p, int R) {
  return p < R / 2 ? p + R / 2 : R + (HD - R) / 2 + (p - R / 2);
}

// Placement of the rows of one q or k head (HD rows) for the rotary
// epilogue: the output rows 4g + e of fragment j (lane group g) are the
// values t = 4j + e of that lane, and value t < HD/8 is the first dim of
// pair g * HD/8 + t while value t + HD/8 is its second, so a lane holds
// whole rotation pairs, and (R a multiple of HD/4) its first and its second
// dims are two runs of HD/8 consecutive dims.
template <int HD>
__host__ __device__ inline int rope_phys(int u, int R) {
  constexpr int Q8 = HD / 8;
  const int h2 = R / 2, rest2 = (HD - R) / 2;
  int p, second;
  if (u < h2) { p = u; second = 0; }
  else if (u < R) { p = u - h2; second = 1; }
  else if (u < R + rest2) { p = h2 + (u - R); second = 0; }
  else { p = h2 + (u - R - rest2); second = 1; }
  const int t = p % Q8 + second * Q8;
  return 16 * (t >> 2) + 4 * (p / Q8) + (t & 3);
}

// Eight int8 codes (one 8-byte half of a 16-byte fragment chunk) widened to
// the binary16 MFMA operand; exact for integers of magnitude <= 128.
__device__ inline actx8 widen8(uint32_t lo, uint32_t hi) {
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  u32x4_t o;
  uint32_t a0, a1, b0, b1;
  widen4h(lo, a0, a1);
  widen4h(hi, b0, b1);
  o = u32x4_t{a0, a1, b0, b1};
  return __builtin_bit_cast(actx8, o);
}

}  // namespace i6g
