// q/k/v projection on gfx950 MFMA for d_model 512 and head size 64: one
// 128-row tile of the normed layer input per workgroup, all q, k and v heads
// of it (pwwt.cn "parameter-golf 16MB 极限压缩实战 …", 架构: GQA attention with
// RoPE on q and k; one binary16 scale per weight row, 后训练量化导出).
//
// The tile's binary16 rows (128 x 512, 128 KB) go into LDS once by direct
// loads, with the rows' RMS factors and the per-column scales; the eight
// waves then run the per-head loop of qkv_phase.h (the block tail runs the
// same loop on its own output rows).  No barrier after the tile has landed.
//
// rinv = 1/sqrt(sum of the row's partial sums of squares / 512 + eps) is
// applied in fp32 to the accumulators, as in the LDS-staged GEMM, so both
// paths round the same products the same way.
#include "common.h"
#include "mfma_util.h"
#include "qkv_phase.h"

namespace i6g {
namespace {

using qkvp::TM;
using qkvp::DM;
using qkvp::HD;
using qkvp::NW;
using qkvp::MAXN;
constexpr int NTH = 64 * NW;            // threads
constexpr int ABYTES = TM * DM * 2;     // 131072

__device__ inline int phys_row(int r) { return (r & ~63) | perm16(r & 63); }

typedef __attribute__((address_space(1))) void* gptr_t;
typedef __attribute__((address_space(3))) void* lptr_t;

__global__ __launch_bounds__(NTH) __attribute__((amdgpu_waves_per_eu(2, 2))) void qkv_kernel(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) char As[ABYTES];
  __shared__ __attribute__((aligned(16))) float rinv_s[TM];
  __shared__ __attribute__((aligned(16))) float sc_s[MAXN];

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int m0 = xcd_remap(blockIdx.x, gridDim.x) * TM;
  const int nqk = a.n_heads + a.n_kv, nall = nqk + a.n_kv;
  const int N = nall * HD;

  // ---- prologue: the A tile by direct loads into LDS, the per-column
  // scales, the codes of the wave's first K step, the per-row partial sums
  // of squares (one 16-byte load for the four of a d_model 512 row; a loop
  // of dependent loads here, ahead of the tile, had made two waves' share of
  // the tile wait four memory round trips); one wait, then the RMS factors
  // and scales into LDS
  uint4 scv = make_uint4(0, 0, 0, 0);
  if (tid < N / 8) scv = *reinterpret_cast<const uint4*>(a.scale + 8 * tid);
#pragma unroll
  for (int u = 0; u < TM / NW; ++u) {
    const int p = w + NW * u;
    const act* g = a.A + (int64_t)min(m0 + phys_row(p), a.M - 1) * DM + 8 * (lane ^ (2 * (p & 15)));
    __builtin_amdgcn_global_load_lds((gptr_t)g, (lptr_t)(As + p * (DM * 2)), 16, 0, 0);
  }
  uint4 cq0, cq1, cq2, cq3;
  if (w < nall) qkvp::load4(a.Bp, w, 0, cq0, cq1, cq2, cq3);
  float ri = 0.0f;
  if (tid < TM && m0 + tid < a.M) {
    // t / 512 + eps rounded twice, as the LDS-staged GEMM (whose K is not a
    // compile-time constant) computes it: no fused multiply-add; the
    // partial sums added in order, as there
#pragma clang fp contract(off)
    const float* sp = a.ss_in + (int64_t)(m0 + tid) * a.nt_in;
    float t = 0.0f;
    if (a.nt_in == 4) {
      const float4 v = *reinterpret_cast<const float4*>(sp);
      t = t + v.x;
      t = t + v.y;
      t = t + v.z;
      t = t + v.w;
    } else {
      for (int u = 0; u < a.nt_in; ++u) t += sp[u];
    }
    ri = 1.0f / sqrtf(t / (float)DM + a.eps);
  }
  if (tid < TM) rinv_s[tid] = ri;
  if (tid < N / 8) {
    const uint32_t sw[4] = {scv.x, scv.y, scv.z, scv.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sc_s[8 * tid + 2 * e] = h2f((uint16_t)(sw[e] & 0xffff));
      sc_s[8 * tid + 2 * e + 1] = h2f((uint16_t)(sw[e] >> 16));
    }
  }
  __builtin_amdgcn_s_waitcnt(0);   // the direct loads into LDS have landed
  __syncthreads();

  // the lane's tile row in accumulator row block i (C^T: physical row 16 i + lr)

  QkvOut out;
  out.frag = a.Bp; out.scale = a.scale; out.q = a.q; out.k = a.k; out.vt = a.vt; out.rope = a.rope;
  out.n_heads = a.n_heads; out.n_kv = a.n_kv; out.rope_dims = a.rope_dims;
  qkvp::heads(out, a.M, a.Lp, As, rinv_s, sc_s, m0, w, cq0, cq1, cq2, cq3);
}

// Codes of the q/k/v projection [N = (Hq + 2 Hkv) * 64, K] in per-head
// fragment order: 16-byte chunk c is lane c % 64 of fragment (c / 64) % 4 in
// K step (c / 256) % (K / 64) of head c / (256 K / 64); it holds, for the
// head's weight row at fragment row 16 * fragment + lane % 16 (q and k
// heads: the dim rope_phys places there; v heads: that dim), the codes of
// k = 64 * step + 8 * (lane / 16) + 0..7 and the same + 32.
__global__ __launch_bounds__(256) void shuffle_qkv_kernel(const int8_t* __restrict__ B, int32_t n_qk, int32_t n_all,
                                                          int32_t K, int32_t rope_dims, int8_t* __restrict__ Bp) {
  const int nk = K / 64;
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= (int64_t)n_all * nk * 256) return;
  const int lane = (int)(c & 63), j = (int)((c >> 6) & 3);
  const int64_t q = c >> 8;
  const int kt = (int)(q % nk), h = (int)(q / nk);
  const int pr = 16 * j + (lane & 15);
  int u = pr;
  if (h < n_qk)
    for (int v = 0; v < HD; ++v)
      if (rope_phys<HD>(v, rope_dims) == pr) u = v;
  const int8_t* src = B + ((int64_t)h * HD + u) * K + kt * 64 + 8 * (lane >> 4);
  const uint2 lo = *reinterpret_cast<const uint2*>(src);
  const uint2 hi = *reinterpret_cast<const uint2*>(src + 32);
  *reinterpret_cast<uint4*>(Bp + c * 16) = make_uint4(lo.x, lo.y, hi.x, hi.y);
}

}  // namespace

bool qkv_tile_supported(int32_t d, int32_t hd, int32_t n_heads, int32_t n_kv, int32_t rope_dims, int32_t lora_r) {
  const int32_t n = (n_heads + 2 * n_kv) * HD;
  return d == DM && hd == HD && lora_r == 0 && n_heads > 0 && n_kv > 0 && n <= MAXN && rope_dims >= 0 &&
         rope_dims <= HD && rope_dims % (HD / 4) == 0;
}

hipError_t launch_shuffle_qkv_codes(const int8_t* B, int32_t n_heads, int32_t n_kv, int32_t K, int32_t rope_dims,
                                    int8_t* Bp, hipStream_t s) {
  if (!qkv_tile_supported(K, HD, n_heads, n_kv, rope_dims, 0)) return hipErrorInvalidValue;
  const int32_t n_all = n_heads + 2 * n_kv;
  const int64_t chunks = (int64_t)n_all * (K / 64) * 256;
  hipLaunchKernelGGL(shuffle_qkv_kernel, dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, s, B,
                     n_heads + n_kv, n_all, K, rope_dims, Bp);
  return hipGetLastError();
}

hipError_t launch_qkv_tile(const GemmArgs& a, hipStream_t s) {
  if (a.M <= 0) return hipSuccess;
  if (!a.Bp || a.K != DM || a.N != (a.n_heads + 2 * a.n_kv) * HD || a.lora_u || a.Lp < TM || a.Lp % 64 != 0 ||
      a.nt_in < 1 || a.M % 64 != 0 || !qkv_tile_supported(a.K, a.hd, a.n_heads, a.n_kv, a.rope_dims, 0))
    return hipErrorInvalidValue;
  const int tiles = (a.M + TM - 1) / TM;
  hipLaunchKernelGGL(qkv_kernel, dim3(tiles), dim3(NTH), 0, s, a);
  return hipGetLastError();
}

}  // namespace i6g
