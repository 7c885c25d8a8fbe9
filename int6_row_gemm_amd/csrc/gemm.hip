// Dequant-fused GEMM on gfx950 MFMA.
//
// C[m, n] = sum_k A[m, k] * code[n, k] with A bf16 [M, K] (activations) and
// code int8 [N, K] (one quantised weight row per output feature, the layout
// of a [out, in] matrix).  The weight of a linear layer is W[n, k] =
// code[n, k] * scale[n] (pwwt.cn "parameter-golf 16MB 极限压缩实战 …",
// 后训练量化导出: one binary16 scale per row), so the scale is a per-column
// factor of C and is applied in the epilogue; the codes (integers in
// [-128, 127]) are exact in bf16 and are widened on their way into LDS.
// When A holds un-normalised activations, the RMSNorm factor of each row
// (a per-row factor of C) is applied in the epilogue as well.
//
// Tiling: 256 threads = 4 waves in a 2 x 2 grid; workgroup tile BM x BN,
// K step 64 through double-buffered LDS with register prefetch; each wave
// issues v_mfma_f32_16x16x32_bf16 on (BM/2) x (BN/2).  The accumulator tile
// is staged through LDS so each epilogue can read rows and columns in the
// order its output layout wants:
//   EPI_QKV   q/k/v projection: * scale * rinv (+ rank-r LoRA), RoPE on the
//             q and k heads, writes Q [W,Hq,Lp,hd], K [W,Hkv,Lp,hd] and
//             V transposed [W,Hkv,hd,Lp] in bf16;
//   EPI_RELU2 MLP up-projection: h = bf16(relu(acc * scale * rinv)^2);
//   EPI_RES   output / down projection: x += acc * scale, then the skip
//             push/pop of the block schedule, and bf16(x) plus per-tile
//             sums of x^2 for the next normed GEMM.
#include "common.h"

namespace i6g {
namespace {

constexpr int BK = 64;
constexpr int LDK = BK + 8;  // LDS row stride in bf16 elements

__device__ inline float h2f(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

__device__ inline uint32_t pack_bf16x2_from_int(int lo, int hi) {
  // integers of magnitude <= 128 are exact in fp32 and keep only 8
  // significant bits, so the upper half of the fp32 pattern is the bf16.
  uint32_t a = __builtin_bit_cast(uint32_t, (float)lo);
  uint32_t b = __builtin_bit_cast(uint32_t, (float)hi);
  return (a >> 16) | (b & 0xffff0000u);
}

__device__ inline uint16_t f2bf_bits(float f) {
  return __builtin_bit_cast(uint16_t, (bf16)f);
}

// Map the launch index to a logical tile so that each XCD (the hardware
// deals workgroups round-robin over 8 XCDs) gets a contiguous range of
// tiles: neighbouring tiles share A rows, which then stay in one L2.
__device__ inline int xcd_remap(int bid, int nblocks) {
  const int q = nblocks / 8, r = nblocks % 8;
  const int xcd = bid % 8, idx = bid / 8;
  return xcd * q + min(xcd, r) + idx;
}

template <int BM, int BN>
struct Smem {
  static constexpr int kAB = 2 * (BM + BN) * LDK * 2;
  static constexpr int kC = BM * (BN + 4) * 4;
  static constexpr int kBytes = kAB > kC ? kAB : kC;
};

template <int BM, int BN, int EPI>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs a) {
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int FM = WM / 16, FN = WN / 16;
  constexpr int A_CHUNKS = BM * BK / 8;       // 16-byte chunks of bf16
  constexpr int B_CHUNKS = BN * BK / 16;      // 16-byte chunks of int8
  constexpr int A_PER = (A_CHUNKS + 255) / 256;
  constexpr int B_PER = (B_CHUNKS + 255) / 256;
  constexpr int CLD = BN + 4;

  __shared__ __attribute__((aligned(16))) char smem[Smem<BM, BN>::kBytes];
  __shared__ float rinv_s[BM];
  bf16* As = reinterpret_cast<bf16*>(smem);
  bf16* Bs = As + 2 * BM * LDK;
  float* Cs = reinterpret_cast<float*>(smem);

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int ntn = a.N / BN;
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int tm = tile / ntn, tn = tile % ntn;
  const int m0 = tm * BM, n0 = tn * BN;

  if constexpr (EPI == EPI_QKV || EPI == EPI_RELU2) {
    for (int r = tid; r < BM; r += 256) {
      int m = m0 + r;
      float v = 0.0f;
      if (m < a.M) {
        float ss = 0.0f;
        for (int t = 0; t < a.nt_in; ++t) ss += a.ss_in[(int64_t)m * a.nt_in + t];
        v = 1.0f / sqrtf(ss / (float)a.K + a.eps);
      }
      rinv_s[r] = v;
    }
  }

  uint4 areg[A_PER];
  uint4 breg[B_PER];
  const int nk = a.K / BK;

  auto load_global = [&](int kt) {
    const int k0 = kt * BK;
#pragma unroll
    for (int i = 0; i < A_PER; ++i) {
      int c = tid + i * 256;
      areg[i] = make_uint4(0, 0, 0, 0);
      if (c < A_CHUNKS) {
        int r = c >> 3, cc = (c & 7) * 8;
        int m = m0 + r;
        if (m < a.M)
          areg[i] = *reinterpret_cast<const uint4*>(a.A + (int64_t)m * a.K + k0 + cc);
      }
    }
#pragma unroll
    for (int i = 0; i < B_PER; ++i) {
      int c = tid + i * 256;
      if (c < B_CHUNKS) {
        int r = c >> 2, cc = (c & 3) * 16;
        breg[i] = *reinterpret_cast<const uint4*>(a.B + (int64_t)(n0 + r) * a.K + k0 + cc);
      }
    }
  };

  auto store_lds = [&](int buf) {
    bf16* as = As + buf * BM * LDK;
    bf16* bs = Bs + buf * BN * LDK;
#pragma unroll
    for (int i = 0; i < A_PER; ++i) {
      int c = tid + i * 256;
      if (c < A_CHUNKS) {
        int r = c >> 3, cc = (c & 7) * 8;
        *reinterpret_cast<uint4*>(as + r * LDK + cc) = areg[i];
      }
    }
#pragma unroll
    for (int i = 0; i < B_PER; ++i) {
      int c = tid + i * 256;
      if (c < B_CHUNKS) {
        int r = c >> 2, cc = (c & 3) * 16;
        const uint32_t w[4] = {breg[i].x, breg[i].y, breg[i].z, breg[i].w};
        uint32_t o[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          int b0 = (int)(int8_t)(w[j] & 0xff);
          int b1 = (int)(int8_t)((w[j] >> 8) & 0xff);
          int b2 = (int)(int8_t)((w[j] >> 16) & 0xff);
          int b3 = (int)(int8_t)(w[j] >> 24);
          o[2 * j] = pack_bf16x2_from_int(b0, b1);
          o[2 * j + 1] = pack_bf16x2_from_int(b2, b3);
        }
        uint4* dst = reinterpret_cast<uint4*>(bs + r * LDK + cc);
        dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
        dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
      }
    }
  };

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  load_global(0);
  store_lds(0);
  __syncthreads();

  const int lr = lane & 15, lk = (lane >> 4) * 8;
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load_global(kt + 1);
    const bf16* as = As + buf * BM * LDK;
    const bf16* bs = Bs + buf * BN * LDK;
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      bf16x8 af[FM], bfg[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        af[i] = *reinterpret_cast<const bf16x8*>(as + (wm * WM + i * 16 + lr) * LDK + ks * 32 + lk);
#pragma unroll
      for (int j = 0; j < FN; ++j)
        bfg[j] = *reinterpret_cast<const bf16x8*>(bs + (wn * WN + j * 16 + lr) * LDK + ks * 32 + lk);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfg[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) store_lds(buf ^ 1);
    __syncthreads();
  }

  // Stage the accumulators: lane holds column (lane & 15), rows 4*(lane>>4)+e.
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        int r = wm * WM + i * 16 + (lane >> 4) * 4 + e;
        int c = wn * WN + j * 16 + (lane & 15);
        Cs[r * CLD + c] = acc[i][j][e];
      }
  __syncthreads();

  if constexpr (EPI == EPI_RELU2) {
    constexpr int UPR = BN / 8;
    for (int u = tid; u < BM * UPR; u += 256) {
      int r = u / UPR, c8 = (u % UPR) * 8;
      int m = m0 + r;
      if (m >= a.M) continue;
      float ri = rinv_s[r];
      uint32_t o[4];
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        float v0 = Cs[r * CLD + c8 + e] * h2f(a.scale[n0 + c8 + e]) * ri;
        float v1 = Cs[r * CLD + c8 + e + 1] * h2f(a.scale[n0 + c8 + e + 1]) * ri;
        v0 = fmaxf(v0, 0.0f); v1 = fmaxf(v1, 0.0f);
        v0 = v0 * v0; v1 = v1 * v1;
        o[e / 2] = (uint32_t)f2bf_bits(v0) | ((uint32_t)f2bf_bits(v1) << 16);
      }
      *reinterpret_cast<uint4*>(a.h + (int64_t)m * a.N + n0 + c8) = make_uint4(o[0], o[1], o[2], o[3]);
    }
  } else if constexpr (EPI == EPI_RES) {
    constexpr int UPR = BN / 8;   // 16 threads per row for BN = 128
    static_assert(BN == 128, "residual epilogue assumes 128-column tiles");
    for (int u = tid; u < BM * UPR; u += 256) {
      int r = u / UPR, c8 = (u % UPR) * 8;
      int m = m0 + r;
      bool ok = m < a.M;
      float sq = 0.0f;
      if (ok) {
        int64_t off = (int64_t)m * a.N + n0 + c8;
        float xn[8];
        const float4* xp = reinterpret_cast<const float4*>(a.x + off);
        float4 x0 = xp[0], x1 = xp[1];
        float xo[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e)
          xn[e] = xo[e] + Cs[r * CLD + c8 + e] * h2f(a.scale[n0 + c8 + e]);
        if (a.push_dst) {
          float4* pd = reinterpret_cast<float4*>(a.push_dst + off);
          pd[0] = make_float4(xn[0], xn[1], xn[2], xn[3]);
          pd[1] = make_float4(xn[4], xn[5], xn[6], xn[7]);
        }
        if (a.pop_src) {
          float pv[8];
          if (a.pop_src == a.push_dst) {
#pragma unroll
            for (int e = 0; e < 8; ++e) pv[e] = xn[e];
          } else {
            const float4* pp = reinterpret_cast<const float4*>(a.pop_src + off);
            float4 p0 = pp[0], p1 = pp[1];
            pv[0] = p0.x; pv[1] = p0.y; pv[2] = p0.z; pv[3] = p0.w;
            pv[4] = p1.x; pv[5] = p1.y; pv[6] = p1.z; pv[7] = p1.w;
          }
#pragma unroll
          for (int e = 0; e < 8; ++e) xn[e] += a.pop_w[n0 + c8 + e] * pv[e];
        }
        float4* xw = reinterpret_cast<float4*>(a.x + off);
        xw[0] = make_float4(xn[0], xn[1], xn[2], xn[3]);
        xw[1] = make_float4(xn[4], xn[5], xn[6], xn[7]);
        if (a.xb) {
          uint32_t o[4];
#pragma unroll
          for (int e = 0; e < 8; e += 2)
            o[e / 2] = (uint32_t)f2bf_bits(xn[e]) | ((uint32_t)f2bf_bits(xn[e + 1]) << 16);
          *reinterpret_cast<uint4*>(a.xb + off) = make_uint4(o[0], o[1], o[2], o[3]);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) sq += xn[e] * xn[e];
      }
      // 16 consecutive lanes hold one row: reduce their partial sums.
      sq += __shfl_xor(sq, 1);
      sq += __shfl_xor(sq, 2);
      sq += __shfl_xor(sq, 4);
      sq += __shfl_xor(sq, 8);
      if (ok && a.ss_out && (u % UPR) == 0) a.ss_out[(int64_t)m * (a.N / 128) + tn] = sq;
    }
  } else {  // EPI_QKV
    const int hd = a.hd, half = hd / 2;
    const int dq = a.n_heads * hd, dkv = a.n_kv * hd;
    if (n0 < dq + dkv) {
      // q or k heads: units of (row, head in tile, 4 rotation pairs)
      const bool is_q = n0 < dq;
      const int heads_in_tile = BN / hd;
      const int cpr = half / 4;                 // pair chunks per head
      const int upr = heads_in_tile * cpr;      // units per row
      for (int u = tid; u < BM * upr; u += 256) {
        int r = u / upr, rem = u % upr;
        int hh = rem / cpr, i0 = (rem % cpr) * 4;
        int m = m0 + r;
        if (m >= a.M) continue;
        float ri = rinv_s[r];
        int w = m / a.Lp, pos = m % a.Lp;
        int cbase = hh * hd;
        float x1[4], x2[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          int c1 = cbase + i0 + e, c2 = c1 + half;
          x1[e] = Cs[r * CLD + c1] * h2f(a.scale[n0 + c1]) * ri;
          x2[e] = Cs[r * CLD + c2] * h2f(a.scale[n0 + c2]) * ri;
        }
        if (is_q && a.lora_u) {
          const float* uu = a.lora_u + (int64_t)m * 2 * a.lora_r;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            int g1 = n0 + cbase + i0 + e, g2 = g1 + half;
            float s1 = 0.f, s2 = 0.f;
            for (int t = 0; t < a.lora_r; ++t) {
              s1 += uu[t] * a.lora_bq[g1 * a.lora_r + t];
              s2 += uu[t] * a.lora_bq[g2 * a.lora_r + t];
            }
            x1[e] += s1; x2[e] += s2;
          }
        }
        uint16_t y1[4], y2[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float2 cs = a.rope[pos * half + i0 + e];
          float a1 = x1[e] * cs.x - x2[e] * cs.y;
          float a2 = x1[e] * cs.y + x2[e] * cs.x;
          y1[e] = f2bf_bits(a1);
          y2[e] = f2bf_bits(a2);
        }
        int head = (is_q ? n0 : n0 - dq) / hd + hh;
        int nh = is_q ? a.n_heads : a.n_kv;
        bf16* dst = (is_q ? a.q : a.k) + (((int64_t)w * nh + head) * a.Lp + pos) * hd;
        uint2 p1 = make_uint2((uint32_t)y1[0] | ((uint32_t)y1[1] << 16), (uint32_t)y1[2] | ((uint32_t)y1[3] << 16));
        uint2 p2 = make_uint2((uint32_t)y2[0] | ((uint32_t)y2[1] << 16), (uint32_t)y2[2] | ((uint32_t)y2[3] << 16));
        *reinterpret_cast<uint2*>(dst + i0) = p1;
        *reinterpret_cast<uint2*>(dst + half + i0) = p2;
      }
    } else {
      // v heads, written transposed: units of (column, 8 consecutive rows)
      const int rcs = BM / 8;
      for (int u = tid; u < BN * rcs; u += 256) {
        int rc = u % rcs, c = u / rcs;
        int r0 = rc * 8;
        int m = m0 + r0;
        if (m >= a.M) continue;          // M is a multiple of 8
        int nv = n0 + c - dq - dkv;      // column inside the v block
        int head = nv / hd, dd = nv % hd;
        float sc = h2f(a.scale[n0 + c]);
        uint16_t y[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float v = Cs[(r0 + e) * CLD + c] * sc * rinv_s[r0 + e];
          if (a.lora_u) {
            const float* uu = a.lora_u + (int64_t)(m + e) * 2 * a.lora_r + a.lora_r;
            float s = 0.f;
            for (int t = 0; t < a.lora_r; ++t) s += uu[t] * a.lora_bv[nv * a.lora_r + t];
            v += s;
          }
          y[e] = f2bf_bits(v);
        }
        int w = m / a.Lp, pos = m % a.Lp;
        bf16* dst = a.vt + (((int64_t)w * a.n_kv + head) * hd + dd) * a.Lp + pos;
        *reinterpret_cast<uint4*>(dst) = make_uint4(
            (uint32_t)y[0] | ((uint32_t)y[1] << 16), (uint32_t)y[2] | ((uint32_t)y[3] << 16),
            (uint32_t)y[4] | ((uint32_t)y[5] << 16), (uint32_t)y[6] | ((uint32_t)y[7] << 16));
      }
    }
  }
}

template <int BM, int BN, int EPI>
hipError_t run(const GemmArgs& a, hipStream_t s) {
  int tiles = ((a.M + BM - 1) / BM) * (a.N / BN);
  hipLaunchKernelGGL((gemm_kernel<BM, BN, EPI>), dim3(tiles), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(int epi, const GemmArgs& a, hipStream_t s) {
  switch (epi) {
    case EPI_QKV:
      if (a.hd == 32) return run<128, 64, EPI_QKV>(a, s);
      if (a.hd == 64) return run<128, 128, EPI_QKV>(a, s);
      if (a.hd == 80) return run<128, 160, EPI_QKV>(a, s);
      return hipErrorInvalidValue;
    case EPI_RELU2:
      return run<128, 128, EPI_RELU2>(a, s);
    case EPI_RES:
      return run<128, 128, EPI_RES>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace i6g
