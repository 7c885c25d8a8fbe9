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
// K step 64 through double-buffered, XOR-swizzled LDS with register prefetch
// two K steps ahead; each wave
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
constexpr int LDK = BK;      // LDS row stride in bf16 elements (128 bytes)

// LDS tiles keep 128-byte rows of eight 16-byte chunks; chunk j of row r is
// stored in slot j ^ ((r >> 1) & 7).  Measured on gfx950, this makes both the
// MFMA fragment reads (16 rows, one chunk each) and the staging writes free of
// bank conflicts, where a 16-byte row padding costs a two-way conflict.
__device__ inline int swz(int row, int chunk) { return chunk ^ ((row >> 1) & 7); }

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
  static constexpr int kAB = (BM + BN) * LDK * 2;        // one A and one B tile
  static constexpr int kC = (BM / 2) * (BN + 4) * 4;     // half of the accumulator tile
  static constexpr int kBytes = kAB > kC ? kAB : kC;
};

template <int BM, int BN, int EPI>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(BN <= 128 ? 3 : 2)))
void gemm_kernel(GemmArgs a) {
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int FM = WM / 16, FN = WN / 16;
  constexpr int A_CHUNKS = BM * BK / 8;       // 16-byte chunks of bf16
  constexpr int B_CHUNKS = BN * BK / 16;      // 16-byte chunks of int8
  constexpr int A_PER = (A_CHUNKS + 255) / 256;
  constexpr int B_PER = (B_CHUNKS + 255) / 256;
  constexpr int CLD = BN + 4;

  __shared__ __attribute__((aligned(16))) char smem[Smem<BM, BN>::kBytes];
  __shared__ float rinv_s[BM];
  __shared__ float scale_s[BN];
  __shared__ float popw_s[BN];
  bf16* As = reinterpret_cast<bf16*>(smem);
  bf16* Bs = As + BM * LDK;
  float* Cs = reinterpret_cast<float*>(smem);

  const int tid = threadIdx.x & 255;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int ntn = a.N / BN;
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int tm = tile / ntn, tn = tile % ntn;
  const int m0 = tm * BM, n0 = tn * BN;

  for (int c = tid; c < BN; c += 256) {
    scale_s[c] = h2f(a.scale[n0 + c]);
    if constexpr (EPI == EPI_RES) popw_s[c] = a.pop_w ? a.pop_w[n0 + c] : 0.0f;
  }
  if constexpr (EPI == EPI_QKV || EPI == EPI_RELU2) {
    for (int r = tid; r < BM; r += 256) {
      int m = m0 + r;
      float v = 0.0f;
      if (m < a.M) {
        const int64_t mr = a.a_map ? scored_row(a.p0 + m, a.k0, a.n_win, a.e0, a.L, a.S, a.Lp) : m;
        float ss = 0.0f;
        for (int t = 0; t < a.nt_in; ++t) ss += a.ss_in[mr * a.nt_in + t];
        v = 1.0f / sqrtf(ss / (float)a.K + a.eps);
      }
      rinv_s[r] = v;
    }
  }

  // Global -> register staging, prefetched two K tiles ahead into two sets
  // of named scalars (arrays of them end up in scratch memory).  Chunk
  // indices past the tile are clamped (those threads reload and rewrite the
  // last chunk with identical data); A rows past M are clamped to M - 1 and
  // their results are never stored.
  static_assert(A_PER <= 4 && B_PER <= 3, "staging holds 4 A and 3 B chunks per thread");
  uint4 sa0_0, sa0_1, sa0_2, sa0_3, sb0_0, sb0_1, sb0_2;
  uint4 sa1_0, sa1_1, sa1_2, sa1_3, sb1_0, sb1_1, sb1_2;
  const int nk = a.K / BK;
  // element offset of each A row this thread loads, for the whole K loop
  int64_t arow0 = 0, arow1 = 0, arow2 = 0, arow3 = 0;
#define GM_AROW(i, V)                                                                 \
  if constexpr (A_PER > i) {                                                          \
    const int c = min(tid + (i) * 256, A_CHUNKS - 1);                                 \
    const int m = min(m0 + (c >> 3), a.M - 1);                                        \
    V = (a.a_map ? scored_row(a.p0 + m, a.k0, a.n_win, a.e0, a.L, a.S, a.Lp) : m) * (int64_t)a.K; \
  }
  GM_AROW(0, arow0) GM_AROW(1, arow1) GM_AROW(2, arow2) GM_AROW(3, arow3)
#undef GM_AROW

#define GM_A(i, R)                                                                    \
  if constexpr (A_PER > i) {                                                          \
    int c = min(tid + (i) * 256, A_CHUNKS - 1);                                       \
    R = *reinterpret_cast<const uint4*>(a.A + arow##i + k0_ + (c & 7) * 8);           \
  }
#define GM_B(i, R)                                                                    \
  if constexpr (B_PER > i) {                                                          \
    int c = min(tid + (i) * 256, B_CHUNKS - 1);                                       \
    R = *reinterpret_cast<const uint4*>(a.B + (int64_t)(n0 + (c >> 2)) * a.K + k0_ + (c & 3) * 16); \
  }
#define GM_LOAD(kt, S)                                                                \
  {                                                                                   \
    const int k0_ = (kt) * BK;                                                        \
    GM_A(0, sa##S##_0) GM_A(1, sa##S##_1) GM_A(2, sa##S##_2) GM_A(3, sa##S##_3)       \
    GM_B(0, sb##S##_0) GM_B(1, sb##S##_1) GM_B(2, sb##S##_2)                          \
  }
#define GM_SA(i, R, as)                                                               \
  if constexpr (A_PER > i) {                                                          \
    int c = min(tid + (i) * 256, A_CHUNKS - 1);                                       \
    *reinterpret_cast<uint4*>(as + (c >> 3) * LDK + swz(c >> 3, c & 7) * 8) = R;      \
  }
#define GM_SB(i, R, bs)                                                               \
  if constexpr (B_PER > i) {                                                          \
    int c = min(tid + (i) * 256, B_CHUNKS - 1);                                       \
    const uint32_t w_[4] = {R.x, R.y, R.z, R.w};                                      \
    uint32_t o_[8];                                                                   \
    _Pragma("unroll") for (int j = 0; j < 4; ++j) {                                   \
      o_[2 * j] = pack_bf16x2_from_int((int)(int8_t)(w_[j] & 0xff), (int)(int8_t)((w_[j] >> 8) & 0xff)); \
      o_[2 * j + 1] = pack_bf16x2_from_int((int)(int8_t)((w_[j] >> 16) & 0xff), (int)(int8_t)(w_[j] >> 24)); \
    }                                                                                 \
    const int r_ = c >> 2, j_ = (c & 3) * 2;                                          \
    *reinterpret_cast<uint4*>(bs + r_ * LDK + swz(r_, j_) * 8) = make_uint4(o_[0], o_[1], o_[2], o_[3]); \
    *reinterpret_cast<uint4*>(bs + r_ * LDK + swz(r_, j_ + 1) * 8) = make_uint4(o_[4], o_[5], o_[6], o_[7]); \
  }
#define GM_STORE(S)                                                                   \
  {                                                                                   \
    bf16* as_ = As;                                                                   \
    bf16* bs_ = Bs;                                                                   \
    GM_SA(0, sa##S##_0, as_) GM_SA(1, sa##S##_1, as_) GM_SA(2, sa##S##_2, as_) GM_SA(3, sa##S##_3, as_) \
    GM_SB(0, sb##S##_0, bs_) GM_SB(1, sb##S##_1, bs_) GM_SB(2, sb##S##_2, bs_)        \
  }

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int lr = lane & 15, lg = lane >> 4;
#define GM_COMPUTE()                                                                  \
  {                                                                                   \
    const bf16* as = As;                                                              \
    const bf16* bs = Bs;                                                              \
    _Pragma("unroll") for (int ks = 0; ks < BK / 32; ++ks) {                          \
      bf16x8 af[FM], bfg[FN];                                                         \
      _Pragma("unroll") for (int i = 0; i < FM; ++i) {                                \
        const int r_ = wm * WM + i * 16 + lr;                                         \
        af[i] = *reinterpret_cast<const bf16x8*>(as + r_ * LDK + swz(r_, ks * 4 + lg) * 8); \
      }                                                                               \
      _Pragma("unroll") for (int j = 0; j < FN; ++j) {                                \
        const int r_ = wn * WN + j * 16 + lr;                                         \
        bfg[j] = *reinterpret_cast<const bf16x8*>(bs + r_ * LDK + swz(r_, ks * 4 + lg) * 8); \
      }                                                                               \
      _Pragma("unroll") for (int i = 0; i < FM; ++i)                                  \
        _Pragma("unroll") for (int j = 0; j < FN; ++j)                                \
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfg[j], acc[i][j], 0, 0, 0); \
    }                                                                                 \
  }
  // One K tile: issue the loads of tile kt+2 into register set L, multiply
  // tile kt out of LDS, then replace it with tile kt+1 (set S, loaded one
  // step earlier).  A single LDS tile keeps the footprint small enough for
  // three workgroups per CU, whose epilogue stores then overlap the others'
  // MFMA work.
#define GM_STEP(kt, L, S)                                                             \
  {                                                                                   \
    GM_LOAD(min((kt) + 2, nk - 1), L);                                                \
    GM_COMPUTE();                                                                     \
    if ((kt) + 1 < nk) {                                                              \
      __syncthreads();                                                                \
      GM_STORE(S);                                                                    \
      __syncthreads();                                                                \
    }                                                                                 \
  }

  GM_LOAD(0, 0);
  GM_STORE(0);
  GM_LOAD(min(1, nk - 1), 1);
  __syncthreads();
  for (int kt = 0; kt < nk; kt += 2) {
    GM_STEP(kt, 0, 1);
    if (kt + 1 < nk) GM_STEP(kt + 1, 1, 0);
  }
#undef GM_STEP
#undef GM_COMPUTE
#undef GM_STORE
#undef GM_SB
#undef GM_SA
#undef GM_LOAD
#undef GM_B
#undef GM_A

  // The accumulator tile goes through LDS in two halves of BM/2 rows (the
  // rows of wave row wm == h); lane holds column (lane & 15) and rows
  // 4*(lane>>4)+e of each 16 x 16 block.
  constexpr int HR = BM / 2;
  __syncthreads();
#pragma unroll
  for (int h = 0; h < 2; ++h) {
  const int hr0 = h * HR;
  if (wm == h) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          int r = i * 16 + (lane >> 4) * 4 + e;
          int c = wn * WN + j * 16 + (lane & 15);
          Cs[r * CLD + c] = acc[i][j][e];
        }
  }
  __syncthreads();

  // Epilogues: each unit of work is 8 consecutive outputs; the unit loops
  // have compile-time trip counts and are unrolled so their global loads
  // are all in flight together.
  if constexpr (EPI == EPI_RELU2) {
    constexpr int UPR = BN / 8;
    static_assert((HR * UPR) % 256 == 0, "unit count");
#pragma unroll
    for (int it = 0; it < HR * UPR / 256; ++it) {
      const int u = tid + it * 256;
      const int r = u / UPR, c8 = (u % UPR) * 8;
      const int m = m0 + hr0 + r;
      if (m >= a.M) continue;
      const float ri = rinv_s[hr0 + r];
      uint32_t o[4];
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        float v0 = fmaxf(Cs[r * CLD + c8 + e] * scale_s[c8 + e] * ri, 0.0f);
        float v1 = fmaxf(Cs[r * CLD + c8 + e + 1] * scale_s[c8 + e + 1] * ri, 0.0f);
        o[e / 2] = (uint32_t)f2bf_bits(v0 * v0) | ((uint32_t)f2bf_bits(v1 * v1) << 16);
      }
      *reinterpret_cast<uint4*>(a.h + (int64_t)m * a.N + n0 + c8) = make_uint4(o[0], o[1], o[2], o[3]);
    }
  } else if constexpr (EPI == EPI_RES) {
    constexpr int UPR = BN / 8;   // 16 consecutive lanes hold one row
    static_assert(BN == 128, "residual epilogue assumes 128-column tiles");
    const bool push = a.push_dst != nullptr;
    const bool pop = a.pop_src != nullptr;
    const bool pop_self = pop && a.pop_src == a.push_dst;
#pragma unroll
    for (int it = 0; it < HR * UPR / 256; ++it) {
      const int u = tid + it * 256;
      const int r = u / UPR, c8 = (u % UPR) * 8;
      const int m = min(m0 + hr0 + r, a.M - 1);  // rows past M recompute row M-1, store nothing
      const bool ok = m0 + hr0 + r < a.M;
      const int64_t mr = a.e_map ? scored_row(a.p0 + m, a.k0, a.n_win, a.e0, a.L, a.S, a.Lp) : m;
      const int64_t off = mr * a.N + n0 + c8;
      const float4* xp = reinterpret_cast<const float4*>(a.x + off);
      const float4 x0 = xp[0], x1 = xp[1];
      float xn[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) xn[e] += Cs[r * CLD + c8 + e] * scale_s[c8 + e];
      if (push && ok) {
        float4* pd = reinterpret_cast<float4*>(a.push_dst + off);
        pd[0] = make_float4(xn[0], xn[1], xn[2], xn[3]);
        pd[1] = make_float4(xn[4], xn[5], xn[6], xn[7]);
      }
      if (pop) {
        float pv[8];
        if (pop_self) {
#pragma unroll
          for (int e = 0; e < 8; ++e) pv[e] = xn[e];
        } else {
          const float4* pp = reinterpret_cast<const float4*>(a.pop_src + off);
          const float4 p0 = pp[0], p1 = pp[1];
          pv[0] = p0.x; pv[1] = p0.y; pv[2] = p0.z; pv[3] = p0.w;
          pv[4] = p1.x; pv[5] = p1.y; pv[6] = p1.z; pv[7] = p1.w;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) xn[e] += popw_s[c8 + e] * pv[e];
      }
      float sq = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) sq += xn[e] * xn[e];
      if (ok) {
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
      }
      sq += __shfl_xor(sq, 1);
      sq += __shfl_xor(sq, 2);
      sq += __shfl_xor(sq, 4);
      sq += __shfl_xor(sq, 8);
      if (ok && a.ss_out && (u % UPR) == 0) a.ss_out[mr * (a.N / 128) + tn] = sq;
    }
  } else {  // EPI_QKV: BN = 2 * head_dim, so a tile holds two whole heads
    constexpr int HDT = BN / 2, HALF = HDT / 2;
    const int dq = a.n_heads * HDT, dkv = a.n_kv * HDT;
    if (n0 < dq + dkv) {
      // q or k heads: units of (row, head in tile, 4 rotation pairs)
      const bool is_q = n0 < dq;
      constexpr int CPR = HALF / 4;             // pair chunks per head
      constexpr int UPR = 2 * CPR;              // units per row
      static_assert((HR * UPR) % 256 == 0, "unit count");
      const int head0 = (is_q ? n0 : n0 - dq) / HDT;
      const int nh = is_q ? a.n_heads : a.n_kv;
      bf16* const base = is_q ? a.q : a.k;
      const bool lora = is_q && a.lora_u;
#pragma unroll
      for (int it = 0; it < HR * UPR / 256; ++it) {
        const int u = tid + it * 256;
        const int r = u / UPR, rem = u % UPR;
        const int hh = rem / CPR, i0 = (rem % CPR) * 4;
        const int m = m0 + hr0 + r;
        if (m >= a.M) continue;
        const float ri = rinv_s[hr0 + r];
        const int w = m / a.Lp, pos = m % a.Lp;
        const int cbase = hh * HDT;
        const float4 cs01 = *reinterpret_cast<const float4*>(a.rope + pos * HALF + i0);
        const float4 cs23 = *reinterpret_cast<const float4*>(a.rope + pos * HALF + i0 + 2);
        const float cs[8] = {cs01.x, cs01.y, cs01.z, cs01.w, cs23.x, cs23.y, cs23.z, cs23.w};
        float x1[4], x2[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int c1 = cbase + i0 + e, c2 = c1 + HALF;
          x1[e] = Cs[r * CLD + c1] * scale_s[c1] * ri;
          x2[e] = Cs[r * CLD + c2] * scale_s[c2] * ri;
        }
        if (lora) {
          const float* uu = a.lora_u + (int64_t)m * 2 * a.lora_r;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int g1 = n0 + cbase + i0 + e, g2 = g1 + HALF;
            float s1 = 0.f, s2 = 0.f;
            for (int t = 0; t < a.lora_r; ++t) {
              s1 += uu[t] * a.lora_bq[g1 * a.lora_r + t];
              s2 += uu[t] * a.lora_bq[g2 * a.lora_r + t];
            }
            x1[e] += s1;
            x2[e] += s2;
          }
        }
        uint16_t y1[4], y2[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float co = cs[2 * e], si = cs[2 * e + 1];
          y1[e] = f2bf_bits(x1[e] * co - x2[e] * si);
          y2[e] = f2bf_bits(x1[e] * si + x2[e] * co);
        }
        bf16* dst = base + (((int64_t)w * nh + head0 + hh) * a.Lp + pos) * HDT;
        *reinterpret_cast<uint2*>(dst + i0) =
            make_uint2((uint32_t)y1[0] | ((uint32_t)y1[1] << 16), (uint32_t)y1[2] | ((uint32_t)y1[3] << 16));
        *reinterpret_cast<uint2*>(dst + HALF + i0) =
            make_uint2((uint32_t)y2[0] | ((uint32_t)y2[1] << 16), (uint32_t)y2[2] | ((uint32_t)y2[3] << 16));
      }
    } else {
      // v heads, written transposed: units of (column, 8 consecutive rows)
      constexpr int RCS = HR / 8;
      static_assert((BN * RCS) % 256 == 0, "unit count");
      const bool lora = a.lora_u != nullptr;
#pragma unroll
      for (int it = 0; it < BN * RCS / 256; ++it) {
        const int u = tid + it * 256;
        const int rc = u % RCS, c = u / RCS;
        const int r0 = rc * 8;
        const int m = m0 + hr0 + r0;
        if (m >= a.M) continue;          // M is a multiple of 8
        const int nv = n0 + c - dq - dkv;      // column inside the v block
        const int head = nv / HDT, dd = nv % HDT;
        const float sc = scale_s[c];
        uint16_t y[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float v = Cs[(r0 + e) * CLD + c] * sc * rinv_s[hr0 + r0 + e];
          if (lora) {
            const float* uu = a.lora_u + (int64_t)(m + e) * 2 * a.lora_r + a.lora_r;
            float sl = 0.f;
            for (int t = 0; t < a.lora_r; ++t) sl += uu[t] * a.lora_bv[nv * a.lora_r + t];
            v += sl;
          }
          y[e] = f2bf_bits(v);
        }
        const int w = m / a.Lp, pos = m % a.Lp;
        bf16* dst = a.vt + (((int64_t)w * a.n_kv + head) * HDT + dd) * a.Lp + pos;
        *reinterpret_cast<uint4*>(dst) = make_uint4(
            (uint32_t)y[0] | ((uint32_t)y[1] << 16), (uint32_t)y[2] | ((uint32_t)y[3] << 16),
            (uint32_t)y[4] | ((uint32_t)y[5] << 16), (uint32_t)y[6] | ((uint32_t)y[7] << 16));
      }
    }
  }
  __syncthreads();
  }  // halves
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
      // the epilogue takes the head size from the tile width (BN = 2 * hd)
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
