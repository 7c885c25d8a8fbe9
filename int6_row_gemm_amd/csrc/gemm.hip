// Dequant-fused GEMM on gfx950 MFMA.
//
// C[m, n] = sum_k A[m, k] * code[n, k] with A binary16 [M, K] (activations) and
// code int8 [N, K] (one quantised weight row per output feature, the layout
// of a [out, in] matrix).  The weight of a linear layer is W[n, k] =
// code[n, k] * scale[n] (pwwt.cn "parameter-golf 16MB 极限压缩实战 …",
// 后训练量化导出: one binary16 scale per row), so the scale is a per-column
// factor of C and is applied in the epilogue; the codes (integers in
// [-128, 127]) are exact in binary16 and are widened on their way into LDS.
// When A holds un-normalised activations, the RMSNorm factor of each row
// (a per-row factor of C) is applied in the epilogue as well.
//
// Tiling: 256 threads = 4 waves in a 2 x 2 grid; workgroup tile BM x BN,
// K step 64 through one XOR-swizzled LDS tile with register prefetch one K
// step ahead; each wave issues v_mfma_f32_16x16x32_f16 on (BM/2) x (BN/2).
// Register-fed variant (the MLP GEMMs, when the caller passes the codes
// rearranged by launch_shuffle_codes): only the A tile goes through LDS;
// the waves split the tile 1 x 4 (128 x 32 each) and load their own code
// fragments with one coalesced 16-byte load per lane and K step, widening
// them in registers.  This halves the LDS writes of a K step, which bound
// the staged loop on gfx950 (timing copies without the staging stores run
// the loop at the full MFMA rate), and was measured 4-6 % faster on fc and
// proj in the full pass; the output projection (K = 512) stays staged, its
// short loop does not repay the longer 8-row epilogue.
// Rows are placed in LDS so that every lane ends up owning runs of
// consecutive output columns of one row (C^T accumulation: two runs of 8,
// or whole rotation pairs of a q/k head), or, for the transposed V output,
// 16 consecutive rows of one column (C accumulation); the epilogues then
// work straight from the accumulator registers with 16- or 32-byte global
// accesses and no LDS round trip:
//   EPI_QKV   q/k/v projection: * scale * rinv (+ rank-r LoRA), RoPE on the
//             q and k heads, writes Q [W,Hq,Lp,hd], K [W,Hkv,Lp,hd] and
//             V transposed [W,Hkv,hd,Lp] in binary16;
//   EPI_RELU2 MLP up-projection: h = binary16(relu(acc * scale * rinv)^2);
//   EPI_RES   output / down projection: x += acc * scale, then the skip
//             push/pop of the block schedule, and binary16(x) plus per-tile
//             sums of x^2 for the next normed GEMM.
#include "common.h"
#include "mfma_util.h"

namespace i6g {
namespace {

constexpr int BK = 64;
constexpr int LDK = BK;      // LDS row stride in binary16 elements (128 bytes)

// LDS tiles keep 128-byte rows of eight 16-byte chunks; chunk j of row r is
// stored in slot j ^ ((r >> 1) & 7).  Measured on gfx950, this makes both the
// MFMA fragment reads (16 rows, one chunk each) and the staging writes free of
// bank conflicts, where a 16-byte row padding costs a two-way conflict.
__device__ inline int swz(int row, int chunk) { return chunk ^ ((row >> 1) & 7); }

template <int BM, int BN, bool RB>
struct Smem {
  static constexpr int kBytes = (BM + (RB ? 0 : BN)) * LDK * 2;   // one A and (unless RB) one B tile
};

// N consecutive values stored as binary16 (N even)
template <int N>
__device__ inline void store_h_run(act* dst, const float (&y)[N]) {
  if constexpr (N == 8) {
    *reinterpret_cast<uint4*>(dst) =
        make_uint4(pack2h(y[0], y[1]), pack2h(y[2], y[3]), pack2h(y[4], y[5]), pack2h(y[6], y[7]));
  } else if constexpr (N == 4) {
    *reinterpret_cast<uint2*>(dst) = make_uint2(pack2h(y[0], y[1]), pack2h(y[2], y[3]));
  } else {
    static_assert(N % 2 == 0, "pairs");
#pragma unroll
    for (int e = 0; e < N; e += 2) reinterpret_cast<uint32_t*>(dst)[e / 2] = pack2h(y[e], y[e + 1]);
  }
}

// Main loop and epilogue of one tile.  CT: accumulate C^T (every epilogue
// except the V heads of the q/k/v projection, which keep C).  RB: the
// weight codes come pre-arranged in fragment order (shuffle_codes) and go
// from global memory straight into each wave's registers; only the A tile
// is staged through LDS, and the four waves split the tile 1 x 4 (128 rows
// x 32 columns each) so that every code is still loaded once per tile.
template <int BM, int BN, int EPI, bool CT, bool RB>
__device__ __forceinline__ void gemm_body(const GemmArgs& a, act* As, act* Bs, float* rinv_s,
                                          float* scale_s, float* popw_s, float (*ss_part)[BM],
                                          int tid, int wave, int m0, int n0, int tn) {
  constexpr int WM = RB ? BM : BM / 2, WN = RB ? BN / 4 : BN / 2;
  constexpr int NWN = BN / WN;                // waves across the columns
  constexpr int FM = WM / 16, FN = WN / 16;
  constexpr int A_CHUNKS = BM * BK / 8;       // 16-byte chunks of binary16
  constexpr int B_CHUNKS = RB ? 0 : BN * BK / 16;   // 16-byte chunks of int8 staged through LDS
  constexpr int A_PER = (A_CHUNKS + 255) / 256;
  constexpr int B_PER = (B_CHUNKS + 255) / 256;
  static_assert(!RB || (CT && EPI != EPI_QKV && WN == 32), "register-fed codes: row-major epilogues only");
  const int lane = tid & 63;
  const int wm = RB ? 0 : wave >> 1, wn = RB ? wave : wave & 1;
  const int dq = a.n_heads * WN, dkv = a.n_kv * WN;

  // Global -> register staging into named scalars (arrays of them end up
  // in scratch memory).  Chunk
  // indices past the tile are clamped (those threads reload and rewrite the
  // last chunk with identical data); A rows past M are clamped to M - 1 and
  // their results are never stored.
  static_assert(A_PER <= 4 && B_PER <= 3, "staging holds 4 A and 3 B chunks per thread");
  uint4 sa0_0, sa0_1, sa0_2, sa0_3, sb0_0, sb0_1, sb0_2;
  const int nk = a.K / BK;
  // per thread, for the whole K loop: the element offset of each A row it
  // loads, and the LDS offsets its A and B chunks go to
  int64_t arow0 = 0, arow1 = 0, arow2 = 0, arow3 = 0;
  int aso0 = 0, aso1 = 0, aso2 = 0, aso3 = 0;
  int bso0a = 0, bso0b = 0, bso1a = 0, bso1b = 0, bso2a = 0, bso2b = 0;
#define GM_AROW(i, V, O)                                                              \
  if constexpr (A_PER > i) {                                                          \
    const int c = min(tid + (i) * 256, A_CHUNKS - 1);                                 \
    const int m = min(m0 + (c >> 3), a.M - 1);                                        \
    V = (a.a_map ? scored_row(a.p0 + m, a.k0, a.n_win, a.e0, a.L, a.S, a.Lp) : m) * (int64_t)a.K; \
    const int pr = ((c >> 3) & ~63) | perm16((c >> 3) & 63);                          \
    O = pr * LDK + swz(pr, c & 7) * 8;                                                \
  }
  GM_AROW(0, arow0, aso0) GM_AROW(1, arow1, aso1) GM_AROW(2, arow2, aso2) GM_AROW(3, arow3, aso3)
#undef GM_AROW
#define GM_BROW(i, OA, OB)                                                            \
  if constexpr (B_PER > i) {                                                          \
    const int c = min(tid + (i) * 256, B_CHUNKS - 1);                                 \
    const int r = c >> 2, j2 = (c & 3) * 2;                                           \
    int pr;                                                                           \
    if constexpr (EPI == EPI_QKV) {                                                   \
      pr = CT ? (r / WN) * WN + rope_phys<WN>(r % WN, a.rope_dims) : r;               \
    } else {                                                                          \
      pr = (r & ~63) | pair_phys(r & 63);                                             \
    }                                                                                 \
    OA = pr * LDK + swz(pr, j2) * 8;                                                  \
    OB = pr * LDK + swz(pr, j2 + 1) * 8;                                              \
  }
  GM_BROW(0, bso0a, bso0b) GM_BROW(1, bso1a, bso1b) GM_BROW(2, bso2a, bso2b)
#undef GM_BROW

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
#define GM_SA(i, R)                                                                   \
  if constexpr (A_PER > i) *reinterpret_cast<uint4*>(As + aso##i) = R;
#define GM_SB(i, R)                                                                   \
  if constexpr (B_PER > i) {                                                          \
    const uint32_t w_[4] = {R.x, R.y, R.z, R.w};                                      \
    uint32_t o_[8];                                                                   \
    _Pragma("unroll") for (int j = 0; j < 4; ++j) widen4h(w_[j], o_[2 * j], o_[2 * j + 1]); \
    *reinterpret_cast<uint4*>(Bs + bso##i##a) = make_uint4(o_[0], o_[1], o_[2], o_[3]); \
    *reinterpret_cast<uint4*>(Bs + bso##i##b) = make_uint4(o_[4], o_[5], o_[6], o_[7]); \
  }
#define GM_STORE(S)                                                                   \
  {                                                                                   \
    GM_SA(0, sa##S##_0) GM_SA(1, sa##S##_1) GM_SA(2, sa##S##_2) GM_SA(3, sa##S##_3)   \
    GM_SB(0, sb##S##_0) GM_SB(1, sb##S##_1) GM_SB(2, sb##S##_2)                       \
  }

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // RB: the wave's codes of one K tile are FN chunks of 16 bytes per lane
  // (both 32-wide halves of its fragment rows), contiguous per wave
  uint4 bq0 = make_uint4(0, 0, 0, 0), bq1 = make_uint4(0, 0, 0, 0);
  const int8_t* bp_wave = nullptr;
  if constexpr (RB) {
    static_assert(FN == 2, "two code chunks per lane");
    bp_wave = a.Bp + ((int64_t)tn * (a.K / BK) * NWN + wn) * (FN * 64 * 16) + lane * 16;
  }
#define GM_BQ_LOAD(kt)                                                                \
  if constexpr (RB) {                                                                 \
    const int8_t* p_ = bp_wave + (int64_t)(kt) * (NWN * FN * 64 * 16);                \
    bq0 = *reinterpret_cast<const uint4*>(p_);                                        \
    bq1 = *reinterpret_cast<const uint4*>(p_ + 64 * 16);                              \
  }

  const int lr = lane & 15, lg = lane >> 4;
  // MF_C: acc block (i, j) = C (A rows x weight rows); MF_T: its transpose.
#define MF_C(x, w, c) __builtin_amdgcn_mfma_f32_16x16x32_f16(x, w, c, 0, 0, 0)
#define MF_T(x, w, c) __builtin_amdgcn_mfma_f32_16x16x32_f16(w, x, c, 0, 0, 0)
#define GM_COMPUTE(MF)                                                                \
  {                                                                                   \
    _Pragma("unroll") for (int ks = 0; ks < BK / 32; ++ks) {                          \
      actx8 af[FM], bfg[FN];                                                         \
      _Pragma("unroll") for (int i = 0; i < FM; ++i) {                                \
        const int r_ = wm * WM + i * 16 + lr;                                         \
        af[i] = *reinterpret_cast<const actx8*>(As + r_ * LDK + swz(r_, ks * 4 + lg) * 8); \
      }                                                                               \
      if constexpr (RB) {                                                             \
        bfg[0] = ks == 0 ? wb0[0] : wb1[0];                                           \
        bfg[1] = ks == 0 ? wb0[1] : wb1[1];                                           \
      } else {                                                                        \
        _Pragma("unroll") for (int j = 0; j < FN; ++j) {                              \
          const int r_ = wn * WN + j * 16 + lr;                                       \
          bfg[j] = *reinterpret_cast<const actx8*>(Bs + r_ * LDK + swz(r_, ks * 4 + lg) * 8); \
        }                                                                             \
      }                                                                               \
      _Pragma("unroll") for (int i = 0; i < FM; ++i)                                  \
        _Pragma("unroll") for (int j = 0; j < FN; ++j)                                \
          acc[i][j] = MF(af[i], bfg[j], acc[i][j]);                                   \
    }                                                                                 \
  }
#define GM_COMPUTE_ANY()                                                              \
  {                                                                                   \
    if constexpr (CT) GM_COMPUTE(MF_T) else GM_COMPUTE(MF_C)                          \
  }
  // One K tile: the loads of tile kt+1 go into the staging registers while
  // tile kt is multiplied out of the single LDS tile, then replace it.  One
  // staging set and one LDS tile keep the kernel within 128 VGPRs and 34 KB
  // of LDS, so four workgroups share a CU and their waves hide the load
  // latency (measured on gfx950 to beat two-deep register prefetch at three
  // workgroups per CU); their epilogues overlap the others' MFMA work.
#define GM_STEP(kt)                                                                   \
  {                                                                                   \
    GM_LOAD(min((kt) + 1, nk - 1), 0);                                                \
    actx8 wb0[2], wb1[2];   /* RB: widened codes of this K tile, by 32-wide half */  \
    if constexpr (RB) {                                                               \
      wb0[0] = widen8(bq0.x, bq0.y); wb1[0] = widen8(bq0.z, bq0.w);                   \
      wb0[1] = widen8(bq1.x, bq1.y); wb1[1] = widen8(bq1.z, bq1.w);                   \
      GM_BQ_LOAD(min((kt) + 1, nk - 1));                                              \
    }                                                                                 \
    GM_COMPUTE_ANY();                                                                 \
    if ((kt) + 1 < nk) {                                                              \
      __syncthreads();                                                                \
      GM_STORE(0);                                                                    \
      __syncthreads();                                                                \
    }                                                                                 \
  }

  GM_LOAD(0, 0);
  GM_BQ_LOAD(0);
  {
    // the per-column weight scales and per-row RMS factors (read by the
    // epilogue only) load while the first K tile is in flight
    static_assert(BN <= 256 && BM <= 256, "one factor per thread");
    float sc_r = 0.0f, pw_r = 0.0f, ri_r = 0.0f;
    if (tid < BN) {
      sc_r = h2f(a.scale[n0 + tid]);
      if constexpr (EPI == EPI_RES) pw_r = a.pop_w ? a.pop_w[n0 + tid] : 0.0f;
    }
    if constexpr (EPI == EPI_QKV || EPI == EPI_RELU2) {
      const int m = m0 + tid;
      if (tid < BM && m < a.M) {
        const int64_t mr = a.a_map ? scored_row(a.p0 + m, a.k0, a.n_win, a.e0, a.L, a.S, a.Lp) : m;
        float ss = 0.0f;
        for (int t = 0; t < a.nt_in; ++t) ss += a.ss_in[mr * a.nt_in + t];
        ri_r = 1.0f / sqrtf(ss / (float)a.K + a.eps);
      }
    }
    GM_STORE(0);
    if (tid < BN) {
      scale_s[tid] = sc_r;
      if constexpr (EPI == EPI_RES) popw_s[tid] = pw_r;
    }
    if (tid < BM) rinv_s[tid] = ri_r;
  }
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) GM_STEP(kt);
#undef GM_STEP
#undef GM_BQ_LOAD
#undef GM_COMPUTE_ANY
#undef GM_COMPUTE
#undef MF_T
#undef MF_C
#undef GM_STORE
#undef GM_SB
#undef GM_SA
#undef GM_LOAD
#undef GM_B
#undef GM_A

  // Epilogues straight from the accumulators.  In the C^T orientation lane
  // (lr, lg) of block (i, j) holds A row wm*WM + 16*(lr>>2) + 4i + (lr&3)
  // and the 4 weight rows the placement above gives output rows 4lg..4lg+3
  // of fragment j; in the C orientation (v heads) it holds weight row
  // wn*WN + 16j + lr and the 16 consecutive A rows wm*WM + 16*lg + 4i + e.
  const int lrow = 16 * (lr >> 2) + (lr & 3);
  // the lane's A row in C^T block i: 64-row slices of four blocks each
  auto arow = [&](int i) { return 64 * (i >> 2) + lrow + 4 * (i & 3); };
  if constexpr (EPI == EPI_RELU2) {
    float vmax = 0.0f;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int ml = wm * WM + arow(i);
      const int m = m0 + ml;
      if (m >= a.M) continue;
      const float ri = rinv_s[ml];
#pragma unroll
      for (int p = 0; p < FN / 2; ++p) {
        const int cl = wn * WN + 32 * p + 8 * lg;   // 8 consecutive columns: blocks 2p, 2p+1
        uint32_t o[4];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const float4 s4 = reinterpret_cast<const float4*>(scale_s + cl)[h];
          const f32x4 c = acc[i][2 * p + h];
          const float v0 = lrelu(c[0] * s4.x * ri, a.leaky), v1 = lrelu(c[1] * s4.y * ri, a.leaky);
          const float v2 = lrelu(c[2] * s4.z * ri, a.leaky), v3 = lrelu(c[3] * s4.w * ri, a.leaky);
          vmax = fmaxf(vmax, fmaxf(fmaxf(fabsf(v0), fabsf(v1)), fmaxf(fabsf(v2), fabsf(v3))));
          o[2 * h] = pack2h(v0 * v0, v1 * v1);
          o[2 * h + 1] = pack2h(v2 * v2, v3 * v3);
        }
        *reinterpret_cast<uint4*>(a.h + (int64_t)m * a.N + n0 + cl) = make_uint4(o[0], o[1], o[2], o[3]);
      }
    }
    if (__any(!(vmax < kRangeSqrt)) && (tid & 63) == 0) atomicOr(a.flags, kFlagRange);
  } else if constexpr (EPI == EPI_RES) {
    static_assert(BN == 128, "partial sums of squares cover 128 columns");
    const bool push = a.push_dst != nullptr;
    const bool pop = a.pop_src != nullptr;
    const bool pop_self = pop && a.pop_src == a.push_dst;
    // the lane's columns: block j holds the 4 starting at colj(j)
    auto colj = [&](int j) { return wn * WN + 32 * (j >> 1) + 8 * lg + 4 * (j & 1); };
    // the residual rows in groups of FH row blocks (eight float4 per lane),
    // each group's loads in flight together; row offsets per group
    constexpr int FH = 8 / FN;
    float sq[FM];
    bool range_bad = false;   // a partial row sum of squares reaches 65504^2
#pragma unroll
    for (int hh = 0; hh < FM / FH; ++hh) {
      int64_t off[FM];
      bool ok[FM];
#pragma unroll
      for (int ii = 0; ii < FH; ++ii) {
        const int i = hh * FH + ii;
        const int m = m0 + wm * WM + arow(i);
        ok[i] = m < a.M;
        const int mm = min(m, a.M - 1);   // rows past M recompute row M-1 and store nothing
        const int64_t mr = a.e_map ? scored_row(a.p0 + mm, a.k0, a.n_win, a.e0, a.L, a.S, a.Lp) : mm;
        off[i] = mr * a.N + n0;
      }
      float4 xv[FH][FN];
#pragma unroll
      for (int ii = 0; ii < FH; ++ii)
#pragma unroll
        for (int j = 0; j < FN; ++j) xv[ii][j] = *reinterpret_cast<const float4*>(a.x + off[hh * FH + ii] + colj(j));
#pragma unroll
      for (int ii = 0; ii < FH; ++ii) {
        const int i = hh * FH + ii;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const float4 s4 = *reinterpret_cast<const float4*>(scale_s + colj(j));
          xv[ii][j].x += acc[i][j][0] * s4.x;
          xv[ii][j].y += acc[i][j][1] * s4.y;
          xv[ii][j].z += acc[i][j][2] * s4.z;
          xv[ii][j].w += acc[i][j][3] * s4.w;
        }
        if (push && ok[i]) {
#pragma unroll
          for (int j = 0; j < FN; ++j) *reinterpret_cast<float4*>(a.push_dst + off[i] + colj(j)) = xv[ii][j];
        }
      }
      if (pop) {
        if (pop_self) {
#pragma unroll
          for (int ii = 0; ii < FH; ++ii)
#pragma unroll
            for (int j = 0; j < FN; ++j) {
              const float4 w4 = *reinterpret_cast<const float4*>(popw_s + colj(j));
              xv[ii][j].x += w4.x * xv[ii][j].x;
              xv[ii][j].y += w4.y * xv[ii][j].y;
              xv[ii][j].z += w4.z * xv[ii][j].z;
              xv[ii][j].w += w4.w * xv[ii][j].w;
            }
        } else {
          float4 pv[FH][FN];
#pragma unroll
          for (int ii = 0; ii < FH; ++ii)
#pragma unroll
            for (int j = 0; j < FN; ++j)
              pv[ii][j] = *reinterpret_cast<const float4*>(a.pop_src + off[hh * FH + ii] + colj(j));
#pragma unroll
          for (int ii = 0; ii < FH; ++ii)
#pragma unroll
            for (int j = 0; j < FN; ++j) {
              const float4 w4 = *reinterpret_cast<const float4*>(popw_s + colj(j));
              xv[ii][j].x += w4.x * pv[ii][j].x;
              xv[ii][j].y += w4.y * pv[ii][j].y;
              xv[ii][j].z += w4.z * pv[ii][j].z;
              xv[ii][j].w += w4.w * pv[ii][j].w;
            }
        }
      }
#pragma unroll
      for (int ii = 0; ii < FH; ++ii) {
        const int i = hh * FH + ii;
        float t = 0.0f;
#pragma unroll
        for (int j = 0; j < FN; ++j)
          t += xv[ii][j].x * xv[ii][j].x + xv[ii][j].y * xv[ii][j].y + xv[ii][j].z * xv[ii][j].z +
               xv[ii][j].w * xv[ii][j].w;
        sq[i] = t;
        range_bad |= a.xb && ok[i] && t >= kRangeSq;
        if (ok[i]) {
#pragma unroll
          for (int j = 0; j < FN; ++j) *reinterpret_cast<float4*>(a.x + off[i] + colj(j)) = xv[ii][j];
          if (a.xb) {
#pragma unroll
            for (int p = 0; p < FN / 2; ++p) {
              const f32x4 u0 = {xv[ii][2 * p].x, xv[ii][2 * p].y, xv[ii][2 * p].z, xv[ii][2 * p].w};
              const f32x4 u1 = {xv[ii][2 * p + 1].x, xv[ii][2 * p + 1].y, xv[ii][2 * p + 1].z, xv[ii][2 * p + 1].w};
              *reinterpret_cast<uint4*>(a.xb + off[i] + colj(2 * p)) = make_uint4(
                  pack2h(u0[0], u0[1]), pack2h(u0[2], u0[3]), pack2h(u1[0], u1[1]), pack2h(u1[2], u1[3]));
            }
          }
        }
      }
    }
    if (__any(range_bad) && (tid & 63) == 0) atomicOr(a.flags, kFlagRange);
    if (a.ss_out) {
      // the four lane groups of a row, then the two waves of a tile row
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        sq[i] += __shfl_xor(sq[i], 16);
        sq[i] += __shfl_xor(sq[i], 32);
        if (lg == 0) ss_part[wn][wm * WM + arow(i)] = sq[i];
      }
      __syncthreads();
      for (int r = tid; r < BM; r += 256) {
        const int m = m0 + r;
        if (m >= a.M) continue;
        const int64_t mr = a.e_map ? scored_row(a.p0 + m, a.k0, a.n_win, a.e0, a.L, a.S, a.Lp) : m;
        float t_ = ss_part[0][r];
#pragma unroll
        for (int u = 1; u < NWN; ++u) t_ += ss_part[u][r];
        a.ss_out[mr * (a.N / 128) + tn] = t_;
      }
    }
  } else {  // EPI_QKV: BN = 2 * head_dim, each wave holds one whole head
    constexpr int HD = WN, HALF = HD / 2, Q8 = HD / 8;
    const int colbase = n0 + wn * HD;
    if constexpr (CT) {
      // q or k head, C^T: lane holds rotation pairs c1b + t, t < Q8, whose
      // first dims are f0 + t and second dims s0 + t
      const bool is_q = colbase < dq;
      const int head = (is_q ? colbase : colbase - dq) / HD;
      const int nh = is_q ? a.n_heads : a.n_kv;
      act* const base = is_q ? a.q : a.k;
      const bool lora = is_q && a.lora_u;
      const int c1b = lg * Q8;
      const int f0 = pair_first<HD>(c1b, a.rope_dims), s0 = pair_second<HD>(c1b, a.rope_dims);
      float sc1[Q8], sc2[Q8];
#pragma unroll
      for (int t = 0; t < Q8; ++t) {
        sc1[t] = scale_s[wn * HD + f0 + t];
        sc2[t] = scale_s[wn * HD + s0 + t];
      }
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int ml = wm * WM + arow(i);
        const int m = m0 + ml;
        if (m >= a.M) continue;
        const float ri = rinv_s[ml];
        const int w = m / a.Lp, pos = m % a.Lp;
        const float4* csp = reinterpret_cast<const float4*>(a.rope + pos * HALF + c1b);
        float x1[Q8], x2[Q8];
#pragma unroll
        for (int t = 0; t < Q8; ++t) {
          x1[t] = acc[i][t >> 2][t & 3] * sc1[t] * ri;
          x2[t] = acc[i][(t + Q8) >> 2][(t + Q8) & 3] * sc2[t] * ri;
        }
        if (lora) {
          // rank <= 8: the row's u and each column's B row are read with
          // unrolled, guarded loads so that they are all in flight at once
          const float* uu = a.lora_u + (int64_t)m * 2 * a.lora_r;
          float ur[8] = {};
#pragma unroll
          for (int r = 0; r < 8; ++r)
            if (r < a.lora_r) ur[r] = uu[r];
#pragma unroll
          for (int t = 0; t < Q8; ++t) {
            const float* b1 = a.lora_bq + (int64_t)(colbase + f0 + t) * a.lora_r;
            const float* b2 = a.lora_bq + (int64_t)(colbase + s0 + t) * a.lora_r;
            float s1 = 0.f, s2 = 0.f;
#pragma unroll
            for (int r = 0; r < 8; ++r)
              if (r < a.lora_r) {
                s1 += ur[r] * b1[r];
                s2 += ur[r] * b2[r];
              }
            x1[t] += s1;
            x2[t] += s2;
          }
        }
        float y1[Q8], y2[Q8];
        {
          // every product rounded on its own, no fused multiply-add (the
          // one-tile q/k/v kernel rotates the same way, so both agree bit
          // for bit)
#pragma clang fp contract(off)
#pragma unroll
          for (int t = 0; t < Q8; t += 2) {
            const float4 cs = csp[t / 2];   // (cos, sin) of indices c1b + t and c1b + t + 1
            y1[t] = x1[t] * cs.x - x2[t] * cs.y;
            y2[t] = x1[t] * cs.y + x2[t] * cs.x;
            y1[t + 1] = x1[t + 1] * cs.z - x2[t + 1] * cs.w;
            y2[t + 1] = x1[t + 1] * cs.w + x2[t + 1] * cs.z;
          }
        }
        act* dst = base + (((int64_t)w * nh + head) * a.Lp + pos) * HD;
        store_h_run<Q8>(dst + f0, y1);
        store_h_run<Q8>(dst + s0, y2);
      }
    } else {
      // v head, C orientation, written transposed: the lane's 16 rows are
      // consecutive positions of one window (windows are 64-row aligned)
      const int head = (colbase - dq - dkv) / HD;
      const int mb = m0 + wm * WM + 16 * lg;
      if (mb < a.M) {
        const bool lora = a.lora_u != nullptr;
        float ri[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 r4 = reinterpret_cast<const float4*>(rinv_s + wm * WM + 16 * lg)[q];
          ri[4 * q] = r4.x; ri[4 * q + 1] = r4.y; ri[4 * q + 2] = r4.z; ri[4 * q + 3] = r4.w;
        }
        const int w = mb / a.Lp, pos = mb % a.Lp;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int dd = 16 * j + lr;
          const float sc = scale_s[wn * HD + dd];
          // rank <= 8: the column's B row once, then each row's u, with
          // unrolled, guarded loads (all in flight at once)
          float bvr[8] = {};
          if (lora) {
            const float* bv = a.lora_bv + (int64_t)(head * HD + dd) * a.lora_r;
#pragma unroll
            for (int r = 0; r < 8; ++r)
              if (r < a.lora_r) bvr[r] = bv[r];
          }
          float y[16];
#pragma unroll
          for (int t = 0; t < 16; ++t) {
            float v = acc[t >> 2][j][t & 3] * sc * ri[t];
            if (lora) {
              const float* uu = a.lora_u + (int64_t)(mb + t) * 2 * a.lora_r + a.lora_r;
              float sl = 0.f;
#pragma unroll
              for (int r = 0; r < 8; ++r)
                if (r < a.lora_r) sl += uu[r] * bvr[r];
              v += sl;
            }
            y[t] = v;
          }
          uint4* dst = reinterpret_cast<uint4*>(a.vt + (((int64_t)w * a.n_kv + head) * HD + dd) * a.Lp + pos);
          dst[0] = make_uint4(pack2h(y[0], y[1]), pack2h(y[2], y[3]), pack2h(y[4], y[5]), pack2h(y[6], y[7]));
          dst[1] = make_uint4(pack2h(y[8], y[9]), pack2h(y[10], y[11]), pack2h(y[12], y[13]), pack2h(y[14], y[15]));
        }
      }
    }
  }
}

template <int BM, int BN, int EPI, bool RB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(BN > 128 ? 2 : 4)))
void gemm_kernel(GemmArgs a) {
  static_assert(BM / 2 == 64, "the row placement works on 64-row slices");
  static_assert(EPI == EPI_QKV || BN / 2 == 64, "the column placement works on 64-column slices");
  __shared__ __attribute__((aligned(16))) char smem[Smem<BM, BN, RB>::kBytes];
  __shared__ __attribute__((aligned(16))) float rinv_s[BM];
  __shared__ __attribute__((aligned(16))) float scale_s[BN];
  __shared__ __attribute__((aligned(16))) float popw_s[BN];
  __shared__ float ss_part[RB ? 4 : 2][BM];
  act* As = reinterpret_cast<act*>(smem);
  act* Bs = RB ? nullptr : As + BM * LDK;

  const int tid = threadIdx.x & 255;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ntn = a.N / BN;
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int tm = tile / ntn, tn = tile % ntn;
  const int m0 = tm * BM, n0 = tn * BN;

  // q/k/v projection: BN = 2 * head_dim and the v block starts on a tile
  // boundary (an even number of kv heads), so a tile is all q/k or all v
  if (EPI == EPI_QKV && n0 >= (a.n_heads + a.n_kv) * (BN / 2))
    gemm_body<BM, BN, EPI, false, false>(a, As, Bs, rinv_s, scale_s, popw_s, ss_part, tid, wave, m0, n0, tn);
  else
    gemm_body<BM, BN, EPI, true, RB>(a, As, Bs, rinv_s, scale_s, popw_s, ss_part, tid, wave, m0, n0, tn);
}

template <int BM, int BN, int EPI, bool RB = false>
hipError_t run(const GemmArgs& a, hipStream_t s) {
  int tiles = ((a.M + BM - 1) / BM) * (a.N / BN);
  hipLaunchKernelGGL((gemm_kernel<BM, BN, EPI, RB>), dim3(tiles), dim3(256), 0, s, a);
  return hipGetLastError();
}

// Weight codes rearranged for the register-fed path: 16-byte chunk c of the
// output is lane c % 64 of code fragment (c / 64) % 2 of wave (c / 128) % 4
// in K tile (c / 512) % nk of column tile c / (512 nk); it holds, for the
// logical column 32 * wave + pair_logical32(16 * fragment + lane % 16), the
// codes of k = 64 * tile + 8 * (lane / 16) + 0..7 and the same + 32.
// With `scale` given, rows whose binary16 scale is zero get zero codes: their
// weights are zero, and kernels that divide by the scale (treating a zero
// scale as 1) then add exactly nothing for them.
__global__ __launch_bounds__(256) void shuffle_codes_kernel(const int8_t* __restrict__ B, int32_t N, int32_t K,
                                                            const uint16_t* __restrict__ scale,
                                                            int8_t* __restrict__ Bp) {
  const int nk = K / BK;
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= (int64_t)(N / 128) * nk * 512) return;
  const int lane = (int)(c & 63), j = (int)((c >> 6) & 1), wv = (int)((c >> 7) & 3);
  const int64_t q = c >> 9;
  const int kt = (int)(q % nk), tn = (int)(q / nk);
  const int row = tn * 128 + 32 * wv + pair_logical32(16 * j + (lane & 15));
  const int8_t* src = B + (int64_t)row * K + kt * BK + 8 * (lane >> 4);
  uint2 lo = *reinterpret_cast<const uint2*>(src);
  uint2 hi = *reinterpret_cast<const uint2*>(src + 32);
  if (scale && (scale[row] & 0x7fffu) == 0) lo = hi = make_uint2(0, 0);
  *reinterpret_cast<uint4*>(Bp + c * 16) = make_uint4(lo.x, lo.y, hi.x, hi.y);
}

}  // namespace

hipError_t launch_shuffle_codes(const int8_t* B, int32_t N, int32_t K, const uint16_t* zero_scale_rows, int8_t* Bp,
                                hipStream_t s) {
  if (N <= 0 || K <= 0 || N % 128 != 0 || K % BK != 0) return hipErrorInvalidValue;
  const int64_t chunks = (int64_t)(N / 128) * (K / BK) * 512;
  hipLaunchKernelGGL(shuffle_codes_kernel, dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, s, B, N, K,
                     zero_scale_rows, Bp);
  return hipGetLastError();
}

hipError_t launch_gemm(int epi, const GemmArgs& a, hipStream_t s) {
  switch (epi) {
    case EPI_QKV:
      // the epilogue takes the head size from the tile width (BN = 2 * hd)
      if (a.hd == 32) return run<128, 64, EPI_QKV>(a, s);
      if (a.hd == 64) return run<128, 128, EPI_QKV>(a, s);
      if (a.hd == 80) return run<128, 160, EPI_QKV>(a, s);
      return hipErrorInvalidValue;
    case EPI_RELU2:
      return a.Bp ? run<128, 128, EPI_RELU2, true>(a, s) : run<128, 128, EPI_RELU2>(a, s);
    case EPI_RES:
      return a.Bp ? run<128, 128, EPI_RES, true>(a, s) : run<128, 128, EPI_RES>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace i6g
