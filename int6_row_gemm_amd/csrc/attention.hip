// Causal grouped-query attention over a batch of windows, flash style.
//
// pwwt.cn "parameter-golf 16MB 极限压缩实战 …", section 架构：11 层 U-Net 变压器:
// GQA with 8 query and 4 KV heads and RoPE (applied by the projection
// epilogue).  Query head h reads KV head h / 2; scores are q.k / sqrt(hd)
// with a causal mask inside each window; softmax over keys 0..j.
//
// One workgroup = (window, KV head, 64 queries) and both query heads of the
// group, so each K/V tile brought into LDS serves 128 query rows.  Each of
// the 4 waves owns 32 queries of one head.
//
// * The scores are formed transposed, S^T = K Q^T, with
//   v_mfma_f32_16x16x32_f16: a lane's accumulator holds one query and 4
//   keys, so a query's running max lives in one lane group and needs two
//   cross-lane steps (gfx950 v_permlane16/32_swap, no LDS round trip).
// * The keys feeding the S^T rows are permuted so that the probabilities a
//   lane holds are exactly the 8 consecutive keys the B operand of
//   O^T += V^T P^T wants; P never leaves registers.  The permutation is
//   applied when K is written to LDS, so fragment reads stay on 16
//   consecutive rows; all LDS tiles use layouts measured free of bank
//   conflicts on gfx950.
// * The softmax denominator comes out of the same MFMAs: a constant block of
//   ones appended to V^T makes one extra O^T block equal to sum_k P[q, k]
//   (of the binary16 P actually used), with no VALU adds.
// * exp is the hardware exp2 with the 1/sqrt(hd) * log2(e) factor folded
//   into one multiply-add.  Probabilities are taken relative to a reference
//   max that only moves when a tile max exceeds it by more than 2^8, so the
//   rescale of O is rare; the causal mask is applied only on the last
//   (diagonal) tile, which is peeled off the loop.
// * Pipelining: K and V tiles go through two LDS buffers each with one
//   barrier per key tile; the global loads of tile kt+1 are issued at the
//   start of step kt and written to LDS at its end.  One score set and one
//   staging set per wave keep head_dim 64 within 168 VGPRs, so three
//   workgroups share a CU and overlap each other's softmax, MFMA and
//   barrier phases (measured faster on gfx950 than keeping the next tile's
//   scores in flight at two workgroups per CU).
#include "common.h"
#include "mfma_util.h"

namespace i6g {
namespace {

typedef float f32x8 __attribute__((ext_vector_type(8)));

// 16-byte chunk j of a 128-byte LDS row r lives in slot j ^ ((r >> 1) & 7).
__device__ inline int swz(int row, int chunk) { return chunk ^ ((row >> 1) & 7); }

// LDS row of key k inside a 64-key tile: S^T row r of block kb reads key
// 32(kb>>1) + 8(r>>2) + 4(kb&1) + (r&3), and key k is stored at row 16 kb + r,
// so every S^T fragment read covers 16 consecutive LDS rows.
__device__ inline int key_row(int k) {
  const int kb = 2 * (k >> 5) + ((k >> 2) & 1);
  const int r = 4 * ((k >> 3) & 3) + (k & 3);
  return 16 * kb + r;
}

__device__ inline float max_xor16(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, v), __builtin_bit_cast(unsigned, v),
                                            false, false);
  return __builtin_fmaxf(__builtin_bit_cast(float, r[0]), __builtin_bit_cast(float, r[1]));
}
__device__ inline float max_xor32(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, v), __builtin_bit_cast(unsigned, v),
                                            false, false);
  return __builtin_fmaxf(__builtin_bit_cast(float, r[0]), __builtin_bit_cast(float, r[1]));
}

// Three workgroups per CU where the registers allow it (head_dim <= 64):
// the waves of the other workgroups then fill the MFMA pipe while one waits
// on its softmax or barrier.
template <int HD>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(HD <= 64 ? 3 : 2))) void attn_kernel(AttnArgs a) {
  constexpr int KS = (HD + 31) / 32;  // 32-wide k steps over the head dim
  constexpr int HDP = KS * 32;
  constexpr int DB = HD / 16;         // 16-row blocks of O^T
  // LDS row strides chosen for conflict-free 16-row fragment reads on gfx950:
  // 128-byte rows with an XOR swizzle of the 16-byte chunks, or 160 / 224-byte
  // rows where the padded head dim does not fill 128 bytes exactly.
  constexpr bool KSWZ = (HDP == 64);
  constexpr int KLD = KSWZ ? 64 : (HDP == 96 ? 112 : 80);
  constexpr int VLD = 64;
  constexpr int KCH = 64 * HD / 8;    // 16-byte chunks per K tile
  constexpr int VCH = HD * 64 / 8;    // 16-byte chunks per V^T tile
  constexpr int KPER = (KCH + 255) / 256;
  constexpr int VPER = (VCH + 255) / 256;

  __shared__ __attribute__((aligned(16))) act Ks[2][64 * KLD];
  __shared__ __attribute__((aligned(16))) act Vs[2][HD * VLD];

  const int tid = threadIdx.x & 255, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  // 1-D grid over (window, KV head, query tile).  The hardware deals
  // workgroups round-robin over 8 XCDs; remap so that every query tile of a
  // (window, KV head) pair runs on one XCD and shares its K/V through that
  // XCD's L2, and hand out the longest (causal) tiles first.
  const int nqt = a.Lp / 64;
  const int npairs = a.W * a.n_kv;
  int qt, pair;
  {
    const int bid = blockIdx.x;
    const int nblk = npairs * nqt;
    if ((npairs & 7) == 0) {
      const int xcd = bid & 7, i = bid >> 3;
      const int per = npairs >> 3;            // pairs owned by this XCD
      pair = xcd * per + i % per;
      qt = nqt - 1 - i / per;
    } else {
      pair = bid % npairs;
      qt = nqt - 1 - bid / npairs;
    }
    (void)nblk;
  }
  const int g = pair % a.n_kv, w = pair / a.n_kv;
  if (a.prune) {
    // final layer: window k's first scored position is 0 for k = 0, else
    // min(L - S, P - kS); query tiles before it are not needed
    const int64_t k = a.k0 + w;
    const int64_t j0 = (k == 0) ? 0 : min((int64_t)(a.L - a.S), a.P - k * a.S);
    if (qt < (int)(j0 / 64)) return;
  }
  const int head = 2 * g + (wave >> 1);
  const int qbase = qt * 64 + 32 * (wave & 1);
  const int nkt = qt + 1;

  if constexpr (HDP > HD) {
    for (int i = tid; i < 2 * 64 * (HDP - HD); i += 256) {
      int b = i / (64 * (HDP - HD)), rem = i % (64 * (HDP - HD));
      int r = rem / (HDP - HD), c = HD + rem % (HDP - HD);
      Ks[b][r * KLD + c] = (act)0.0f;
    }
  }

  const act* Qh = a.q + ((int64_t)w * a.n_heads + head) * a.Lp * HD;
  const act* Kg = a.k + ((int64_t)w * a.n_kv + g) * a.Lp * HD;
  const act* Vg = a.vt + ((int64_t)w * a.n_kv + g) * HD * a.Lp;

  actx8 qf[2][KS];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      int d0 = ks * 32 + 8 * lg;
      if (d0 < HD)
        qf[qb][ks] = *reinterpret_cast<const actx8*>(Qh + (int64_t)(qbase + 16 * qb + lr) * HD + d0);
      else
        qf[qb][ks] = actx8{};
    }

  // Register staging, up to three 16-byte chunks per thread and tile, as
  // named scalars (arrays of them end up in scratch memory).
  static_assert(KPER <= 3 && VPER <= 3, "staging holds three chunks per thread");
  uint4 kreg_0, kreg_1, kreg_2, vreg_0, vreg_1, vreg_2;
  // Chunk indices past the tile are clamped: those threads reload and rewrite
  // the last chunk with identical data.
#define ATT_CHUNKS(PER, R, BODY) \
  { if constexpr ((PER) > 0) { constexpr int i = 0; uint4& r_ = R##_0; BODY } \
    if constexpr ((PER) > 1) { constexpr int i = 1; uint4& r_ = R##_1; BODY } \
    if constexpr ((PER) > 2) { constexpr int i = 2; uint4& r_ = R##_2; BODY } }
#define ATT_LOAD_K(kt, R)                                                             \
  {                                                                                   \
    const int64_t k0_ = (int64_t)(kt) * 64;                                           \
    ATT_CHUNKS(KPER, R, { int c = min(tid + 256 * i, KCH - 1);                           \
                       r_ = *reinterpret_cast<const uint4*>(Kg + k0_ * HD + c * 8); }) \
  }
#define ATT_LOAD_V(kt, R)                                                             \
  {                                                                                   \
    const int k0_ = (kt) * 64;                                                        \
    ATT_CHUNKS(VPER, R, { int c = min(tid + 256 * i, VCH - 1);                           \
                       r_ = *reinterpret_cast<const uint4*>(Vg + (int64_t)(c >> 3) * a.Lp + k0_ + (c & 7) * 8); }) \
  }
#define ATT_STORE_K(buf, R)                                                           \
  ATT_CHUNKS(KPER, R, { int c = min(tid + 256 * i, KCH - 1);                             \
                     const int kr_ = key_row(c / (HD / 8));                             \
                     const int kc_ = c % (HD / 8);                                      \
                     *reinterpret_cast<uint4*>(&Ks[buf][kr_ * KLD + (KSWZ ? swz(kr_, kc_) : kc_) * 8]) = r_; })
#define ATT_STORE_V(buf, R)                                                           \
  ATT_CHUNKS(VPER, R, { int c = min(tid + 256 * i, VCH - 1);                             \
                     *reinterpret_cast<uint4*>(&Vs[buf][(c >> 3) * VLD + swz(c >> 3, c & 7) * 8]) = r_; })
  // S^T for one key tile: row lr of block kb reads LDS row 16 kb + lr.
#define ATT_QK(dst, buf)                                                              \
  {                                                                                   \
    _Pragma("unroll") for (int kb = 0; kb < 4; ++kb) {                                \
      const int kr = 16 * kb + lr;                                                    \
      actx8 kf[KS];                                                                  \
      _Pragma("unroll") for (int ks = 0; ks < KS; ++ks) {                             \
        const int ch = ks * 4 + lg;                                                   \
        kf[ks] = *reinterpret_cast<const actx8*>(&Ks[buf][kr * KLD + (KSWZ ? swz(kr, ch) : ch) * 8]); \
      }                                                                               \
      _Pragma("unroll") for (int qb = 0; qb < 2; ++qb) {                              \
        f32x4 acc_ = f32x4{0.f, 0.f, 0.f, 0.f};                                       \
        _Pragma("unroll") for (int ks = 0; ks < KS; ++ks)                             \
          acc_ = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf[ks], qf[qb][ks], acc_, 0, 0, 0); \
        dst[qb][kb] = acc_;                                                           \
      }                                                                               \
    }                                                                                 \
  }

  f32x4 o[2][DB];
  f32x4 osum[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
    for (int db = 0; db < DB; ++db) o[qb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
    osum[qb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  actx8 ones;
#pragma unroll
  for (int i = 0; i < 8; ++i) ones[i] = (act)1.0f;
  float mref[2] = {-1e30f, -1e30f};
  const float c = a.scale_log2;

  // prologue: LDS holds K[0] and V[0]
  ATT_LOAD_K(0, kreg);
  ATT_LOAD_V(0, vreg);
  ATT_STORE_K(0, kreg);
  ATT_STORE_V(0, vreg);
  __syncthreads();
  f32x4 s_cur[2][4];

  // One key tile: S^T of tile kt into SC, softmax, O^T += V^T P^T.  The
  // registers KR/VR receive K[kt+1] and V[kt+1], written to LDS at the end
  // into the buffers tile kt-1 used (read before the previous barrier).
  // DIAG is true only for the last tile, the one that straddles the causal
  // diagonal.
  //
  // The probabilities use a per-query reference max mref that is only moved
  // when the tile max exceeds it by more than 2^8 in the exp2 domain (or on
  // the first tile); otherwise p <= 256 and O, the denominator and the final
  // O / denominator are unchanged by the choice of reference, so the rescale
  // of O (and its multiplies) is skipped on almost every tile.
#define ATT_STEP(kt, SC, KR, VR, DIAG)                                                 \
  {                                                                                   \
    ATT_LOAD_K(min((kt) + 1, nkt - 1), KR);                                           \
    ATT_LOAD_V(min((kt) + 1, nkt - 1), VR);                                           \
    ATT_QK(SC, (kt) & 1);                                                             \
    if (DIAG) {                                                                       \
      _Pragma("unroll") for (int qb = 0; qb < 2; ++qb) {                              \
        const int qabs = qbase + 16 * qb + lr;                                        \
        _Pragma("unroll") for (int kb = 0; kb < 4; ++kb)                              \
          _Pragma("unroll") for (int i = 0; i < 4; ++i) {                             \
            int kabs = (kt) * 64 + 32 * (kb >> 1) + 8 * lg + 4 * (kb & 1) + i;        \
            if (kabs > qabs) SC[qb][kb][i] = -1e30f;                                  \
          }                                                                           \
      }                                                                               \
    }                                                                                 \
    float mt[2];                                                                      \
    bool grow = false;                                                                \
    _Pragma("unroll") for (int qb = 0; qb < 2; ++qb) {                                \
      float m_ = SC[qb][0][0];                                                        \
      _Pragma("unroll") for (int kb = 0; kb < 4; ++kb)                                \
        _Pragma("unroll") for (int i = 0; i < 4; ++i) m_ = __builtin_fmaxf(m_, SC[qb][kb][i]); \
      m_ = max_xor16(m_);                                                             \
      mt[qb] = max_xor32(m_);                                                         \
      grow |= (mt[qb] - mref[qb]) * c > 8.0f;                                         \
    }                                                                                 \
    if (__any(grow)) {                                                                \
      _Pragma("unroll") for (int qb = 0; qb < 2; ++qb) {                              \
        const float mnew = __builtin_fmaxf(mref[qb], mt[qb]);                         \
        const float alpha = __builtin_amdgcn_exp2f((mref[qb] - mnew) * c);            \
        mref[qb] = mnew;                                                              \
        _Pragma("unroll") for (int db = 0; db < DB; ++db) o[qb][db] *= alpha;         \
        osum[qb] *= alpha;                                                            \
      }                                                                               \
    }                                                                                 \
    actx8 pf[2][2];                                                                  \
    _Pragma("unroll") for (int qb = 0; qb < 2; ++qb) {                                \
      const float mc = mref[qb] * c;                                                  \
      _Pragma("unroll") for (int kk = 0; kk < 2; ++kk) {                              \
        f32x8 v;                                                                      \
        _Pragma("unroll") for (int i = 0; i < 4; ++i) {                               \
          v[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(SC[qb][2 * kk][i], c, -mc));   \
          v[4 + i] = __builtin_amdgcn_exp2f(__builtin_fmaf(SC[qb][2 * kk + 1][i], c, -mc)); \
        }                                                                             \
        pf[qb][kk] = __builtin_convertvector(v, actx8); /* v_cvt_pk_f16_f32, nearest even */ \
      }                                                                               \
    }                                                                                 \
    const int vb_ = (kt) & 1;                                                         \
    _Pragma("unroll") for (int kk = 0; kk < 2; ++kk) {                                \
      _Pragma("unroll") for (int db = 0; db < DB; ++db) {                             \
        const int vr_ = db * 16 + lr;                                                 \
        actx8 vf = *reinterpret_cast<const actx8*>(&Vs[vb_][vr_ * VLD + swz(vr_, 4 * kk + lg) * 8]); \
        _Pragma("unroll") for (int qb = 0; qb < 2; ++qb)                              \
          o[qb][db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, pf[qb][kk], o[qb][db], 0, 0, 0); \
      }                                                                               \
      _Pragma("unroll") for (int qb = 0; qb < 2; ++qb)                                \
        osum[qb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, pf[qb][kk], osum[qb], 0, 0, 0); \
    }                                                                                 \
    if (!(DIAG)) {                                                                    \
      /* K[kt+1] and V[kt+1] replace tile kt-1's; the barrier publishes */            \
      /* them for the next step. */                                                   \
      ATT_STORE_K(((kt) + 1) & 1, KR);                                                \
      ATT_STORE_V(((kt) + 1) & 1, VR);                                                \
      __syncthreads();                                                                \
    }                                                                                 \
  }

  // the diagonal tile is the last one (kt = qt): peel it off the loop
  int kt = 0;
  for (; kt + 2 < nkt; kt += 2) {
    ATT_STEP(kt, s_cur, kreg, vreg, false);
    ATT_STEP(kt + 1, s_cur, kreg, vreg, false);
  }
  if (nkt - kt == 2) {
    ATT_STEP(kt, s_cur, kreg, vreg, false);
    ATT_STEP(kt + 1, s_cur, kreg, vreg, true);
  } else {
    ATT_STEP(kt, s_cur, kreg, vreg, true);
  }
#undef ATT_STEP
#undef ATT_LOAD_K
#undef ATT_LOAD_V
#undef ATT_STORE_K
#undef ATT_STORE_V
#undef ATT_CHUNKS
#undef ATT_QK

  // Output rows: a lane holds dims db*16 + 4*lg + i of query q; the four
  // lane groups (lanes lr, lr^16, lr^32, lr^48) together hold the row.
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float inv = 1.0f / osum[qb][0];
    const int q = qbase + 16 * qb + lr;
    act* dst = a.o + ((int64_t)w * a.Lp + q) * (a.n_heads * HD) + head * HD;
    float ov[DB][4];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) ov[db][i] = o[qb][db][i] * inv;
    if (a.xsa) {
      // exclusive self attention ([363] XSA): remove the component along
      // this position's value vector v (binary16, as the P.V product used it)
      float vv[DB][4], dot = 0.0f, nn = 0.0f;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          vv[db][i] = (float)Vg[(int64_t)(db * 16 + 4 * lg + i) * a.Lp + q];
          dot += ov[db][i] * vv[db][i];
          nn += vv[db][i] * vv[db][i];
        }
      dot += __shfl_xor(dot, 16);
      dot += __shfl_xor(dot, 32);
      nn += __shfl_xor(nn, 16);
      nn += __shfl_xor(nn, 32);
      const float coef = nn > 0.0f ? dot / nn : 0.0f;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) ov[db][i] -= coef * vv[db][i];
    }
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      *reinterpret_cast<uint2*>(dst + db * 16 + 4 * lg) =
          make_uint2(pack2h(ov[db][0], ov[db][1]), pack2h(ov[db][2], ov[db][3]));
    }
  }
}

}  // namespace

hipError_t launch_attention(const AttnArgs& a, hipStream_t s) {
  dim3 grid((unsigned)(a.Lp / 64) * a.n_kv * a.W);
  switch (a.hd) {
    case 32: hipLaunchKernelGGL(attn_kernel<32>, grid, dim3(256), 0, s, a); break;
    case 64: hipLaunchKernelGGL(attn_kernel<64>, grid, dim3(256), 0, s, a); break;
    case 80: hipLaunchKernelGGL(attn_kernel<80>, grid, dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace i6g
