// Causal grouped-query attention over a batch of windows, flash style.
//
// pwwt.cn "parameter-golf 16MB 极限压缩实战 …", section 架构：11 层 U-Net 变压器:
// GQA with 8 query and 4 KV heads and RoPE (applied by the projection
// epilogue).  Query head h reads KV head h / 2; scores are q.k / sqrt(hd)
// with a causal mask inside each window; softmax over keys 0..j.
//
// One workgroup = (window, KV head, 64 queries) and both query heads of the
// group, so each K/V tile brought into LDS serves 128 query rows.  Each of
// the 4 waves owns 32 queries of one head.  The scores are formed transposed,
// S^T = K Q^T, with v_mfma_f32_16x16x32_bf16: a lane's accumulator then
// holds one query and 4 keys, so the running max and sum of a query live in
// one lane group and the softmax needs only two cross-lane steps for the
// max.  The keys feeding the S^T rows are permuted so that the probabilities
// a lane holds are exactly the 8 consecutive keys the B operand of
// O^T += V^T P^T wants; P never leaves registers.  exp is exp2 with the
// 1/sqrt(hd) * log2(e) factor folded into one multiply-add.
#include "common.h"

namespace i6g {
namespace {

template <int HD>
__global__ __launch_bounds__(256) void attn_kernel(AttnArgs a) {
  constexpr int KS = (HD + 31) / 32;  // 32-wide k steps over the head dim
  constexpr int HDP = KS * 32;
  constexpr int DB = HD / 16;         // 16-row blocks of O^T
  constexpr int KLD = HDP + 8;
  constexpr int VLD = 64 + 8;
  constexpr int KCH = 64 * HD / 8;    // 16-byte chunks per K tile
  constexpr int VCH = HD * 64 / 8;    // 16-byte chunks per V^T tile
  constexpr int KPER = (KCH + 255) / 256;
  constexpr int VPER = (VCH + 255) / 256;

  __shared__ __attribute__((aligned(16))) bf16 Ks[2][64 * KLD];
  __shared__ __attribute__((aligned(16))) bf16 Vs[2][HD * VLD];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int nqt = a.Lp / 64;
  const int qt = nqt - 1 - (int)blockIdx.x;  // longest rows first
  const int g = blockIdx.y, w = blockIdx.z;
  const int head = 2 * g + (wave >> 1);
  const int qbase = qt * 64 + 32 * (wave & 1);

  if constexpr (HDP > HD) {
    for (int i = tid; i < 2 * 64 * (HDP - HD); i += 256) {
      int b = i / (64 * (HDP - HD)), rem = i % (64 * (HDP - HD));
      int r = rem / (HDP - HD), c = HD + rem % (HDP - HD);
      Ks[b][r * KLD + c] = (bf16)0.0f;
    }
  }

  const bf16* Qh = a.q + ((int64_t)w * a.n_heads + head) * a.Lp * HD;
  const bf16* Kg = a.k + ((int64_t)w * a.n_kv + g) * a.Lp * HD;
  const bf16* Vg = a.vt + ((int64_t)w * a.n_kv + g) * HD * a.Lp;

  bf16x8 qf[2][KS];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      int d0 = ks * 32 + 8 * lg;
      if (d0 < HD)
        qf[qb][ks] = *reinterpret_cast<const bf16x8*>(Qh + (int64_t)(qbase + 16 * qb + lr) * HD + d0);
      else
        qf[qb][ks] = bf16x8{};
    }

  uint4 kreg[KPER], vreg[VPER];
  auto load_tile = [&](int kt) {
    const int k0 = kt * 64;
#pragma unroll
    for (int i = 0; i < KPER; ++i) {
      int c = tid + 256 * i;
      if (c < KCH) kreg[i] = *reinterpret_cast<const uint4*>(Kg + (int64_t)k0 * HD + c * 8);
    }
#pragma unroll
    for (int i = 0; i < VPER; ++i) {
      int c = tid + 256 * i;
      if (c < VCH) {
        int d = c >> 3, c8 = (c & 7) * 8;
        vreg[i] = *reinterpret_cast<const uint4*>(Vg + (int64_t)d * a.Lp + k0 + c8);
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < KPER; ++i) {
      int c = tid + 256 * i;
      if (c < KCH) {
        int r = c / (HD / 8), c8 = (c % (HD / 8)) * 8;
        *reinterpret_cast<uint4*>(&Ks[buf][r * KLD + c8]) = kreg[i];
      }
    }
#pragma unroll
    for (int i = 0; i < VPER; ++i) {
      int c = tid + 256 * i;
      if (c < VCH) {
        int d = c >> 3, c8 = (c & 7) * 8;
        *reinterpret_cast<uint4*>(&Vs[buf][d * VLD + c8]) = vreg[i];
      }
    }
  };

  f32x4 o[2][DB];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int db = 0; db < DB; ++db) o[qb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float mrow[2] = {-1e30f, -1e30f};
  float lrow[2] = {0.f, 0.f};
  const float c = a.scale_log2;

  const int nkt = qt + 1;
  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int kt = 0; kt < nkt; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nkt) load_tile(kt + 1);
    const bf16* ks_ = Ks[buf];
    const bf16* vs_ = Vs[buf];

    f32x4 s[2][4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      // S^T row lr of block kb reads physical key pk (see header comment)
      const int pk = 32 * (kb >> 1) + 8 * (lr >> 2) + 4 * (kb & 1) + (lr & 3);
      bf16x8 kf[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        kf[ks] = *reinterpret_cast<const bf16x8*>(ks_ + pk * KLD + ks * 32 + 8 * lg);
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[ks], qf[qb][ks], acc, 0, 0, 0);
        s[qb][kb] = acc;
      }
    }

    const bool diag = (kt == qt);
    bf16x8 pf[2][2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int qabs = qbase + 16 * qb + lr;
      if (diag) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            int kabs = kt * 64 + 32 * (kb >> 1) + 8 * lg + 4 * (kb & 1) + i;
            if (kabs > qabs) s[qb][kb][i] = -1e30f;
          }
      }
      float mt = s[qb][0][0];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) mt = fmaxf(mt, s[qb][kb][i]);
      mt = fmaxf(mt, __shfl_xor(mt, 16));
      mt = fmaxf(mt, __shfl_xor(mt, 32));
      const float mnew = fmaxf(mrow[qb], mt);
      const float alpha = exp2f((mrow[qb] - mnew) * c);
      const float mc = mnew * c;
      mrow[qb] = mnew;
      float ls = 0.f;
      float p[4][4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p[kb][i] = exp2f(s[qb][kb][i] * c - mc);
          ls += p[kb][i];
        }
      lrow[qb] = lrow[qb] * alpha + ls;
#pragma unroll
      for (int db = 0; db < DB; ++db) o[qb][db] *= alpha;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        bf16x8 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[i] = (bf16)p[2 * kk][i];
          v[4 + i] = (bf16)p[2 * kk + 1][i];
        }
        pf[qb][kk] = v;
      }
    }

#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        bf16x8 vf = *reinterpret_cast<const bf16x8*>(vs_ + (db * 16 + lr) * VLD + 32 * kk + 8 * lg);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
          o[qb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[qb][kk], o[qb][db], 0, 0, 0);
      }

    if (kt + 1 < nkt) store_tile(buf ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    float l = lrow[qb];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    const float inv = 1.0f / l;
    const int q = qbase + 16 * qb + lr;
    bf16* dst = a.o + ((int64_t)w * a.Lp + q) * (a.n_heads * HD) + head * HD;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      uint16_t y[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        y[i] = __builtin_bit_cast(uint16_t, (bf16)(o[qb][db][i] * inv));
      *reinterpret_cast<uint2*>(dst + db * 16 + 4 * lg) =
          make_uint2((uint32_t)y[0] | ((uint32_t)y[1] << 16), (uint32_t)y[2] | ((uint32_t)y[3] << 16));
    }
  }
}

}  // namespace

hipError_t launch_attention(const AttnArgs& a, hipStream_t s) {
  dim3 grid(a.Lp / 64, a.n_kv, a.W);
  switch (a.hd) {
    case 32: hipLaunchKernelGGL(attn_kernel<32>, grid, dim3(256), 0, s, a); break;
    case 64: hipLaunchKernelGGL(attn_kernel<64>, grid, dim3(256), 0, s, a); break;
    case 80: hipLaunchKernelGGL(attn_kernel<80>, grid, dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace i6g
