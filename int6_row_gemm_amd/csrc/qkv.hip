// q/k/v projection on gfx950 MFMA for d_model 512 and head size 64: one
// 128-row tile of the normed layer input per workgroup, all q, k and v heads
// of it (pwwt.cn "parameter-golf 16MB 极限压缩实战 …", 架构: GQA attention with
// RoPE on q and k; one binary16 scale per weight row, 后训练量化导出).
//
// The tile's binary16 rows (128 x 512, 128 KB) go into LDS once by direct
// loads; the eight waves then take whole heads (wave w: heads w, w + 8, ..),
// each a 128 x 64 block accumulated over K = 512 in eight steps of 64, the
// code fragments loaded from global memory straight into registers half a
// step ahead (codes rearranged once at load time into per-head fragment
// order, launch_shuffle_qkv_codes).  No barrier after the tile has landed.
//
//   q and k heads accumulate C^T, with the head's weight rows placed so that
//   a lane holds whole rotation pairs (rope_phys): * scale * rinv, RoPE from
//   the (cos, sin) table, two 16-byte runs per row into Q [W, Hq, Lp, 64] or
//   K [W, Hkv, Lp, 64];
//   v heads accumulate C, so a lane holds 16 consecutive positions of one
//   column: * scale * rinv, two 16-byte stores into V^T [W, Hkv, 64, Lp].
//
// rinv = 1/sqrt(sum of the row's partial sums of squares / 512 + eps) is
// applied in fp32 to the accumulators, as in the LDS-staged GEMM, so both
// paths round the same products the same way.
#include <type_traits>

#include "common.h"
#include "mfma_util.h"

namespace i6g {
namespace {

constexpr int TM = 128;                 // rows per tile
constexpr int NB = TM / 16;             // 16-row blocks per tile
constexpr int DM = 512;                 // model width (K)
constexpr int HD = 64;                  // head size
constexpr int NW = 8;                   // waves
constexpr int NTH = 64 * NW;            // threads
constexpr int ABYTES = TM * DM * 2;     // 131072
constexpr int HSTEP = 4 * 64 * 16;      // one head, one K step of 64: four 1 KB fragments
constexpr int NK = DM / 64;             // K steps
constexpr int MAXN = 2048;              // output columns (32 heads) whose scales are staged in LDS

__device__ inline int phys_row(int r) { return (r & ~63) | perm16(r & 63); }
// byte offset of 16-byte chunk c of physical row p of the A tile (1 KB rows,
// slot c ^ 2(p & 15): every LDS pass of a fragment read, 16 rows x two
// adjacent chunks, touches 32 distinct 16-byte bank groups)
__device__ inline int a_off(int p, int c) { return p * (DM * 2) + ((c ^ (2 * (p & 15))) << 4); }

typedef __attribute__((address_space(1))) void* gptr_t;
typedef __attribute__((address_space(3))) void* lptr_t;

__global__ __launch_bounds__(NTH) __attribute__((amdgpu_waves_per_eu(2, 2))) void qkv_kernel(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) char As[ABYTES];
  __shared__ __attribute__((aligned(16))) float rinv_s[TM];
  __shared__ __attribute__((aligned(16))) float sc_s[MAXN];

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, lr = lane & 15, lg = lane >> 4;
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
  // the lane's 16-byte offset, recomputed where used (see the block tail)
  auto loff16 = [&]() -> uint32_t {
    uint32_t l;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
    return l << 4;
  };
  uint4 cq0, cq1, cq2, cq3;
  // the four fragments of head h, K step kt (offsets below 2^31: at most
  // 32 heads x 8 steps x 4 KB)
  auto load4 = [&](int h, int kt) {
    const int8_t* b = a.Bp + (h * NK + kt) * HSTEP;
    const uint32_t l = loff16();
    cq0 = *reinterpret_cast<const uint4*>(b + l);
    cq1 = *reinterpret_cast<const uint4*>(b + 1024 + l);
    cq2 = *reinterpret_cast<const uint4*>(b + 2048 + l);
    cq3 = *reinterpret_cast<const uint4*>(b + 3072 + l);
  };
  if (w < nall) load4(w, 0);
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

  // One K step: the first 32 codes of each fragment are widened and used,
  // then the other 32; the next step's loads take the code registers after
  // the second widening, fenced above the MFMAs.  CT: q/k heads (C^T).
  auto kstep = [&](auto ct, f32x4 (&acc)[NB][4], int kc0, auto&& next_load) {
    constexpr bool CT = decltype(ct)::value;
    asm volatile("" : "+s"(kc0));   // LDS addresses computed where used, not held
    {
      const actx8 wf[4] = {widen8(cq0.x, cq0.y), widen8(cq1.x, cq1.y), widen8(cq2.x, cq2.y), widen8(cq3.x, cq3.y)};
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const actx8 af = *reinterpret_cast<const actx8*>(As + a_off(16 * i + lr, kc0 + lg));
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = CT ? __builtin_amdgcn_mfma_f32_16x16x32_f16(wf[j], af, acc[i][j], 0, 0, 0)
                         : __builtin_amdgcn_mfma_f32_16x16x32_f16(af, wf[j], acc[i][j], 0, 0, 0);
      }
    }
    const actx8 wf[4] = {widen8(cq0.z, cq0.w), widen8(cq1.z, cq1.w), widen8(cq2.z, cq2.w), widen8(cq3.z, cq3.w)};
    next_load();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const actx8 af = *reinterpret_cast<const actx8*>(As + a_off(16 * i + lr, kc0 + 4 + lg));
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = CT ? __builtin_amdgcn_mfma_f32_16x16x32_f16(wf[j], af, acc[i][j], 0, 0, 0)
                       : __builtin_amdgcn_mfma_f32_16x16x32_f16(af, wf[j], acc[i][j], 0, 0, 0);
    }
  };

  // the tile's first window and position (Lp >= TM, so a row block lies in
  // this window or the next)
  const int win0 = m0 / a.Lp, pos0 = m0 - win0 * a.Lp;

  auto pass = [&](auto ct, int h) {
    constexpr bool CT = decltype(ct)::value;
    f32x4 acc[NB][4];
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
    for (int kt = 0; kt < NK - 1; ++kt) kstep(ct, acc, 8 * kt, [&] { load4(h, kt + 1); });
    kstep(ct, acc, 8 * (NK - 1), [] {});
    // the epilogue's loads stay below the last MFMAs
    __builtin_amdgcn_sched_barrier(0);
    // the next head's first codes, loaded once this head's values are out
    // of the accumulators and before its stores (so their wait does not
    // include the stores)
    auto prefetch_next = [&] {
      if (h + NW < nall) load4(h + NW, 0);
      __builtin_amdgcn_sched_barrier(0);
    };

    // opaque copies of the lane's row and column indices and of the tile
    // position: the epilogue's addresses are recomputed in every pass
    // rather than hoisted out of the head loop and held (they would spill)
    int lrv = lr, lgv = lg, m0v = m0, pos0v = pos0, win0v = win0;
    asm volatile("" : "+v"(lrv), "+v"(lgv), "+s"(m0v), "+s"(pos0v), "+s"(win0v));
    auto erow = [&](int i) { return 64 * (i >> 2) + 16 * (lrv >> 2) + (lrv & 3) + 4 * (i & 3); };
    if constexpr (CT) {
      // q or k head: the lane holds rotation pairs c1b + t, t < 8, whose
      // first dims are f0 + t and second dims s0 + t
      const bool is_q = h < a.n_heads;
      const int head = is_q ? h : h - a.n_heads;
      const int nh = is_q ? a.n_heads : a.n_kv;
      act* const base = is_q ? a.q : a.k;
      const int c1b = 8 * lgv;
      const int f0 = pair_first<HD>(c1b, a.rope_dims), s0 = pair_second<HD>(c1b, a.rope_dims);
      float sc1[8], sc2[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        sc1[t] = sc_s[h * HD + f0 + t];
        sc2[t] = sc_s[h * HD + s0 + t];
      }
      // (cos, sin) of the row's 8 pairs, loaded one row block ahead and
      // before the previous block's stores (a load issued after a store
      // waits for it on this hardware's single vector-memory counter)
      auto cs_of = [&](int i, float4 (&cs)[4]) {
        int pos = pos0v + erow(i);
        if (pos >= a.Lp) pos -= a.Lp;
        const float4* csp = reinterpret_cast<const float4*>(a.rope + pos * (HD / 2) + c1b);
#pragma unroll
        for (int q = 0; q < 4; ++q) cs[q] = csp[q];
      };
      float4 csn[4];
      cs_of(0, csn);
      prefetch_next();
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const float4 cs[4] = {csn[0], csn[1], csn[2], csn[3]};
        const float r = rinv_s[erow(i)];
        float x1[8], x2[8], y1[8], y2[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          x1[t] = acc[i][t >> 2][t & 3] * sc1[t] * r;
          x2[t] = acc[i][(t + 8) >> 2][(t + 8) & 3] * sc2[t] * r;
        }
        {
          // every product rounded on its own, as in the LDS-staged GEMM
#pragma clang fp contract(off)
#pragma unroll
          for (int t = 0; t < 8; t += 2) {
            const float4 c = cs[t / 2];   // (cos, sin) of pairs c1b + t and c1b + t + 1
            y1[t] = x1[t] * c.x - x2[t] * c.y;
            y2[t] = x1[t] * c.y + x2[t] * c.x;
            y1[t + 1] = x1[t + 1] * c.z - x2[t + 1] * c.w;
            y2[t + 1] = x1[t + 1] * c.w + x2[t + 1] * c.z;
          }
        }
        if (i + 1 < NB) cs_of(i + 1, csn);
        __builtin_amdgcn_sched_barrier(0);
        const int ml = erow(i);
        if (m0v + ml < a.M) {
          int pos = pos0v + ml, win = win0v;
          if (pos >= a.Lp) {
            pos -= a.Lp;
            ++win;
          }
          act* dst = base + (((int64_t)win * nh + head) * a.Lp + pos) * HD;
          *reinterpret_cast<uint4*>(dst + f0) =
              make_uint4(pack2h(y1[0], y1[1]), pack2h(y1[2], y1[3]), pack2h(y1[4], y1[5]), pack2h(y1[6], y1[7]));
          *reinterpret_cast<uint4*>(dst + s0) =
              make_uint4(pack2h(y2[0], y2[1]), pack2h(y2[2], y2[3]), pack2h(y2[4], y2[5]), pack2h(y2[6], y2[7]));
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      // v head, C: in 64-row slice s the lane holds rows 64 s + 16 lg + t,
      // t < 16 (consecutive positions of one window), of column 16 j + lr
      const int head = h - nqk;
      prefetch_next();
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int ml = 64 * s + 16 * lgv;
        if (m0v + ml >= a.M) continue;
        float rv[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 r4 = reinterpret_cast<const float4*>(rinv_s + ml)[q];
          rv[4 * q] = r4.x; rv[4 * q + 1] = r4.y; rv[4 * q + 2] = r4.z; rv[4 * q + 3] = r4.w;
        }
        int pos = pos0v + ml, win = win0v;
        if (pos >= a.Lp) {
          pos -= a.Lp;
          ++win;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int dd = 16 * j + lrv;
          const float sc = sc_s[h * HD + dd];
          float y[16];
#pragma unroll
          for (int t = 0; t < 16; ++t) y[t] = acc[4 * s + (t >> 2)][j][t & 3] * sc * rv[t];
          uint4* dst = reinterpret_cast<uint4*>(a.vt + (((int64_t)win * a.n_kv + head) * HD + dd) * a.Lp + pos);
          dst[0] = make_uint4(pack2h(y[0], y[1]), pack2h(y[2], y[3]), pack2h(y[4], y[5]), pack2h(y[6], y[7]));
          dst[1] = make_uint4(pack2h(y[8], y[9]), pack2h(y[10], y[11]), pack2h(y[12], y[13]), pack2h(y[14], y[15]));
        }
      }
    }
  };

  for (int h = w; h < nall; h += NW) {
    if (h < nqk) pass(std::true_type{}, h);
    else pass(std::false_type{}, h);
  }
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
