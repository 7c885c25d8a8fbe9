// The per-head loop of the one-tile q/k/v projection (d_model 512, head
// size 64), shared by the q/k/v kernel and by the block tail that computes
// the next layer's q, k and v from its own output rows (pwwt.cn
// "parameter-golf 16MB 极限压缩实战 …", 架构: GQA attention with RoPE on q and
// k; one binary16 scale per weight row, 后训练量化导出).
//
// The caller holds a 128-row tile of binary16 layer-input rows in LDS (1 KB
// rows placed by perm16 within 64-row slices, 16-byte chunk c of physical
// row p in slot c ^ 2(p & 15)), the rows' RMS factors and the projection's
// per-column scales (as floats) in LDS, and the first K step of its first
// head's codes in four registers.  Wave w then computes heads w, w + 8, ..
// as 128 x 64 blocks over K = 512 in eight steps of 64, code fragments
// loaded from global memory straight into registers half a step ahead:
//
//   q and k heads accumulate C^T, with the head's weight rows placed so that
//   a lane holds whole rotation pairs (rope_phys): * scale * rinv, RoPE from
//   the (cos, sin) table, two 16-byte runs per row into Q [W, Hq, Lp, 64] or
//   K [W, Hkv, Lp, 64];
//   v heads accumulate C, so a lane holds 16 consecutive positions of one
//   column: * scale * rinv, two 16-byte stores into V^T [W, Hkv, 64, Lp].
#pragma once

#include <type_traits>

#include "common.h"
#include "mfma_util.h"

namespace i6g {
namespace qkvp {

constexpr int TM = 128;                 // rows per tile
constexpr int NB = TM / 16;             // 16-row blocks per tile
constexpr int DM = 512;                 // model width (K)
constexpr int HD = 64;                  // head size
constexpr int NW = 8;                   // waves
constexpr int HSTEP = 4 * 64 * 16;      // one head, one K step of 64: four 1 KB fragments
constexpr int NK = DM / 64;             // K steps
constexpr int MAXN = 2048;              // output columns (32 heads) whose scales fit the callers' LDS

// byte offset of 16-byte chunk c of physical row p of the A tile
__device__ inline int a_off(int p, int c) { return p * (DM * 2) + ((c ^ (2 * (p & 15))) << 4); }

// the lane's 16-byte offset, recomputed where used (under full register
// pressure a held copy is spilled, and its reload waits for every load in
// flight)
__device__ __forceinline__ uint32_t loff16() {
  uint32_t l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l << 4;
}

// the four fragments of head h, K step kt (offsets below 2^31: at most 32
// heads x 8 steps x 4 KB)
__device__ __forceinline__ void load4(const int8_t* frag, int h, int kt, uint4& c0, uint4& c1, uint4& c2, uint4& c3) {
  const int8_t* b = frag + (h * NK + kt) * HSTEP;
  const uint32_t l = loff16();
  c0 = *reinterpret_cast<const uint4*>(b + l);
  c1 = *reinterpret_cast<const uint4*>(b + 1024 + l);
  c2 = *reinterpret_cast<const uint4*>(b + 2048 + l);
  c3 = *reinterpret_cast<const uint4*>(b + 3072 + l);
}

// Every head of the tile that starts at row m0 (M rows in all, windows of
// Lp >= TM rows) for wave w; cq0 .. cq3 hold head w's first K step.
__device__ __forceinline__ void heads(const QkvOut& a, int M, int Lp, const char* As, const float* rinv_s,
                                      const float* sc_s, int m0, int w, uint4& cq0, uint4& cq1, uint4& cq2,
                                      uint4& cq3) {
  // the lane index from an opaque mbcnt, so that nothing of this loop is
  // merged with a caller's values computed earlier (a block tail would
  // then hold them through its own loops)
  const int lane = (int)(loff16() >> 4), lr = lane & 15, lg = lane >> 4;
  const int nqk = a.n_heads + a.n_kv, nall = nqk + a.n_kv;
  auto load4h = [&](int h, int kt) { load4(a.frag, h, kt, cq0, cq1, cq2, cq3); };

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
  const int win0 = m0 / Lp, pos0 = m0 - win0 * Lp;

  auto pass = [&](auto ct, int h) {
    constexpr bool CT = decltype(ct)::value;
    f32x4 acc[NB][4];
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
    for (int kt = 0; kt < NK - 1; ++kt) kstep(ct, acc, 8 * kt, [&] { load4h(h, kt + 1); });
    kstep(ct, acc, 8 * (NK - 1), [] {});
    // the epilogue's loads stay below the last MFMAs
    __builtin_amdgcn_sched_barrier(0);
    // the next head's first codes, loaded once this head's values are out
    // of the accumulators and before its stores (so their wait does not
    // include the stores)
    auto prefetch_next = [&] {
      if (h + NW < nall) load4h(h + NW, 0);
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
        if (pos >= Lp) pos -= Lp;
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
        if (m0v + ml < M) {
          int pos = pos0v + ml, win = win0v;
          if (pos >= Lp) {
            pos -= Lp;
            ++win;
          }
          act* dst = base + (((int64_t)win * nh + head) * Lp + pos) * HD;
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
        if (m0v + ml >= M) continue;
        float rv[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 r4 = reinterpret_cast<const float4*>(rinv_s + ml)[q];
          rv[4 * q] = r4.x; rv[4 * q + 1] = r4.y; rv[4 * q + 2] = r4.z; rv[4 * q + 3] = r4.w;
        }
        int pos = pos0v + ml, win = win0v;
        if (pos >= Lp) {
          pos -= Lp;
          ++win;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int dd = 16 * j + lrv;
          const float sc = sc_s[h * HD + dd];
          float y[16];
#pragma unroll
          for (int t = 0; t < 16; ++t) y[t] = acc[4 * s + (t >> 2)][j][t & 3] * sc * rv[t];
          uint4* dst = reinterpret_cast<uint4*>(a.vt + (((int64_t)win * a.n_kv + head) * HD + dd) * Lp + pos);
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

}  // namespace qkvp
}  // namespace i6g
