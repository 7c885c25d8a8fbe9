// Fused block tail on gfx950 MFMA, d_model = 512: the attention output
// projection with its residual add, the RMSNorm of the result, and the
// ReLU^2 MLP with its residual add, for one 128-row tile of the residual
// stream per workgroup (pwwt.cn "parameter-golf 16MB 极限压缩实战 …", 架构:
// x = x + attn(norm(x)); x = x + proj(relu(fc(norm(x)))^2); pigsec.cn
// openai/parameter-golf README mirror, leaderboard: parallel attention / MLP
// residual lanes, x + attn(norm(x)) + mlp(norm(x))).
//
// The three GEMMs of a block tail are dense contractions over int8 codes
// widened exactly to binary16 (one binary16 scale per output row, pwwt.cn write-up,
// 后训练量化导出).  Run as three launches they move the fp32 residual through
// HBM twice and the hidden activations (3 d per row) once each way; here the
// tile's attention output, residual and the normed MLP input stay in LDS and
// registers, and the hidden activations exist only as 128-column chunks in
// LDS.  Per tile:
//
//   prologue  x rows -> the 128 x 512 fp32 accumulators (8 waves x 64
//             columns), pre-divided by the output-projection scale; the
//             attention output tile -> LDS (128 KB, binary16);
//   oproj     acc += o . code_o^T over K = 512 (A fragments from LDS, code
//             fragments from global memory straight into registers);
//   norm      x1 = acc * s_o; per-row sums of squares across the waves;
//             binary16(x1) (or, for parallel lanes, the layer input) replaces
//             the attention tile in LDS as the MLP input; the accumulators
//             become x1 / s_proj;
//   chunks    for every 128 hidden columns: h = act(a . code_fc^T * s_fc *
//             rinv)^2 (8 waves of 64 rows x 32 columns) -> LDS (32 KB,
//             binary16); acc += h . code_proj^T over those 128 columns;
//   epilogue  x2 = acc * s_proj, skip push / pop, x2, binary16(x2) and the
//             per-128-column sums of squares to global memory;
//   q/k/v     (when the next layer's q/k/v projection is fused in)
//             binary16(x2) into the A buffer instead of global memory, the
//             rows' RMS factors from the sums of squares, then the per-head
//             loop of the one-tile q/k/v kernel (qkv_phase.h) on the tile:
//             the next layer's q, k and v without x2's binary16 copy going
//             through HBM.
//
// Folding the residual into the accumulators as x / s (a zero scale counted
// as 1, its row's codes zeroed when the fragment-order copy is made) keeps
// the 128 accumulator registers per lane the only copy of the residual: the
// extra rounding is about one ulp of x per MFMA step, far below the
// binary16 rounding of the GEMM inputs.
//
// LDS (160 KB, one workgroup per CU): A tile 128 x 512 binary16 and one
// hidden chunk 128 x 128 binary16, rows placed by perm16 within 64-row slices
// and 16-byte chunks XOR-swizzled by the low bits of the row, so that every
// LDS pass of a fragment read or an epilogue store (16 rows, two adjacent
// chunks) touches 32 distinct 16-byte bank groups.
#include "common.h"
#include "mfma_util.h"
#include "qkv_phase.h"

namespace i6g {
namespace {

constexpr int TM = 128;                 // rows per tile
constexpr int NB = TM / 16;             // 16-row blocks per tile
constexpr int FB = TM / 32;             // 16-row blocks per wave of the up projection (2 x 4 waves)
constexpr int DM = 512;                 // model width
constexpr int HC = 128;                 // hidden columns per chunk
constexpr int NTH = 512;                // threads (8 waves)
constexpr int ABYTES = TM * DM * 2;     // 131072
constexpr int HBYTES = TM * HC * 2;     // 32768
constexpr int KSTEP_BYTES = 4 * 2 * 64 * 16;   // one 128-column tile, one K step of 64, fragment order

__device__ inline int phys_row(int r) { return (r & ~63) | perm16(r & 63); }
// byte offset of 16-byte chunk c (elements 8c .. 8c+7) of physical row p
// (A tile: 1 KB rows, slot c ^ 2(p & 15): the 32 lanes of one LDS pass (16
// rows, two adjacent chunks) land in 32 distinct 16-byte slots of the 512
// bytes the 128 banks cover; XOR with p & 15 alone would map chunks 2j and
// 2j + 1 onto the same 16 slots, a two-way conflict)
__device__ inline int a_off(int p, int c) { return p * (DM * 2) + ((c ^ (2 * (p & 15))) << 4); }
__device__ inline int h_off(int p, int c) { return p * (HC * 2) + ((c ^ (p & 15)) << 4); }

// a zero scale counts as 1 (its row's codes are zero)
__device__ inline float scale_or_one(float s) { return s == 0.0f ? 1.0f : s; }

// Eight binary16 scales (one 16-byte load) as floats.
__device__ inline void load_scales8(const uint16_t* p, float (&out)[8]) {
  const uint4 v = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    out[2 * e] = h2f((uint16_t)(w[e] & 0xffff));
    out[2 * e + 1] = h2f((uint16_t)(w[e] >> 16));
  }
}

typedef __attribute__((address_space(1))) void* gptr_t;
typedef __attribute__((address_space(3))) void* lptr_t;

#define MFMA(w_, x_, c_) __builtin_amdgcn_mfma_f32_16x16x32_f16(w_, x_, c_, 0, 0, 0)

// PAR: parallel residual lanes (the MLP reads the layer input); otherwise
// the MLP reads x + attention, normalised before it enters LDS.
// SPREAD: the residual rows enter the accumulators one 16-row block per
// output-projection K step (block i before step i, loaded a step ahead)
// instead of all in the prologue, so their loads overlap the MFMAs.  A
// row's rounding order then depends on its row block in the tile, which
// is the same for every batching when windows are padded to a multiple of
// 128 rows and the rows are not remapped; the host asks for SPREAD only
// then, and never in the final layer (whose rows are remapped when the
// batch is pruned, which depends on the batching).
// 160 KB of LDS: one workgroup (two waves per SIMD) per CU.
template <bool PAR, bool SPREAD>
__global__ __launch_bounds__(NTH) __attribute__((amdgpu_waves_per_eu(2, 2))) void tail_kernel(TailArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[ABYTES + HBYTES];
  char* const As = smem;
  char* const Hs = smem + ABYTES;
  float* const ss_part = reinterpret_cast<float*>(Hs);   // [8][TM] while Hs holds no hidden chunk
  // the output- and down-projection scales, staged in the (still unused)
  // hidden buffer for the norm phase: [2][512] after ss_part
  uint16_t* const sc_lds = reinterpret_cast<uint16_t*>(Hs + 4 * 8 * TM);

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  const int wm = w >> 2, wn = w & 3;             // MLP up-projection: 2 x 4 waves of TM/2 rows x 32 columns
  const int m0 = xcd_remap(blockIdx.x, gridDim.x) * TM;
  const int nk_proj = a.F / 64;                  // K steps of the down projection

  // memory row of tile row r (rows past M repeat row M - 1 and store
  // nothing); in scored-rows mode the caller keeps every prediction index
  // below 2^31, so the window arithmetic is 32-bit
  int m0v = m0, lrow_v = 16 * (lr >> 2) + (lr & 3);   // both made opaque before the epilogue (see there)
  auto grow = [&](int r) -> int {
    const int m = min(m0v + r, a.M - 1);
    if (!a.row_map) return m;
    const int p = (int)a.p0 + m;
    int k = (p < (int)a.e0) ? 0 : (p - a.L) / a.S + 1;
    k = min(k, (int)a.n_win - 1);
    return (k - (int)a.k0) * a.Lp + (p - k * a.S);
  };
  // the lane's tile row in accumulator row block i (physical row 16 i + lr),
  // and its four columns of block j in wave w's 64-column slice (C^T
  // accumulation, pair placement)
  auto arow = [&](int i) { return 64 * (i >> 2) + lrow_v + 4 * (i & 3); };
  auto colj = [&](int j) { return 64 * w + 32 * (j >> 1) + 8 * lg + 4 * (j & 1); };

  // code fragments of wave w: output projection / down projection (64
  // columns = tile w/2, slices 2(w&1), 2(w&1)+1: four 1 KB fragments in a
  // row) and up projection (32 columns: slice wn of a 128-column chunk);
  // wave-uniform bases, each lane adds its own 16 bytes.  Output- and
  // down-projection codes are loaded half a K step ahead of the MFMAs that
  // use them, up-projection codes two K steps ahead (in the registers the
  // down projection's four fragments use; the up projection needs two per
  // step).  sched_barrier fences keep the compiler from sinking those loads
  // below the MFMAs or pulling the widening of loads in flight up among them.
  const int8_t* const o_codes = a.o_frag + ((int64_t)(w >> 1) * 8 * 4 + 2 * (w & 1)) * 2 * 64 * 16;
  const int8_t* const p_codes = a.proj_frag + ((int64_t)(w >> 1) * nk_proj * 4 + 2 * (w & 1)) * 2 * 64 * 16;
  const int8_t* const f_codes = a.fc_frag + (int64_t)wn * 2 * 64 * 16;
  // the lane's 16-byte offset, recomputed at every code load (two VALU
  // ops) rather than held for the whole kernel: under full register
  // pressure a held copy is spilled, and its reload waits for every load in
  // flight
  auto loff16 = [&]() -> int {
    int l;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
    return l << 4;
  };
  uint4 cq0, cq1, cq2, cq3;
  auto load4 = [&](const int8_t* base) {
    const int loff = loff16();
    cq0 = *reinterpret_cast<const uint4*>(base + loff);
    cq1 = *reinterpret_cast<const uint4*>(base + loff + 1024);
    cq2 = *reinterpret_cast<const uint4*>(base + loff + 2048);
    cq3 = *reinterpret_cast<const uint4*>(base + loff + 3072);
  };
  // (offsets below 2^31: at most F / 64 K steps of 8 KB per 128-column tile)
  auto load_o = [&](int kt) { load4(o_codes + kt * KSTEP_BYTES); };
  auto load_p = [&](int kt) { load4(p_codes + kt * KSTEP_BYTES); };
  // up projection: chunk c (128 hidden columns), K step kt of 8; even steps
  // (odd = 0) go to cq0 / cq1, odd steps to cq2 / cq3 (the loop keeps two
  // steps in flight)
  auto load_f = [&](int c, int kt, int odd) {
    const int off = (c * 8 + kt) * KSTEP_BYTES + loff16();
    if (odd) {
      cq2 = *reinterpret_cast<const uint4*>(f_codes + off);
      cq3 = *reinterpret_cast<const uint4*>(f_codes + off + 1024);
    } else {
      cq0 = *reinterpret_cast<const uint4*>(f_codes + off);
      cq1 = *reinterpret_cast<const uint4*>(f_codes + off + 1024);
    }
  };
  // half h of a down-projection step's four fragments (cq0 / cq1 or cq2 / cq3)
  auto load_p_half = [&](int kt, int h) {
    const int8_t* base = p_codes + kt * KSTEP_BYTES + loff16();
    if (h) {
      cq2 = *reinterpret_cast<const uint4*>(base + 2048);
      cq3 = *reinterpret_cast<const uint4*>(base + 3072);
    } else {
      cq0 = *reinterpret_cast<const uint4*>(base);
      cq1 = *reinterpret_cast<const uint4*>(base + 1024);
    }
  };

  // A TM x 512 binary16 tile of rows m0.. into the A buffer by direct loads
  // into LDS: each wave instruction fills one physical row (1 KB), lane s
  // fetching the chunk that belongs in slot s (chunk s ^ 2(p & 15) of logical
  // row phys_row(p))
  auto load_tile = [&](const act* src) {
#pragma unroll
    for (int u = 0; u < TM / 8; ++u) {
      const int p = w + 8 * u;
      const act* g = src + (int64_t)grow(phys_row(p)) * DM + 8 * (lane ^ (2 * (p & 15)));
      __builtin_amdgcn_global_load_lds((gptr_t)g, (lptr_t)(As + p * (DM * 2)), 16, 0, 0);
    }
  };

  f32x4 acc[NB][4];
  bool out_of_range = false;   // a binary16 value of this lane would leave the range

  // ---- prologue: codes of the first K step, the attention tile into LDS,
  // the residual rows into the accumulators as x / s_o
  load_o(0);
  load_tile(a.o);
  if (tid < 64)
    *reinterpret_cast<uint4*>(sc_lds + 8 * tid) = *reinterpret_cast<const uint4*>(a.o_scale + 8 * tid);
  else if (tid < 128)
    *reinterpret_cast<uint4*>(sc_lds + DM + 8 * (tid - 64)) =
        *reinterpret_cast<const uint4*>(a.proj_scale + 8 * (tid - 64));
  // SPREAD: the 1 / s_o factors as fp32 in the hidden buffer (after the
  // partial sums and the staged scales), read where a row block is added
  float* const rs_lds = reinterpret_cast<float*>(Hs + 8192);
  float4 xres[4];
  auto load_res = [&](int i) {
    const float* xr = a.x_in + (int64_t)grow(arow(i)) * DM;
#pragma unroll
    for (int j = 0; j < 4; ++j) xres[j] = *reinterpret_cast<const float4*>(xr + colj(j));
  };
  auto add_res = [&](int i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float4 r4 = *reinterpret_cast<const float4*>(rs_lds + colj(j));
      acc[i][j] += f32x4{xres[j].x * r4.x, xres[j].y * r4.y, xres[j].z * r4.z, xres[j].w * r4.w};
    }
  };
  if constexpr (SPREAD) {
    if (tid < DM / 4) {
      const uint2 v = *reinterpret_cast<const uint2*>(a.o_scale + 4 * tid);
      *reinterpret_cast<float4*>(rs_lds + 4 * tid) =
          make_float4(__builtin_amdgcn_rcpf(scale_or_one(h2f((uint16_t)(v.x & 0xffff)))),
                      __builtin_amdgcn_rcpf(scale_or_one(h2f((uint16_t)(v.x >> 16)))),
                      __builtin_amdgcn_rcpf(scale_or_one(h2f((uint16_t)(v.y & 0xffff)))),
                      __builtin_amdgcn_rcpf(scale_or_one(h2f((uint16_t)(v.y >> 16)))));
    }
    load_res(0);
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  } else {
    float rs[2][8];
    load_scales8(a.o_scale + 64 * w + 8 * lg, rs[0]);
    load_scales8(a.o_scale + 64 * w + 32 + 8 * lg, rs[1]);
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) rs[h][e] = __builtin_amdgcn_rcpf(scale_or_one(rs[h][e]));
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const float* xr = a.x_in + (int64_t)grow(arow(i)) * DM;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float4 v = *reinterpret_cast<const float4*>(xr + colj(j));
        const float* r4 = &rs[j >> 1][4 * (j & 1)];
        acc[i][j] = f32x4{v.x * r4[0], v.y * r4[1], v.z * r4[2], v.w * r4[3]};
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0);   // the direct loads into LDS have landed
  __syncthreads();

  // ---- output projection, K = 512 in 8 steps of 64
  // One K step of the output or down projection: the first 32 codes of each
  // fragment chunk are widened and used, then the other 32, and only then
  // do the next step's loads take over the code registers (fewer live
  // registers than widening both halves first).
  auto wide_step = [&](const char* base, int rowbytes, int kc0, auto&& next_load) {
    asm volatile("" : "+s"(kc0));   // LDS addresses computed where used, not held
    {
      const actx8 wf[4] = {widen8(cq0.x, cq0.y), widen8(cq1.x, cq1.y), widen8(cq2.x, cq2.y), widen8(cq3.x, cq3.y)};
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const actx8 af = *reinterpret_cast<const actx8*>(base + (rowbytes == DM * 2 ? a_off(16 * i + lr, kc0 + lg)
                                                                                    : h_off(16 * i + lr, kc0 + lg)));
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = MFMA(wf[j], af, acc[i][j]);
      }
    }
    const actx8 wf[4] = {widen8(cq0.z, cq0.w), widen8(cq1.z, cq1.w), widen8(cq2.z, cq2.w), widen8(cq3.z, cq3.w)};
    next_load();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const actx8 af = *reinterpret_cast<const actx8*>(base + (rowbytes == DM * 2 ? a_off(16 * i + lr, kc0 + 4 + lg)
                                                                                  : h_off(16 * i + lr, kc0 + 4 + lg)));
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = MFMA(wf[j], af, acc[i][j]);
    }
  };
  if constexpr (SPREAD) {
    // step kt: block kt's residual rows (loaded during step kt - 1) are
    // added, block kt + 1's are loaded, then the step's MFMAs
#pragma unroll
    for (int kt = 0; kt < 7; ++kt) {
      add_res(kt);
      load_res(kt + 1);
      wide_step(As, DM * 2, 8 * kt, [&] { load_o(kt + 1); });
    }
    add_res(7);
  } else {
#pragma unroll 1
    for (int kt = 0; kt < 7; ++kt) wide_step(As, DM * 2, 8 * kt, [&] { load_o(kt + 1); });
  }
  wide_step(As, DM * 2, 56, [&] {
    load_f(0, 0, 0);
    load_f(0, 1, 1);
  });

  // ---- x1 = acc * s_o; the MLP input and (parallel lanes) its RMS factors
  float rinv[FB];
#pragma unroll
  for (int ii = 0; ii < FB; ++ii) rinv[ii] = 1.0f;
  {
    float so[2][8];
    load_scales8(sc_lds + 64 * w + 8 * lg, so[0]);
    load_scales8(sc_lds + 64 * w + 32 + 8 * lg, so[1]);
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[i][j][e] *= scale_or_one(so[j >> 1][4 * (j & 1) + e]);
    if constexpr (!PAR) {
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        float t = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e) t += acc[i][j][e] * acc[i][j][e];
        t += __shfl_xor(t, 16);
        t += __shfl_xor(t, 32);
        if (lg == 0) ss_part[w * TM + arow(i)] = t;
      }
    }
    __syncthreads();   // the attention tile is consumed; partial sums are in
    if constexpr (!PAR) {
      // N(x1) over the attention tile (|values| <= sqrt(512), well inside
      // binary16): the lane's two runs of 8 columns of each of its rows are
      // chunks 8w + 4h + lg of physical row 16i + lr
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        float t = 0.0f;
#pragma unroll
        for (int u = 0; u < 8; ++u) t += ss_part[u * TM + arow(i)];
        const float ri = 1.0f / sqrtf(t / (float)DM + a.eps);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const f32x4 u0 = acc[i][2 * h], u1 = acc[i][2 * h + 1];
          *reinterpret_cast<uint4*>(As + a_off(16 * i + lr, 8 * w + 4 * h + lg)) =
              make_uint4(pack2h(u0[0] * ri, u0[1] * ri), pack2h(u0[2] * ri, u0[3] * ri),
                         pack2h(u1[0] * ri, u1[1] * ri), pack2h(u1[2] * ri, u1[3] * ri));
        }
      }
    } else {
      // parallel lanes: the MLP reads the layer input (binary16 copy and sums
      // of squares written by the kernel that produced it)
      load_tile(a.xb_in);
      // the row's partial sums: one 16-byte load per row when there are
      // four (all rows' loads in flight at once), added in order
      if (a.nt_in == 4) {
        float4 pv[FB];
#pragma unroll
        for (int ii = 0; ii < FB; ++ii)
          pv[ii] = *reinterpret_cast<const float4*>(a.ss_in + (int64_t)grow(arow(FB * wm + ii)) * 4);
#pragma unroll
        for (int ii = 0; ii < FB; ++ii) {
          float t = 0.0f;
          t += pv[ii].x;
          t += pv[ii].y;
          t += pv[ii].z;
          t += pv[ii].w;
          rinv[ii] = 1.0f / sqrtf(t / (float)DM + a.eps);
        }
      } else {
#pragma unroll
        for (int ii = 0; ii < FB; ++ii) {
          const float* sp = a.ss_in + (int64_t)grow(arow(FB * wm + ii)) * a.nt_in;
          float t = 0.0f;
          for (int u = 0; u < a.nt_in; ++u) t += sp[u];
          rinv[ii] = 1.0f / sqrtf(t / (float)DM + a.eps);
        }
      }
    }
    // the accumulators now carry x1 / s_proj
    float sp[2][8];
    load_scales8(sc_lds + DM + 64 * w + 8 * lg, sp[0]);
    load_scales8(sc_lds + DM + 64 * w + 32 + 8 * lg, sp[1]);
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[i][j][e] *= __builtin_amdgcn_rcpf(scale_or_one(sp[j >> 1][4 * (j & 1) + e]));
    if constexpr (PAR) __builtin_amdgcn_s_waitcnt(0);   // the direct loads have landed
    __syncthreads();   // the MLP input tile is complete, the partial sums read
  }

  // ---- MLP, 128 hidden columns at a time
  const int nchunks = a.F / HC;
  for (int c = 0; c < nchunks; ++c) {
    // up projection: wave (wm, wn) makes rows TM/2 wm .. (blocks FB wm ..)
    // x hidden columns 32 wn .. of the chunk
    f32x4 hacc[FB][2];
#pragma unroll
    for (int ii = 0; ii < FB; ++ii) hacc[ii][0] = hacc[ii][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    // the scales of the lane's 8 hidden columns, kept packed until used
    const uint4 sfp = *reinterpret_cast<const uint4*>(a.fc_scale + HC * c + 32 * wn + 8 * lg);
    // two K steps per trip: step kt's codes sit in cq0 / cq1 and step
    // kt + 1's in cq2 / cq3, each loaded two steps before it is used; after
    // the last step the down projection's first step follows, half by half
    auto fc_step = [&](uint4 ca, uint4 cb, int k8, auto&& next_load) {
      // an opaque copy of the K offset keeps the compiler from computing
      // every step's LDS addresses up front and holding them (it spills them)
      asm volatile("" : "+s"(k8));
      const actx8 w0 = widen8(ca.x, ca.y), w1 = widen8(cb.x, cb.y);
      const actx8 w2 = widen8(ca.z, ca.w), w3 = widen8(cb.z, cb.w);
      next_load();
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ii = 0; ii < FB; ++ii) {
        const actx8 af = *reinterpret_cast<const actx8*>(As + a_off(16 * (FB * wm + ii) + lr, k8 + lg));
        hacc[ii][0] = MFMA(w0, af, hacc[ii][0]);
        hacc[ii][1] = MFMA(w1, af, hacc[ii][1]);
      }
#pragma unroll
      for (int ii = 0; ii < FB; ++ii) {
        const actx8 af = *reinterpret_cast<const actx8*>(As + a_off(16 * (FB * wm + ii) + lr, k8 + 4 + lg));
        hacc[ii][0] = MFMA(w2, af, hacc[ii][0]);
        hacc[ii][1] = MFMA(w3, af, hacc[ii][1]);
      }
      // nothing that waits on the loads above is pulled in among the MFMAs
      __builtin_amdgcn_sched_barrier(0);
    };
#pragma unroll 1
    for (int kt = 0; kt < 6; kt += 2) {
      fc_step(cq0, cq1, 8 * kt, [&] { load_f(c, kt + 2, 0); });
      fc_step(cq2, cq3, 8 * kt + 8, [&] { load_f(c, kt + 3, 1); });
    }
    fc_step(cq0, cq1, 48, [&] { load_p_half(2 * c, 0); });
    fc_step(cq2, cq3, 56, [&] { load_p_half(2 * c, 1); });
    // act(acc * s_fc * rinv)^2 in binary16: the lane's 8 hidden columns
    // 32 wn + 8 lg .. are chunk 4 wn + lg of physical row 16 i + lr
    float sf[8];
    {
      const uint32_t sw[4] = {sfp.x, sfp.y, sfp.z, sfp.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sf[2 * e] = h2f((uint16_t)(sw[e] & 0xffff));
        sf[2 * e + 1] = h2f((uint16_t)(sw[e] >> 16));
      }
    }
    uint4 hv[FB];
#pragma unroll
    for (int ii = 0; ii < FB; ++ii) {
      float v[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[e] = lrelu(hacc[ii][0][e] * sf[e] * rinv[ii], a.leaky);
        v[4 + e] = lrelu(hacc[ii][1][e] * sf[4 + e] * rinv[ii], a.leaky);
      }
      hv[ii] = make_uint4(pack2h(v[0] * v[0], v[1] * v[1]), pack2h(v[2] * v[2], v[3] * v[3]),
                          pack2h(v[4] * v[4], v[5] * v[5]), pack2h(v[6] * v[6], v[7] * v[7]));
    }
    __syncthreads();   // the previous chunk's down projection has read Hs
    {
      // a square that rounded past 65504 became Inf in binary16 (the
      // largest packed value tells, no float copies kept alive)
      typedef _Float16 h2 __attribute__((ext_vector_type(2)));
      h2 hm = __builtin_bit_cast(h2, hv[0].x);
#pragma unroll
      for (int ii = 0; ii < FB; ++ii) {
        hm = __builtin_elementwise_max(hm, __builtin_bit_cast(h2, hv[ii].x));
        hm = __builtin_elementwise_max(hm, __builtin_bit_cast(h2, hv[ii].y));
        hm = __builtin_elementwise_max(hm, __builtin_bit_cast(h2, hv[ii].z));
        hm = __builtin_elementwise_max(hm, __builtin_bit_cast(h2, hv[ii].w));
      }
      out_of_range |= !((float)hm[0] <= 65504.0f && (float)hm[1] <= 65504.0f);
    }
#pragma unroll
    for (int ii = 0; ii < FB; ++ii)
      *reinterpret_cast<uint4*>(Hs + h_off(16 * (FB * wm + ii) + lr, 4 * wn + lg)) = hv[ii];
    __syncthreads();
    // down projection of the chunk: acc += h . code_proj^T, K = 128
    wide_step(Hs, HC * 2, 0, [&] { load_p(2 * c + 1); });
    wide_step(Hs, HC * 2, 8, [&] {
      if (c + 1 < nchunks) {
        load_f(c + 1, 0, 0);
        load_f(c + 1, 1, 1);
      }
    });
  }

  // ---- epilogue: x2 = acc * s_proj, skip push / pop, stores
  {
    float sp[2][8], pw[2][8];
    load_scales8(a.proj_scale + 64 * w + 8 * lg, sp[0]);
    load_scales8(a.proj_scale + 64 * w + 32 + 8 * lg, sp[1]);
    const bool push = a.push_dst != nullptr;
    const bool pop = a.pop_src != nullptr;
    const bool pop_self = pop && a.pop_src == a.push_dst;
    if (pop) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const float4 p0 = *reinterpret_cast<const float4*>(a.pop_w + 64 * w + 32 * h + 8 * lg);
        const float4 p1 = *reinterpret_cast<const float4*>(a.pop_w + 64 * w + 32 * h + 8 * lg + 4);
        pw[h][0] = p0.x; pw[h][1] = p0.y; pw[h][2] = p0.z; pw[h][3] = p0.w;
        pw[h][4] = p1.x; pw[h][5] = p1.y; pw[h][6] = p1.z; pw[h][7] = p1.w;
      }
    }
    __syncthreads();   // the last chunk's down projection has read Hs (partial sums go there)
    // the fused q/k/v phase's first codes, loaded before this epilogue's
    // stores (a load issued after a store waits for it on the single
    // vector-memory counter)
    const bool qkv = a.qkv.frag != nullptr;
    if (qkv && w < a.qkv.n_heads + 2 * a.qkv.n_kv) qkvp::load4(a.qkv.frag, w, 0, cq0, cq1, cq2, cq3);
    // the row addresses are recomputed here rather than kept from the
    // prologue: an opaque copy of the tile base stops the compiler from
    // holding them in registers through the MLP (it would spill them)
    // (the lane indices too: the q/k/v phase's LDS addresses depend on
    // nothing else and would be computed before the MLP and held)
    int lr_e = lr, lg_e = lg;
    asm volatile("" : "+s"(m0v), "+v"(lrow_v), "+v"(lr_e), "+v"(lg_e));
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const bool ok = m0v + arow(i) < a.M;
      const int64_t off = (int64_t)grow(arow(i)) * DM;
      float t = 0.0f;
      // the lane's two runs of 8 columns, one at a time
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        f32x4 xv[2];
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
          for (int e = 0; e < 4; ++e) xv[jj][e] = acc[i][2 * h + jj][e] * scale_or_one(sp[h][4 * jj + e]);
        if (push && ok) {
#pragma unroll
          for (int jj = 0; jj < 2; ++jj)
            *reinterpret_cast<float4*>(a.push_dst + off + colj(2 * h + jj)) =
                make_float4(xv[jj][0], xv[jj][1], xv[jj][2], xv[jj][3]);
        }
        if (pop) {
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) {
            f32x4 pv = xv[jj];
            if (!pop_self) {
              const float4 q = *reinterpret_cast<const float4*>(a.pop_src + off + colj(2 * h + jj));
              pv = f32x4{q.x, q.y, q.z, q.w};
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) xv[jj][e] += pw[h][4 * jj + e] * pv[e];
          }
        }
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
          for (int e = 0; e < 4; ++e) t += xv[jj][e] * xv[jj][e];
        const uint4 xbv = make_uint4(pack2h(xv[0][0], xv[0][1]), pack2h(xv[0][2], xv[0][3]),
                                     pack2h(xv[1][0], xv[1][1]), pack2h(xv[1][2], xv[1][3]));
        // the q/k/v phase's A tile: the same binary16 values, in the layout
        // of the MLP input (chunks 8w + 4h + lg of physical row 16i + lr)
        if (qkv) *reinterpret_cast<uint4*>(As + a_off(16 * i + lr_e, 8 * w + 4 * h + lg_e)) = xbv;
        if (ok && a.x) {
#pragma unroll
          for (int jj = 0; jj < 2; ++jj)
            *reinterpret_cast<float4*>(a.x + off + colj(2 * h + jj)) = make_float4(xv[jj][0], xv[jj][1], xv[jj][2], xv[jj][3]);
        }
        if (ok) {
          if (a.xb) *reinterpret_cast<uint4*>(a.xb + off + colj(2 * h)) = xbv;
        }
      }
      t += __shfl_xor(t, 16);
      t += __shfl_xor(t, 32);
      if (lg == 0) ss_part[w * TM + arow(i)] = t;
      out_of_range |= (a.xb || qkv) && ok && t >= kRangeSq;
    }
    if (__any(out_of_range) && lane == 0) atomicOr(a.flags, kFlagRange);
    if (a.ss_out || qkv) __syncthreads();   // partial sums (and the binary16 rows) complete
    if (a.ss_out) {
      // TM rows x 4 column tiles of 128: threads 0 .. 4 TM - 1
      const int r = tid & (TM - 1), tn = tid / TM;
      if (tn < DM / 128 && m0v + r < a.M)
        a.ss_out[(int64_t)grow(r) * (DM / 128) + tn] = ss_part[(2 * tn) * TM + r] + ss_part[(2 * tn + 1) * TM + r];
    }
    if (qkv) {
      // the rows' RMS factors as the q/k/v kernel computes them from the
      // four per-128-column sums this kernel would otherwise write (added in
      // order, t / 512 + eps without a fused multiply-add), and the
      // projection's scales as floats, both after the partial sums in Hs
      float* const rinv_s = reinterpret_cast<float*>(Hs + 4 * 8 * TM);
      float* const sc_s = rinv_s + TM;
      const int nall = a.qkv.n_heads + 2 * a.qkv.n_kv;
      if (tid < TM) {
        float ri = 0.0f;
        if (m0v + tid < a.M) {
#pragma clang fp contract(off)
          float t = 0.0f;
#pragma unroll
          for (int tn = 0; tn < DM / 128; ++tn) t = t + (ss_part[(2 * tn) * TM + tid] + ss_part[(2 * tn + 1) * TM + tid]);
          ri = 1.0f / sqrtf(t / (float)DM + a.eps);
        }
        rinv_s[tid] = ri;
      }
      if (tid < nall * 8) {
        const uint4 v = *reinterpret_cast<const uint4*>(a.qkv.scale + 8 * tid);
        const uint32_t sw[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sc_s[8 * tid + 2 * e] = h2f((uint16_t)(sw[e] & 0xffff));
          sc_s[8 * tid + 2 * e + 1] = h2f((uint16_t)(sw[e] >> 16));
        }
      }
      __syncthreads();
      qkvp::heads(a.qkv, a.M, a.Lp, As, rinv_s, sc_s, m0v, w, cq0, cq1, cq2, cq3);
    }
  }
}

#undef MFMA

}  // namespace

hipError_t launch_tail(const TailArgs& a, hipStream_t s) {
  if (a.M <= 0) return hipSuccess;
  if (a.F <= 0 || a.F % HC != 0 || !a.flags || (a.parallel && (!a.ss_in || !a.xb_in || a.nt_in < 1)))
    return hipErrorInvalidValue;
  // the result goes to x, or (x null) only to the skip slot of a push with no pop
  if (!a.x_in || (!a.x && (!a.push_dst || a.pop_src))) return hipErrorInvalidValue;
  if (a.qkv.frag &&
      (a.row_map || a.M % 64 != 0 || a.Lp < TM || a.Lp % 64 != 0 || !a.qkv.scale || !a.qkv.q || !a.qkv.k ||
       !a.qkv.vt || !a.qkv.rope || !qkv_tile_supported(DM, qkvp::HD, a.qkv.n_heads, a.qkv.n_kv, a.qkv.rope_dims, 0)))
    return hipErrorInvalidValue;
  const int tiles = (a.M + TM - 1) / TM;
  if (a.spread_residual && a.row_map) return hipErrorInvalidValue;
  if (a.parallel) {
    if (a.spread_residual) hipLaunchKernelGGL((tail_kernel<true, true>), dim3(tiles), dim3(NTH), 0, s, a);
    else hipLaunchKernelGGL((tail_kernel<true, false>), dim3(tiles), dim3(NTH), 0, s, a);
  } else {
    if (a.spread_residual) hipLaunchKernelGGL((tail_kernel<false, true>), dim3(tiles), dim3(NTH), 0, s, a);
    else hipLaunchKernelGGL((tail_kernel<false, false>), dim3(tiles), dim3(NTH), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace i6g
