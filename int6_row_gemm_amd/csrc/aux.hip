// Embedding gather, LoRA down-projection, tied head + cross-entropy, the
// bits-per-byte reduction, and the constant tables built at load time.
#include "common.h"
#include <algorithm>

namespace i6g {
namespace {

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// ---------------------------------------------------------------------------
// Embedding: x0 = E[u] (+ bigram row), pwwt.cn "parameter-golf 16MB 极限压缩
// 实战 …" 架构 (tied embedding) and the kwkr.cn PR #363 write-up (BigramHash:
// adjacent-token hash into a table, projected to the model width; the
// table is pre-multiplied by the projection at load time).  Row m of the
// batch is position j = m % Lp of window k0 + m / Lp; positions past the end
// of the window's inputs read token 0 and are never scored.  One wave per row;
// it also writes binary16(x) and the row's sum of squares for the first normed
// GEMM.
__global__ __launch_bounds__(256) void embed_kernel(EmbedArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t m = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (m >= (int64_t)a.W * a.Lp) return;
  const int64_t k = a.k0 + m / a.Lp;
  const int64_t j = m % a.Lp;
  const int64_t s = k * a.S;
  const int64_t e = min(s + (int64_t)a.L, a.P);
  const bool valid = s + j < e;
  int tok = valid ? a.tokens[s + j] : 0;
  if (tok < 0 || tok >= a.vocab) {
    if (lane == 0) atomicOr(a.flags, 2);
    tok = 0;
  }
  const float* brow = nullptr;
  if (a.bigram && valid && j >= 1) {
    int prev = a.tokens[s + j - 1];
    if (prev < 0 || prev >= a.vocab) prev = 0;
    int64_t hsh = ((int64_t)prev * 1000003 + (int64_t)tok) % a.buckets;
    brow = a.bigram + hsh * a.d;
  }
  float sq = 0.f;
  for (int c = lane; c < a.d; c += 64) {
    float v = a.embed_f32 ? reinterpret_cast<const float*>(a.embed)[(int64_t)tok * a.d + c]
                          : (float)reinterpret_cast<const _Float16*>(a.embed)[(int64_t)tok * a.d + c];
    if (brow) v += brow[c];
    a.x[m * a.d + c] = v;
    a.xb[m * a.d + c] = (act)v;
    sq += v * v;
  }
  sq = wave_sum(sq);
  if (lane < a.nt) a.ss[m * a.nt + lane] = (lane == 0) ? sq : 0.f;
}

// ---------------------------------------------------------------------------
// DepthLoRA down-projection (kwkr.cn PR #363 write-up, per-depth low-rank
// adapter on Q and V): u = N(x) A^T for the q and v adapters.
__global__ __launch_bounds__(256) void lora_down_kernel(LoraArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t m = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (m >= a.M) return;
  const float* xr = a.x + m * a.d;
  const int nt = 2 * a.r;
  float rinv = 0.f;
  // The row is read once per group of eight adapter rows (once for rank <= 4)
  // in blocks of 1024 columns, each lane's eight 8-byte loads of a block
  // issued together (d is a multiple of 128); the eight dot products and the
  // sum of squares are reduced over the wave together.
  for (int t0 = 0; t0 < nt; t0 += 8) {
    float acc[8] = {};
    float sq = 0.f;
    for (int c0 = 0; c0 < a.d; c0 += 1024) {
      float2 xv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        xv[i] = make_float2(0.f, 0.f);
        const int c = c0 + 128 * i + 2 * lane;
        if (c < a.d) xv[i] = *reinterpret_cast<const float2*>(xr + c);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) sq += xv[i].x * xv[i].x + xv[i].y * xv[i].y;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int t = t0 + j;
        if (t < nt) {
          const float* ar = t < a.r ? a.aq + (int64_t)t * a.d : a.av + (int64_t)(t - a.r) * a.d;
          float2 av[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            av[i] = make_float2(0.f, 0.f);
            const int c = c0 + 128 * i + 2 * lane;
            if (c < a.d) av[i] = *reinterpret_cast<const float2*>(ar + c);
          }
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[j] += xv[i].x * av[i].x + xv[i].y * av[i].y;
        }
      }
    }
    if (t0 == 0) rinv = 1.0f / sqrtf(wave_sum(sq) / (float)a.d + a.eps);
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = wave_sum(acc[j]);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (lane == j && t0 + j < nt) a.u[m * nt + t0 + j] = acc[j] * rinv;
  }
}

// ---------------------------------------------------------------------------
// Tied head + log-softmax cross-entropy on the scored rows of a batch
// (pwwt.cn "parameter-golf 16MB 极限压缩实战 …": tied input/output embedding;
// 滑动窗口评估: only the scored positions of a window reach the loss).
// A workgroup takes 16 scored predictions.  Their rows are normalised (final
// RMSNorm) into fp16 in LDS and held by every wave as the B operand; the NW
// waves split the vocabulary and stream the binary16 embedding as the A
// operand of v_mfma_f32_16x16x32_f16, so logits^T arrive with one prediction
// per lane column: each lane keeps an online log-sum-exp and the target
// logit, merged over lane groups and then over the waves through LDS.
// Logits never reach memory.  The normalised rows carry a factor log2(e), so
// the logits come out in base 2 and each probability is one exp2; the nats
// are ln 2 times the base-2 result.  Work per batch is small (about 1,500
// predictions): eight waves per workgroup (two per SIMD) halve each wave's
// chain of embedding blocks, and a wave loads all its rows for the norm at
// once.
constexpr int HEAD_ROWS = 16;

template <int NKS, int NW>   // d / 32, waves per workgroup
__global__ __launch_bounds__(64 * NW) void head_kernel(HeadArgs a) {
  __shared__ __attribute__((aligned(16))) _Float16 zs[HEAD_ROWS * (640 + 8)];   // d <= 640
  __shared__ float part_m[NW][HEAD_ROWS], part_s[NW][HEAD_ROWS], part_t[NW][HEAD_ROWS];
  __shared__ int part_g[NW][HEAD_ROWS];
  constexpr int RPW = HEAD_ROWS / NW;    // rows normalised per wave
  constexpr int CPL = NKS / 2;           // row elements per lane (d / 64)
  constexpr float kLog2e = 1.44269504088896340736f;
  constexpr float kLn2 = 0.69314718055994530942f;
  const int tid = threadIdx.x & (64 * NW - 1), lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int zld = a.d + 8;
  const int64_t pb = a.p0 + (int64_t)blockIdx.x * HEAD_ROWS;

  // final norm: the wave's rows are loaded together, then reduced
  {
    float xv[RPW][CPL];
    bool ok[RPW];
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      const int64_t p = pb + wave * RPW + r;
      ok[r] = p < a.p1;
      int64_t row = 0;
      if (ok[r]) {
        if (a.compact) {
          row = p - a.p0;
        } else {
          int64_t k = (p < a.e0) ? 0 : (p - a.L) / a.S + 1;
          if (k > a.K - 1) k = a.K - 1;
          row = (k - a.k0) * a.Lp + (p - k * a.S);
        }
      }
      const float* xr = a.x + row * a.d;
#pragma unroll
      for (int u = 0; u < CPL; ++u) xv[r][u] = ok[r] ? xr[lane + 64 * u] : 0.0f;
    }
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      _Float16* zrow = zs + (wave * RPW + r) * zld;
      float sq = 0.f;
#pragma unroll
      for (int u = 0; u < CPL; ++u) sq += xv[r][u] * xv[r][u];
      sq = wave_sum(sq);
      // the evaluation temperature divides every logit, so it scales the
      // normed row once instead, as does the base-2 factor
      const float rinv = 1.0f / sqrtf(sq / (float)a.d + a.eps) * a.inv_temp * kLog2e;
#pragma unroll
      for (int u = 0; u < CPL; ++u) zrow[lane + 64 * u] = (_Float16)(ok[r] ? xv[r][u] * rinv : 0.0f);
    }
  }
  __syncthreads();

  const int64_t p_mine = pb + lr;
  const bool have = p_mine < a.p1;
  int tgt = have ? a.tokens[p_mine + 1] : -1;
  if (have && (tgt < 0 || tgt >= a.vocab)) {
    if (lg == 0 && wave == 0) atomicOr(a.flags, 2);
    tgt = -1;
  }

  f16x8 zf[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) zf[ks] = *reinterpret_cast<const f16x8*>(zs + lr * zld + ks * 32 + 8 * lg);

  const int vper = a.vocab / NW;
  const int vlo = wave * vper, vhi = vlo + vper;
  float mrun = -1e30f, srun = 0.f, tl = 0.f;
  int got = 0;
  // Embedding fragments of the next vocabulary block are loaded while the
  // current block is multiplied (two register sets, 16 vocab rows each).
  f16x8 ea[NKS], eb[NKS];
  auto load_e = [&](f16x8 (&dst)[NKS], int vb) {
    const _Float16* er = a.E + (int64_t)(vb + lr) * a.d + 8 * lg;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) dst[ks] = *reinterpret_cast<const f16x8*>(er + ks * 32);
  };
  auto block = [&](const f16x8 (&ef)[NKS], int vb) {
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ef[ks], zf[ks], acc, 0, 0, 0);
    const int vbase = vb + 4 * lg;
    const float mt = fmaxf(fmaxf(acc[0], acc[1]), fmaxf(acc[2], acc[3]));
    const float mn = fmaxf(mrun, mt);
    srun = srun * __builtin_amdgcn_exp2f(mrun - mn) + __builtin_amdgcn_exp2f(acc[0] - mn) +
           __builtin_amdgcn_exp2f(acc[1] - mn) + __builtin_amdgcn_exp2f(acc[2] - mn) +
           __builtin_amdgcn_exp2f(acc[3] - mn);
    mrun = mn;
    if (tgt >= vbase && tgt < vbase + 4) {
      const int i = tgt - vbase;
      tl = (i == 0) ? acc[0] : (i == 1) ? acc[1] : (i == 2) ? acc[2] : acc[3];
      got = 1;
    }
  };
  load_e(ea, vlo);
  for (int vb = vlo; vb < vhi; vb += 32) {
    if (vb + 16 < vhi) load_e(eb, vb + 16);
    block(ea, vb);
    if (vb + 16 < vhi) {
      if (vb + 32 < vhi) load_e(ea, vb + 32);
      block(eb, vb + 16);
    }
  }
#pragma unroll
  for (int off = 16; off < 64; off <<= 1) {
    const float mo = __shfl_xor(mrun, off);
    const float so = __shfl_xor(srun, off);
    const float to = __shfl_xor(tl, off);
    const int go = __shfl_xor(got, off);
    const float mn = fmaxf(mrun, mo);
    srun = srun * __builtin_amdgcn_exp2f(mrun - mn) + so * __builtin_amdgcn_exp2f(mo - mn);
    mrun = mn;
    if (go) { tl = to; got = 1; }
  }
  if (lg == 0) {
    part_m[wave][lr] = mrun;
    part_s[wave][lr] = srun;
    part_t[wave][lr] = tl;
    part_g[wave][lr] = got;
  }
  __syncthreads();
  if (wave == 0 && lg == 0 && have) {
    float m = part_m[0][lr], s = part_s[0][lr], t = got ? tl : 0.f;
    for (int w2 = 1; w2 < NW; ++w2) {
      const float mo = part_m[w2][lr];
      const float mn = fmaxf(m, mo);
      s = s * __builtin_amdgcn_exp2f(m - mn) + part_s[w2][lr] * __builtin_amdgcn_exp2f(mo - mn);
      m = mn;
      if (part_g[w2][lr]) t = part_t[w2][lr];
    }
    a.nats[p_mine] = (m + log2f(s) - t) * kLn2;
  }
}

// ---------------------------------------------------------------------------
// Bits per byte (pigsec.cn openai/parameter-golf README mirror: the score is
// tokenizer-agnostic bits per byte): sum of nats over the sum of the byte
// counts of the predicted tokens, times 1/ln 2.  Two deterministic passes
// (fixed partition, fixed tree) in fp64 / int64.
__global__ __launch_bounds__(256) void reduce_part_kernel(ReduceArgs a) {
  __shared__ double sn[256];
  __shared__ long long sb[256];
  const int tid = threadIdx.x;
  const int64_t per = (a.P + a.n_parts - 1) / a.n_parts;
  const int64_t lo = (int64_t)blockIdx.x * per;
  const int64_t hi = min(lo + per, a.P);
  double n = 0.0;
  long long b = 0;
  int bad = 0;
  for (int64_t p = lo + tid; p < hi; p += 256) {
    n += (double)a.nats[p];
    int by = a.bytes[p + 1];
    if (by < 0) { bad = 1; by = 0; }
    b += by;
  }
  if (bad) atomicOr(a.flags, 4);
  sn[tid] = n;
  sb[tid] = b;
  __syncthreads();
  for (int st = 128; st > 0; st >>= 1) {
    if (tid < st) { sn[tid] += sn[tid + st]; sb[tid] += sb[tid + st]; }
    __syncthreads();
  }
  if (tid == 0) { a.part_nats[blockIdx.x] = sn[0]; a.part_bytes[blockIdx.x] = sb[0]; }
}

__global__ void reduce_final_kernel(ReduceArgs a) {
  if (threadIdx.x != 0) return;
  double n = 0.0;
  long long b = 0;
  for (int i = 0; i < a.n_parts; ++i) { n += a.part_nats[i]; b += a.part_bytes[i]; }
  a.totals[0] = n;
  a.totals[1] = (double)b;
  a.totals[2] = (double)a.P;
  a.totals[3] = (b > 0) ? n / (0.69314718055994530942 * (double)b) : __builtin_nan("");
  if (b <= 0) atomicOr(a.flags, 4);
}

// ---------------------------------------------------------------------------
// RoPE table: (cos, sin) of p * base^(-2i/hd), evaluated in fp64.
// (cos, sin) of rotation pair i at position p, [Lmax, hd/2]: pairs
// i < R/2 turn by p * base^(-2i/R) (R = rotated dims per head); the other
// pairs hold the identity (1, 0) (partial RoPE, [363] Partial RoPE 16/64).
__global__ void rope_table_kernel(float2* tab, int Lmax, int hd, int R, double base) {
  const int half = hd / 2;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)Lmax * half) return;
  const int p = (int)(idx / half), i = (int)(idx % half);
  if (i >= R / 2) {
    tab[idx] = make_float2(1.0f, 0.0f);
    return;
  }
  const double theta = pow(base, -2.0 * (double)i / (double)R);
  const double ang = (double)p * theta;
  tab[idx] = make_float2((float)cos(ang), (float)sin(ang));
}

// Bigram table pre-multiplied by its projection: out[b, n] = sum_t table[b, t] * proj[n, t].
__global__ void bigram_table_kernel(const uint16_t* table, const uint16_t* proj, float* out,
                                    int buckets, int dim, int d) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)buckets * d) return;
  const int b = (int)(idx / d), n = (int)(idx % d);
  double acc = 0.0;
  for (int t = 0; t < dim; ++t)
    acc += (double)(float)__builtin_bit_cast(_Float16, table[(int64_t)b * dim + t]) *
           (double)(float)__builtin_bit_cast(_Float16, proj[(int64_t)n * dim + t]);
  out[idx] = (float)acc;
}

__global__ void f16_to_f32_kernel(const uint16_t* in, float* out, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) out[i] = (float)__builtin_bit_cast(_Float16, in[i]);
}

__global__ void f32_to_f16_kernel(const float* in, _Float16* out, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) out[i] = (_Float16)in[i];
}

// OR I6G_FLAG_NONFINITE into *flags when any of n values is NaN or Inf
// (binary16 bit patterns or fp32): a loaded model must not hold non-finite
// scales or passthrough tensors.
__global__ void nonfinite_f16_kernel(const uint16_t* p, int64_t n, int32_t* flags) {
  int bad = 0;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    bad |= (p[i] & 0x7c00u) == 0x7c00u;
  if (__any(bad) && (threadIdx.x & 63) == 0) atomicOr(flags, 1);
}

__global__ void nonfinite_f32_kernel(const float* p, int64_t n, int32_t* flags) {
  int bad = 0;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    bad |= (__builtin_bit_cast(uint32_t, p[i]) & 0x7f800000u) == 0x7f800000u;
  if (__any(bad) && (threadIdx.x & 63) == 0) atomicOr(flags, 1);
}

inline unsigned nblk(int64_t n, int b) { return (unsigned)((n + b - 1) / b); }

}  // namespace

hipError_t launch_embed(const EmbedArgs& a, hipStream_t s) {
  int64_t rows = (int64_t)a.W * a.Lp;
  hipLaunchKernelGGL(embed_kernel, dim3(nblk(rows, 4)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_lora_down(const LoraArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(lora_down_kernel, dim3(nblk(a.M, 4)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_head(const HeadArgs& a, hipStream_t s) {
  if (a.d % 32 != 0 || a.d > 640 || a.vocab % 64 != 0) return hipErrorInvalidValue;
  int64_t rows = a.p1 - a.p0;
  if (rows <= 0) return hipSuccess;
  const dim3 grid(nblk(rows, HEAD_ROWS));
  // eight waves when each gets whole 16-row vocabulary blocks and the
  // registers allow two waves per SIMD (d <= 512), else four
  const bool w8 = a.vocab % 128 == 0 && a.d <= 512;
#define HEAD_LAUNCH(NKS)                                                                          \
  if (w8) hipLaunchKernelGGL((head_kernel<NKS, 8>), grid, dim3(512), 0, s, a);                     \
  else hipLaunchKernelGGL((head_kernel<NKS, 4>), grid, dim3(256), 0, s, a)
  switch (a.d) {
    case 128: HEAD_LAUNCH(4); break;
    case 256: HEAD_LAUNCH(8); break;
    case 384: HEAD_LAUNCH(12); break;
    case 512: HEAD_LAUNCH(16); break;
    case 640: HEAD_LAUNCH(20); break;
    default: return hipErrorInvalidValue;
  }
#undef HEAD_LAUNCH
  return hipGetLastError();
}

hipError_t launch_reduce(const ReduceArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(reduce_part_kernel, dim3(a.n_parts), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(reduce_final_kernel, dim3(1), dim3(64), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_rope_table(float2* tab, int32_t Lmax, int32_t hd, int32_t rope_dims, double base,
                             hipStream_t s) {
  int64_t n = (int64_t)Lmax * (hd / 2);
  hipLaunchKernelGGL(rope_table_kernel, dim3(nblk(n, 256)), dim3(256), 0, s, tab, Lmax, hd, rope_dims, base);
  return hipGetLastError();
}

hipError_t launch_bigram_table(const uint16_t* table, const uint16_t* proj, float* out,
                               int32_t buckets, int32_t dim, int32_t d, hipStream_t s) {
  int64_t n = (int64_t)buckets * d;
  hipLaunchKernelGGL(bigram_table_kernel, dim3(nblk(n, 256)), dim3(256), 0, s, table, proj, out,
                     buckets, dim, d);
  return hipGetLastError();
}

hipError_t launch_f16_to_f32(const uint16_t* in, float* out, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(f16_to_f32_kernel, dim3(nblk(n, 256)), dim3(256), 0, s, in, out, n);
  return hipGetLastError();
}

hipError_t launch_f32_to_f16(const float* in, _Float16* out, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(f32_to_f16_kernel, dim3(nblk(n, 256)), dim3(256), 0, s, in, out, n);
  return hipGetLastError();
}

hipError_t launch_check_finite(const void* p, int64_t n, bool f32, int32_t* flags, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const unsigned blocks = (unsigned)std::min<int64_t>(nblk(n, 256), 1024);
  if (f32) hipLaunchKernelGGL(nonfinite_f32_kernel, dim3(blocks), dim3(256), 0, s, (const float*)p, n, flags);
  else hipLaunchKernelGGL(nonfinite_f16_kernel, dim3(blocks), dim3(256), 0, s, (const uint16_t*)p, n, flags);
  return hipGetLastError();
}

}  // namespace i6g
