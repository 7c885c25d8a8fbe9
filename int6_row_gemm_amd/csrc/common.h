// Internal declarations shared by the HIP kernels and the C-ABI host code.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

namespace i6g {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// Device flag bit set by the packer for a byte that is not a code of the
// format being packed; equals I6G_FLAG_CODE of the C ABI.
constexpr int32_t kFlagCode = 8;

// ---------------------------------------------------------------------------
// Row quantiser
struct QuantArgs {
  const float* w;
  int8_t* codes;
  uint16_t* scales;
  int32_t* flags;
  int64_t rows;
  int32_t cols;
  int32_t bits;
  int32_t topk;   // number of largest |w| kept per row (cols - lo)
  float frac;     // fp32 interpolation weight f
  void* fq;       // fake quantisation: [rows, cols] output, fp32 or bf16
  int32_t fq_bf16;
};
hipError_t launch_quantize(const QuantArgs& a, hipStream_t s);
// code * fp32 scale per element (fake quantisation) into a.fq
hipError_t launch_fake_quantize(const QuantArgs& a, hipStream_t s);

// Noisy-QAT weights: out = w + (U - 0.5) * max(amax, 1e-12) / levels per
// row, U from Philox4x32-10 (key = seed, counter = element index / 4).
struct NoisyArgs {
  const float* w;
  void* out;
  int32_t* flags;
  int64_t rows;
  int32_t cols;
  int32_t out_bf16;
  float levels;
  uint32_t key0, key1;
};
hipError_t launch_noisy_weights(const NoisyArgs& a, hipStream_t s);

// Several matrices in one launch: row r of the concatenated rows belongs to
// the last job j with row0[j] <= r.  The table travels in the kernel
// arguments (at most 4 KiB), so no device buffer is needed.
constexpr int kQuantJobs = 80;   // the 66 matrices of an 11-layer model fit one launch
struct QuantJob {
  const float* w;
  int8_t* codes;
  uint16_t* scales;
  int32_t cols, topk;
  float frac;
};
struct QuantManyArgs {
  int32_t n, bits;
  int32_t* flags;
  int64_t row0[kQuantJobs + 1];
  QuantJob job[kQuantJobs];
};
static_assert(sizeof(QuantManyArgs) <= 4096, "kernel arguments are limited to 4 KB");
hipError_t launch_quantize_many(const QuantManyArgs& a, hipStream_t s);

// ---------------------------------------------------------------------------
// Dequant-fused GEMM: C[m, n] = sum_k A[m, k] * code[n, k], A bf16 [M, K],
// codes int8 [N, K]; the per-row scale of B (and, for normed inputs, the
// per-row RMS factor of A) is applied in the epilogue.
enum EpiKind { EPI_QKV = 0, EPI_RELU2 = 1, EPI_RES = 2 };

struct GemmArgs {
  const bf16* A;          // [M, K]
  const int8_t* B;        // [N, K]
  // the same codes rearranged by launch_shuffle_codes, or null; when set, the
  // row-major epilogues (EPI_RELU2, EPI_RES) feed them from global memory
  // straight into registers instead of staging them through LDS
  const int8_t* Bp;
  const uint16_t* scale;  // [N] binary16
  int32_t M, N, K;
  // RMS factor of the A rows (EPI_QKV, EPI_RELU2): rinv = 1/sqrt(sum_t ss[m,t]/K + eps)
  const float* ss_in;     // [M, nt_in]
  int32_t nt_in;
  float eps;
  // EPI_QKV
  bf16* q; bf16* k; bf16* vt;
  int32_t n_heads, n_kv, hd, Lp;
  const float2* rope;     // [Lp, hd/2] (cos, sin) of rotation pair p
  int32_t rope_dims;      // rotated dims per head (pairs (i, i + rope_dims/2))
  const float* lora_u;    // [M, 2r] or null
  const float* lora_bq;   // [d, r]
  const float* lora_bv;   // [Hkv*hd, r]
  int32_t lora_r;
  // EPI_RELU2: h = leaky_relu(acc, leaky)^2 (leaky 0 = ReLU^2)
  bf16* h;                // [M, N]
  float leaky;
  // EPI_RES
  float* x;               // [M, N] residual, updated in place
  bf16* xb;               // [M, N] bf16 copy of the new x (or null)
  float* ss_out;          // [M, N/128] partial sums of squares (or null)
  float* push_dst;        // [M, N] skip slot to store the new x into (or null)
  const float* pop_src;   // [M, N] skip slot to add (or null); may equal push_dst
  const float* pop_w;     // [N] fp32 skip weight
  // Scored-rows mode (final layer): GEMM row r stands for prediction p0 + r,
  // whose row in the batch layout is RowMap::row(r).  a_map maps the A rows
  // (and ss_in); e_map maps the epilogue's x / xb / ss / skip rows.
  int32_t a_map, e_map;
  int64_t p0, k0, n_win, e0;
  int32_t L, S;
};
// Rearranges int8 codes [N, K] (N % 128 == 0, K % 64 == 0) into the
// fragment order of the register-fed GEMM path; Bp holds N * K bytes.
hipError_t launch_shuffle_codes(const int8_t* B, int32_t N, int32_t K, int8_t* Bp, hipStream_t s);
hipError_t launch_gemm(int epi, const GemmArgs& a, hipStream_t s);

// Row of prediction p in a batch of windows k0.. laid out Lp rows apart:
// window k scores p in [max(kS, e_{k-1}), e_k); window 0 ends at e0.
__host__ __device__ inline int64_t scored_row(int64_t p, int64_t k0, int64_t n_win, int64_t e0,
                                              int32_t L, int32_t S, int32_t Lp) {
  int64_t k = (p < e0) ? 0 : (p - L) / S + 1;
  if (k > n_win - 1) k = n_win - 1;
  return (k - k0) * Lp + (p - k * S);
}

// ---------------------------------------------------------------------------
// Causal GQA attention over a batch of windows.
struct AttnArgs {
  const bf16* q;   // [W, Hq, Lp, hd]
  const bf16* k;   // [W, Hkv, Lp, hd]
  const bf16* vt;  // [W, Hkv, hd, Lp]
  bf16* o;         // [W*Lp, Hq*hd]
  int32_t W, n_heads, n_kv, hd, Lp;
  float scale_log2;  // log2(e) / sqrt(hd)
  // exclusive self attention: remove from each output row its component
  // along the same position's value vector
  int32_t xsa;
  // final layer: only query tiles holding scored positions are computed
  int32_t prune;
  int64_t k0, P;
  int32_t L, S;
};
hipError_t launch_attention(const AttnArgs& a, hipStream_t s);

// ---------------------------------------------------------------------------
// Embedding gather (+ bigram), writes x, bf16 x and row sums of squares.
struct EmbedArgs {
  const int32_t* tokens;
  int64_t n_tokens;
  int64_t P;           // n_tokens - 1
  int64_t k0;          // first window of the batch
  int32_t W, Lp, L, S;
  const void* embed; int32_t embed_f32;
  const float* bigram; // [buckets, d] fp32 (table * proj^T) or null
  int32_t buckets;
  int32_t vocab, d, nt;  // nt partial-sum slots per row
  float* x; bf16* xb; float* ss;
  int32_t* flags;
};
hipError_t launch_embed(const EmbedArgs& a, hipStream_t s);

// LoRA down-projection: u[m, 0:r] = N(x[m]) . aq^T, u[m, r:2r] = N(x[m]) . av^T
struct LoraArgs {
  const float* x; int32_t M, d, r; float eps;
  const float* aq; const float* av;   // [r, d] fp32
  float* u;                           // [M, 2r]
};
hipError_t launch_lora_down(const LoraArgs& a, hipStream_t s);

// Tied head + log-softmax cross-entropy on the scored rows of a batch.
struct HeadArgs {
  const float* x;        // [W*Lp, d]
  const _Float16* E;     // [V, d] binary16
  const int32_t* tokens;
  float* nats;           // [P]
  int64_t p0, p1;        // predictions scored by this batch
  int64_t k0, K, e0;     // first window, window count, end of window 0
  int32_t L, S, Lp, d, vocab;
  float eps;
  float inv_temp;        // logits are multiplied by 1 / temperature
  int32_t* flags;
  int32_t compact;       // 1: row of prediction p is p - p0 (pruned last layer)
};
hipError_t launch_head(const HeadArgs& a, hipStream_t s);

// Totals: sum nats (fp64), sum bytes[p+1] (int64), count, bpb.
struct ReduceArgs {
  const float* nats; const int32_t* bytes; int64_t P;
  double* part_nats; long long* part_bytes; int32_t n_parts;
  double* totals; int32_t* flags;
};
hipError_t launch_reduce(const ReduceArgs& a, hipStream_t s);

// Constant tables built at load time on the device.
hipError_t launch_rope_table(float2* tab, int32_t Lmax, int32_t hd, int32_t rope_dims, double base,
                             hipStream_t s);
hipError_t launch_bigram_table(const uint16_t* table, const uint16_t* proj, float* out,
                               int32_t buckets, int32_t dim, int32_t d, hipStream_t s);
hipError_t launch_f16_to_f32(const uint16_t* in, float* out, int64_t n, hipStream_t s);
hipError_t launch_f32_to_f16(const float* in, _Float16* out, int64_t n, hipStream_t s);
// ORs bit 1 (I6G_FLAG_NONFINITE) into *flags if any of n binary16 (f32 =
// false) or fp32 values is NaN or Inf.
hipError_t launch_check_finite(const void* p, int64_t n, bool f32, int32_t* flags, hipStream_t s);

// ---------------------------------------------------------------------------
// Export side: bit packing of int6 codes (3 bytes per 4) and int5 codes (5
// bytes per 8), its inverse, dequantisation (from int8 codes, bits = 8, or
// packed codes) to fp32 or bfloat16, and the code histogram / entropy.  Code
// and output pointers must be 16-byte aligned, packed pointers 4-byte
// aligned (checked by the callers).
hipError_t launch_pack_codes(const int8_t* codes, int64_t n, int bits, uint8_t* packed, int32_t* flags,
                             hipStream_t s);
hipError_t launch_unpack_codes(const uint8_t* packed, int64_t n, int bits, int8_t* codes, hipStream_t s);
hipError_t launch_dequantize(const void* src, int bits, const uint16_t* scales, int64_t rows, int64_t cols,
                             bool bf16_out, void* out, hipStream_t s);
hipError_t launch_code_histogram(const int8_t* codes, int64_t n, bool accumulate, int64_t* hist, hipStream_t s);
hipError_t launch_code_entropy(const int64_t* hist, double* out, hipStream_t s);

}  // namespace i6g
