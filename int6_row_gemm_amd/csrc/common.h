// Internal declarations shared by the HIP kernels and the C-ABI host code.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

namespace i6g {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
// Activations on the scoring path -- the GEMM inputs (the residual stream's
// copy, the attention output, the MLP hidden values), q, k, v and the
// attention probabilities -- are binary16: with 11 significant bits their
// rounding error is 8x below bfloat16's, at the same MFMA rate on gfx950
// (measured against the float64 oracle: mean per-token error about 10x
// lower).  Residual rows beyond the binary16 range are reported (see
// I6G_FLAG_RANGE).
typedef _Float16 act;
typedef _Float16 actx8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// Device flag bit set by the packer for a byte that is not a code of the
// format being packed; equals I6G_FLAG_CODE of the C ABI.
constexpr int32_t kFlagCode = 8;
// Device flag bit set when a value held in binary16 on the scoring path would
// leave its range (a residual row whose sum of squares reaches 65504^2, which
// includes every row holding an element beyond 65504, or an MLP hidden value
// of 65504 or more); equals I6G_FLAG_RANGE of the C ABI.
constexpr int32_t kFlagRange = 16;
constexpr float kRangeSq = 65504.0f * 65504.0f;
constexpr float kRangeSqrt = 255.9375f;   // sqrt(65504) rounded down: v^2 < 65504 for |v| < this

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
  int32_t shape;  // quant_unit_shape of the matrix
};

// How a quantiser wavefront takes rows.  Vector rows (cols a multiple of 4,
// 16-byte aligned weights, aligned outputs) of at most 2048 columns whose
// quantile needs at most the two largest |w| are held in registers, in
// units of one to four rows (at most 8 KiB per wave): shape 0 = four rows
// of <= 512 columns, 1 = two rows of <= 1024, 2 = one row of <= 1536,
// 3 = one row of <= 2048.  Other rows (kShapeRowwise) are read twice, one
// row per wave.
constexpr int kShapeRowwise = 4;
__host__ __device__ inline int quant_unit_shape(int64_t cols, bool vec, int topk) {
  if (!vec || cols > 2048 || topk > 2) return kShapeRowwise;
  return cols <= 512 ? 0 : cols <= 1024 ? 1 : cols <= 1536 ? 2 : 3;
}
__host__ __device__ inline int quant_unit_rows(int shape) { return shape == 0 ? 4 : shape == 1 ? 2 : 1; }

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

// Several matrices in one launch: job j's rows are cut into units of
// quant_unit_rows(shape) rows (its last unit holds `last`), and unit u of
// the concatenation belongs to the last job j with unit0[j] <= u.  The table
// travels in the kernel arguments (at most 4 KiB), so no device buffer is
// needed.
constexpr int kQuantJobs = 80;   // the 66 matrices of an 11-layer model fit one launch
struct QuantJob {
  const float* w;
  int8_t* codes;
  uint16_t* scales;
  int32_t cols;
  int16_t topk;
  uint8_t shape, last;
  float frac;
};
struct QuantManyArgs {
  int32_t n, bits;
  int32_t* flags;
  int64_t unit0[kQuantJobs + 1];
  QuantJob job[kQuantJobs];
};
static_assert(sizeof(QuantManyArgs) <= 4096, "kernel arguments are limited to 4 KB");
hipError_t launch_quantize_many(const QuantManyArgs& a, hipStream_t s);

// ---------------------------------------------------------------------------
// Dequant-fused GEMM: C[m, n] = sum_k A[m, k] * code[n, k], A binary16 [M, K],
// codes int8 [N, K]; the per-row scale of B (and, for normed inputs, the
// per-row RMS factor of A) is applied in the epilogue.
enum EpiKind { EPI_QKV = 0, EPI_RELU2 = 1, EPI_RES = 2 };

struct GemmArgs {
  const act* A;           // [M, K]
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
  act* q; act* k; act* vt;
  int32_t n_heads, n_kv, hd, Lp;
  const float2* rope;     // [Lp, hd/2] (cos, sin) of rotation pair p
  int32_t rope_dims;      // rotated dims per head (pairs (i, i + rope_dims/2))
  const float* lora_u;    // [M, 2r] or null
  const float* lora_bq;   // [d, r]
  const float* lora_bv;   // [Hkv*hd, r]
  int32_t lora_r;
  // EPI_RELU2: h = leaky_relu(acc, leaky)^2 (leaky 0 = ReLU^2)
  act* h;                 // [M, N]
  float leaky;
  // EPI_RES
  float* x;               // [M, N] residual, updated in place
  act* xb;                // [M, N] binary16 copy of the new x (or null)
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
  int32_t* flags;         // kFlagRange (EPI_RELU2, EPI_RES)
};
// Rearranges int8 codes [N, K] (N % 128 == 0, K % 64 == 0) into the
// fragment order of the register-fed GEMM path; Bp holds N * K bytes.  When
// zero_scale_rows (binary16 [N]) is given, rows whose scale is +-0 are
// written as zero codes.
// q/k/v projection as one 128-row tile per workgroup (d_model 512, head size
// 64, no LoRA): codes in per-head fragment order (launch_shuffle_qkv_codes)
// passed as GemmArgs::Bp; the other arguments as for launch_gemm(EPI_QKV).
bool qkv_tile_supported(int32_t d, int32_t hd, int32_t n_heads, int32_t n_kv, int32_t rope_dims, int32_t lora_r);
hipError_t launch_shuffle_qkv_codes(const int8_t* B, int32_t n_heads, int32_t n_kv, int32_t K, int32_t rope_dims,
                                    int8_t* Bp, hipStream_t s);
hipError_t launch_qkv_tile(const GemmArgs& a, hipStream_t s);
hipError_t launch_shuffle_codes(const int8_t* B, int32_t N, int32_t K, const uint16_t* zero_scale_rows, int8_t* Bp,
                                hipStream_t s);
hipError_t launch_gemm(int epi, const GemmArgs& a, hipStream_t s);

// Fused block tail for d_model = 512: x += o . Wo^T; then (sequential
// block) a = N(x), or (parallel lanes) a = N(layer input);
// x += act(a . Wfc^T)^2 . Wproj^T; then the skip push / pop of the block
// schedule, and a binary16 copy of x plus per-128-column sums of squares for the next
// normed GEMM.  One 128-row tile per workgroup; the hidden activations stay
// on chip.  Codes come in the fragment order of launch_shuffle_codes (o and
// proj rows with a zero scale as zero codes).
// The q/k/v projection's codes and outputs, for the one-tile q/k/v kernel
// and for a block tail that computes the next layer's q, k and v from its
// own output rows (frag null: no such phase).
struct QkvOut {
  const int8_t* frag;       // codes in per-head fragment order (launch_shuffle_qkv_codes)
  const uint16_t* scale;    // [(Hq + 2 Hkv) * 64] binary16
  act* q;                   // [W, Hq, Lp, 64]
  act* k;                   // [W, Hkv, Lp, 64]
  act* vt;                  // [W, Hkv, 64, Lp]
  const float2* rope;       // [Lp, 32] (cos, sin) of rotation pair p
  int32_t n_heads, n_kv, rope_dims;
};

struct TailArgs {
  const act* o;             // [rows, 512] attention output
  const int8_t* o_frag;     // Wo [512, 512]
  const uint16_t* o_scale;  // [512] binary16
  const int8_t* fc_frag;    // Wfc [F, 512]
  const uint16_t* fc_scale; // [F]
  const int8_t* proj_frag;  // Wproj [512, F]
  const uint16_t* proj_scale;
  int32_t M, F;
  float eps, leaky;
  const float* x_in;        // [rows, 512] residual read (may equal x)
  float* x;                 // [rows, 512] result (null: stored only to push_dst)
  act* xb;                  // [rows, 512] binary16 copy of the result (or null)
  float* ss_out;            // [rows, 4] per-128-column sums of squares of the result (or null)
  float* push_dst;          // skip slot to store the result into (or null)
  const float* pop_src;     // skip slot added with weight pop_w (or null); may equal push_dst
  const float* pop_w;       // [512] fp32
  // parallel lanes: the MLP input is the layer input, read from xb_in and
  // ss_in (nt_in partial sums per row) before xb and ss_out are written
  int32_t parallel;
  const act* xb_in;
  const float* ss_in;
  int32_t nt_in;
  // scored-rows mode (final layer): tile row r is prediction p0 + r
  int32_t row_map;
  int64_t p0, k0, n_win, e0;
  int32_t L, S, Lp;
  int32_t* flags;           // kFlagRange
  // the next layer's q/k/v projection from this tail's output rows (qkv.frag
  // null: none); needs row_map 0, M and Lp multiples of 64, Lp >= 128
  QkvOut qkv;
  // 1: the residual rows enter the accumulators one row block per output-
  // projection K step (row_map must be 0; results then depend on a row's
  // place in its 128-row tile)
  int32_t spread_residual;
};
hipError_t launch_tail(const TailArgs& a, hipStream_t s);

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
  const act* q;    // [W, Hq, Lp, hd]
  const act* k;    // [W, Hkv, Lp, hd]
  const act* vt;   // [W, Hkv, hd, Lp]
  act* o;          // [W*Lp, Hq*hd]
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
// Embedding gather (+ bigram), writes x, its binary16 copy and row sums of squares.
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
  float* x; act* xb; float* ss;
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
// The same histogram with its partial histograms in the library's static
// device scratch (no allocation); code_histogram_scratch resolves that
// scratch on the current device (first call per device: hipGetSymbolAddress).
hipError_t launch_code_histogram_noalloc(const int8_t* codes, int64_t n, bool accumulate, int64_t* hist,
                                         hipStream_t s);
hipError_t code_histogram_scratch(unsigned long long** out);
// Largest n one histogram launch covers.
int64_t code_histogram_max_codes();
hipError_t launch_code_entropy(const int64_t* hist, double* out, hipStream_t s);

}  // namespace i6g
