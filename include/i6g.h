/*
 * i6g.h -- C ABI of the int6/int8 per-row scoring library for MI355X (gfx950).
 *
 * The library runs the scoring forward pass of a small GPT whose block
 * matrices are stored as per-row integer codes with one binary16 scale per
 * row, and reduces the per-token cross-entropy to bits per byte over
 * sliding windows.  The operations follow these web pages (cited by page
 * and section; the same citations appear beside each entry point):
 *
 *   [11L]  pwwt.cn, "parameter-golf 16MB 极限压缩实战：11L MLP3x + Int6 QAT +
 *          zstd-22 记录详解" -- 训练时的模拟量化, 后训练量化导出, 架构：11 层
 *          U-Net 变压器, 滑动窗口评估：每 64 token 计一次分.
 *   [363]  kwkr.cn write-up of parameter-golf PR #363 "Depth Recurrence +
 *          Mixed-Precision Quantization" -- Middle-Cycle Stem/Core/Tail
 *          layout, DepthLoRA, BigramHash, Noisy-QAT code block.
 *   [RM]   pigsec.cn mirror of the openai/parameter-golf README -- bits per
 *          byte; parallel residual lanes and looped layers 4-5.
 *
 * Conventions
 *   - Pointers named *_dev are HIP device pointers.  Pointers inside
 *     i6g_model_desc may be host or device memory (copied with
 *     hipMemcpyDefault).  All other pointers are host pointers.
 *   - Every function that takes a `stream` enqueues its GPU work on that HIP
 *     stream (hipStream_t passed as void*; NULL = the null stream) and
 *     returns after enqueueing.  Outputs are valid once the stream has
 *     synchronised.
 *   - Functions return an i6g_status.  No function aborts the process.  On
 *     failure i6g_last_error() gives a readable reason (thread-local).
 *   - All arrays are row-major and densely packed.
 */
#ifndef I6G_H
#define I6G_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  I6G_OK = 0,
  I6G_EINVAL = -1,        /* invalid argument (shape, range, null pointer) */
  I6G_ENOMEM = -2,        /* device allocation failed */
  I6G_EDEVICE = -3,       /* a HIP runtime call failed */
  I6G_ENONFINITE = -4,    /* a weight row held NaN or Inf */
  I6G_ETOKEN = -5,        /* a token id outside [0, vocab) */
  I6G_EUNSUPPORTED = -6,  /* valid but unsupported shape (see each call) */
  I6G_EBYTES = -7         /* a negative byte count, or zero total bytes */
} i6g_status;

/* Bits of the device flag word written by kernels (see i6g_quantize_rows and
 * i6g_model_status). */
enum { I6G_FLAG_NONFINITE = 1, I6G_FLAG_TOKEN = 2, I6G_FLAG_BYTES = 4, I6G_FLAG_CODE = 8, I6G_FLAG_RANGE = 16 };

enum { I6G_SKIP_NONE = 0, I6G_SKIP_UNET = 1, I6G_SKIP_STEM_TAIL = 2 };
enum { I6G_DTYPE_F16 = 0, I6G_DTYPE_F32 = 1, I6G_DTYPE_BF16 = 2 };

/*
 * i6g_quantize_rows -- per-row int8 / int6 / int5 quantisation of an fp32
 * matrix.
 *
 * [11L] 训练时的模拟量化 and 后训练量化导出: one scale per row, scale =
 * c / 127 where c is the row's clipped absolute maximum; codes are
 * round(w / scale) and, in int6 mode, round(code / 4) * 4 clamped to
 * [-128, 124] (64 levels in an int8 container); the stored scale is binary16.
 * [363] Noisy-QAT block: c is floored at 1e-12.  [363] run commands
 * (MLP_INT5, ATTN_INT5) and closing notes (int5 step amax / 15): in int5
 * mode scale = c / 15 and codes are round(w / scale) clamped to [-16, 15].
 *
 * Exact steps (all binary32, each operation rounded separately):
 *   c      = s[lo] + f * (s[hi] - s[lo]), s = |w| sorted ascending,
 *            pos = clip_quantile * (cols - 1) (binary64), lo = floor(pos),
 *            hi = min(lo + 1, cols - 1), f = (float)(pos - lo);
 *   c      = max(c, 1e-12f);   scale = c / L (correctly rounded), L = 127.0f
 *            for bits 8 and 6, 15.0f for bits 5;
 *   r      = clamp(w, -c, c) / scale;   k = rint(r) (half to even);
 *   bits 8: code = clamp(k, -127, 127)
 *   bits 6: code = clamp(rint(k / 4) * 4, -128, 124)
 *   bits 5: code = clamp(k, -16, 15)
 *   scale_f16 = binary16 round-to-nearest-even of scale (subnormals kept).
 *
 * w_dev          [rows, cols] fp32, device.
 * bits           5, 6 or 8.
 * clip_quantile  in (0, 1]; 1.0 = plain absolute maximum.
 * codes_dev      [rows, cols] int8 output, device (caller-owned).
 * scales_dev     [rows] binary16 bit patterns output, device (caller-owned).
 * flags_dev      optional device int32; I6G_FLAG_NONFINITE is OR-ed in when
 *                a row holds NaN/Inf (that row's codes are then 0 and its
 *                scale is the binary16 NaN 0x7e00).  May be NULL: the flag
 *                then goes to the library's own latch on the current device,
 *                which i6g_weights_status() reports as I6G_ENONFINITE.
 * Errors: I6G_EINVAL for rows/cols < 1, bits not in {5, 6, 8}, quantile out of
 * (0, 1] or a NULL array; I6G_EUNSUPPORTED if cols - floor(pos) > 8 (the
 * kernel keeps the 8 largest |w| of a row) or cols > 65536.
 */
int i6g_quantize_rows(const float* w_dev, int64_t rows, int64_t cols, int bits,
                      double clip_quantile, int8_t* codes_dev, uint16_t* scales_dev,
                      int32_t* flags_dev, void* stream);

/* One matrix of an i6g_quantize_rows_many call (device pointers). */
typedef struct {
  const float* w;     /* [rows, cols] fp32 */
  int8_t* codes;      /* [rows, cols] int8 output */
  uint16_t* scales;   /* [rows] binary16 output */
  int64_t rows, cols;
} i6g_quant_job;

/*
 * i6g_quantize_rows_many -- i6g_quantize_rows (same steps, same results) on
 * n_jobs matrices at once, the rows of up to 80 matrices in one launch (a
 * wavefront per row or per group of up to four short rows), so that a
 * model's many small matrices fill the device (the export
 * step of [11L] 后训练量化导出 quantises every block matrix this way).
 * jobs is a host array of n_jobs entries; bits, clip_quantile and flags_dev
 * apply to all of them.  Errors: I6G_EINVAL for n_jobs < 1 or a NULL jobs
 * array, otherwise as i6g_quantize_rows for each job (checked before any
 * work is enqueued).
 */
int i6g_quantize_rows_many(const i6g_quant_job* jobs, int32_t n_jobs, int bits, double clip_quantile,
                           int32_t* flags_dev, void* stream);

/*
 * i6g_weights_status -- synchronise `stream`, then report and clear the
 * library's non-finite latch of the current device: I6G_ENONFINITE if any
 * i6g_quantize_rows, i6g_quantize_rows_many, i6g_fake_quantize_rows or
 * i6g_noisy_weights call made with flags_dev NULL on this device met a
 * NaN/Inf weight since the last report ([11L] 后训练量化导出: every exported
 * row has a finite binary16 scale, so such a row cannot be exported), else
 * I6G_OK.  The latch is shared by every caller on the device.
 * Errors: I6G_EDEVICE if the runtime calls fail.
 */
int i6g_weights_status(void* stream);

/*
 * Forward-only quantisation-aware weights (the training forward's view of a
 * weight matrix; no backward pass is involved).
 *
 * i6g_fake_quantize_rows -- [11L] 训练时的模拟量化: the straight-through
 * estimator's forward value w + (w_q - w) = w_q, with w_q = code * scale
 * from the steps of i6g_quantize_rows (same bits and clip_quantile; 1.0 is
 * the plain absolute maximum of the training-time simulation) but the fp32
 * scale, not its binary16 rounding: out = code * scale in fp32 (one
 * rounding), or that value rounded to bfloat16 (nearest even).  A row with
 * NaN/Inf gives NaN outputs and sets I6G_FLAG_NONFINITE in *flags_dev (NULL:
 * in the latch read by i6g_weights_status).  out_dev [rows, cols] fp32 or bf16.  Errors as
 * i6g_quantize_rows, and I6G_EINVAL for an unknown out_dtype.
 */
int i6g_fake_quantize_rows(const float* w_dev, int64_t rows, int64_t cols, int bits, double clip_quantile,
                           int out_dtype, void* out_dev, int32_t* flags_dev, void* stream);

/*
 * i6g_noisy_weights -- [363] Noisy QAT: out = w + (U - 0.5) * step per row,
 * step = max(amax, 1e-12) / levels (127 in the write-up's code block; 15 to
 * match an int5 export), each fp32 operation rounded once.  U is uniform on
 * [0, 1): U = (x >> 8) * 2^-24 with x word (i % 4) of Philox4x32-10 (Salmon,
 * Moraes, Dror, Shaw, SC 2011) at key (seed low 32 bits, seed high 32 bits)
 * and counter (i / 4 low 32 bits, i / 4 high 32 bits, 0, 0), i = r * cols + c.
 * Output fp32, or bfloat16 (nearest even).  A row with NaN/Inf gives NaN
 * outputs and sets I6G_FLAG_NONFINITE in *flags_dev (NULL: in the latch read
 * by i6g_weights_status).  w_dev and out_dev must be 16-byte
 * aligned.  Errors: I6G_EINVAL for rows/cols < 1, levels not positive and
 * finite, an unknown out_dtype or a NULL array; I6G_EUNSUPPORTED for
 * misaligned buffers.
 */
int i6g_noisy_weights(const float* w_dev, int64_t rows, int64_t cols, double levels, uint64_t seed,
                      int out_dtype, void* out_dev, int32_t* flags_dev, void* stream);

/* One quantised [out, in] matrix: codes (int8) and per-row binary16 scales. */
typedef struct {
  const int8_t* codes;
  const uint16_t* scales;
} i6g_matrix;

/* The six matrices of a transformer block, [out, in] each:
 * q [d, d], k [Hkv*hd, d], v [Hkv*hd, d], o [d, d], fc [d_ff, d],
 * proj [d, d_ff]. */
typedef struct {
  i6g_matrix q, k, v, o, fc, proj;
} i6g_block;

/*
 * Model descriptor.  Architecture per [11L] 架构 (GQA attention with RoPE,
 * ReLU^2 MLP, tied embedding, U-Net skips), [363] (Stem/Core x R/Tail with
 * stem->tail skips, DepthLoRA on Q/V per effective depth, BigramHash) and
 * [RM] (parallel attention/MLP lanes, looped layers).
 *
 * vocab, d_model, n_heads, n_kv_heads, head_dim, d_ff   model sizes;
 *     d_model = n_heads * head_dim; n_heads = 2 * n_kv_heads; vocab a
 *     multiple of 64;
 *     head_dim in {32, 64, 80}; d_model and d_ff multiples of 128.
 * rope_base          RoPE base (pairs (i, i + hd/2), theta_i = base^(-2i/hd)).
 * norm_eps           RMSNorm epsilon (no gain).
 * n_unique, blocks   unique blocks (host array of n_unique i6g_block).
 * n_eff, schedule    effective depth and the unique block run at each
 *                    effective layer (host int32 [n_eff]).
 * embed_dtype, embed tied embedding [vocab, d_model], binary16 or fp32.
 * skip_kind, n_skip, skip_weights
 *     I6G_SKIP_UNET: encoder = first n_eff/2 layers push their output;
 *       decoder layer i < n_eff/2 adds skip_weights[i] * pop() first.
 *     I6G_SKIP_STEM_TAIL: the first n_skip layers push; the last n_skip
 *       layers (tail j) add skip_weights[j] * pop() first.
 *     skip_weights is binary16 [n_skip, d_model].
 * parallel_residual  1: x += Attn(N(x)) + MLP(N(x)); 0: sequential.
 * lora_rank, lora_*  rank r (0 = off) and binary16 factors for every
 *     effective layer: aq [n_eff, r, d], bq [n_eff, d, r],
 *     av [n_eff, r, d], bv [n_eff, Hkv*hd, r];
 *     q += (N(x) aq^T) bq^T, v += (N(x) av^T) bv^T.  r <= 8.
 * bigram_buckets, bigram_dim, bigram_table [buckets, dim], bigram_proj
 *     [d, dim] (binary16): x0[j] += proj * table[(u[j-1]*1000003 + u[j])
 *     mod buckets] for window positions j >= 1.  0 buckets = off.
 *
 * Evaluation variants ([363]: EVAL_TEMPERATURE, LeakyReLU, Partial RoPE
 * 16/64, XSA on the last layers); zero selects the base model:
 * logit_temperature  the logits are divided by it before the log-softmax
 *                    (0 or 1 = off; otherwise >= 0.01).
 * leaky_slope        MLP activation leaky_relu(z, slope)^2 (0 = ReLU^2).
 * rope_dims          RoPE on the first rope_dims dims of each head: pairs
 *                    (i, i + rope_dims/2), theta_i = base^(-2i/rope_dims);
 *                    the other dims are not rotated.  0 = head_dim;
 *                    otherwise a multiple of head_dim/4 in [head_dim/4,
 *                    head_dim].
 * xsa_last_n         exclusive self attention on the last xsa_last_n
 *                    effective layers (0..n_eff): each head's attention
 *                    output loses its component along the value vector of
 *                    the same position (unchanged where that vector is 0).
 */
typedef struct {
  int32_t vocab, d_model, n_heads, n_kv_heads, head_dim, d_ff;
  double rope_base, norm_eps;
  int32_t n_unique, n_eff;
  const int32_t* schedule;
  const i6g_block* blocks;
  int32_t embed_dtype;
  const void* embed;
  int32_t skip_kind, n_skip;
  const uint16_t* skip_weights;
  int32_t parallel_residual;
  int32_t lora_rank;
  const uint16_t *lora_aq, *lora_bq, *lora_av, *lora_bv;
  int32_t bigram_buckets, bigram_dim;
  const uint16_t *bigram_table, *bigram_proj;
  double logit_temperature, leaky_slope;
  int32_t rope_dims, xsa_last_n;
} i6g_model_desc;

typedef struct i6g_model i6g_model; /* opaque, owned by the library */

/*
 * i6g_load_model -- copy a quantised model into library-owned device memory
 * on the current HIP device and prepare its constant tables.  The caller may
 * free everything `desc` points to once the stream has synchronised.
 * Errors: I6G_EINVAL (inconsistent sizes, bad schedule or skip plan, NULL
 * tensors), I6G_EUNSUPPORTED (head_dim, head ratio or tile alignment not
 * supported; a logit_temperature in (0, 0.01): the head holds the normed
 * row times log2(e) / temperature in binary16), I6G_ENONFINITE (a NaN or Inf
 * row scale, embedding value, skip weight, LoRA factor or bigram value:
 * checked on the host before any allocation for tensors in host memory, and
 * on the device after the copy for the others), I6G_ENOMEM, I6G_EDEVICE.
 * On error *out is NULL.
 */
int i6g_load_model(const i6g_model_desc* desc, void* stream, i6g_model** out);

/*
 * i6g_score_tokens -- sliding-window scoring of a token stream.
 *
 * [11L] 滑动窗口评估: windows of `window` tokens every `stride` tokens, each
 * scored on its last `stride` positions, every token evaluated with up to a
 * full window of context; the chunked eval is stride == window.
 * [RM]: the score is bits per byte.
 *
 * Exact plan: P = n_tokens - 1 predictions, prediction p predicts
 * tokens[p+1]; window k has inputs tokens[s_k, e_k) at positions
 * 0..e_k-s_k-1 with s_k = k*stride, e_k = min(s_k + window, P), and scores
 * p in [max(s_k, e_{k-1}), e_k) (e_{-1} = 0); K = 1 + ceil((P - window) /
 * stride) windows (1 if P <= window).  Every prediction is scored once.
 *
 * tokens_dev  [n_tokens] int32 token ids, device.
 * bytes_dev   [n_tokens] int32 byte count of each token, device.
 * nats_dev    [n_tokens - 1] fp32 output: nats_dev[p] = -ln p(tokens[p+1]).
 * totals_dev  [4] fp64 output: sum of nats, sum of bytes[1..P], number of
 *             scored predictions (P), bits per byte = sum_nats / (ln 2 *
 *             sum_bytes).
 * Errors (returned now): I6G_EINVAL for n_tokens < 2, window < 1,
 * stride < 1 or > window, NULL arrays, or a current HIP device other than
 * the one the model was loaded on (the model's memory lives there);
 * I6G_EUNSUPPORTED when one window of min(window, n_tokens - 1) positions,
 * rounded up to 64, exceeds the rows a batch can hold (row and tile
 * indices are 32-bit in the kernels): at most 2^24 - 1, and at most
 * 128 * floor((2^31 - 1) / ceil(w / 64)) for w = max(d_model +
 * 2*n_kv_heads*head_dim, d_ff); I6G_ENOMEM; I6G_EDEVICE.
 * Errors detected on the device (token outside [0, vocab): that token is
 * read as id 0; negative byte count: counted as 0) are latched in the
 * model and returned by i6g_model_status().
 * A model must not be used from two streams at once (its scratch is shared).
 */
int i6g_score_tokens(i6g_model* m, const int32_t* tokens_dev, const int32_t* bytes_dev,
                     int64_t n_tokens, int32_t window, int32_t stride, float* nats_dev,
                     double* totals_dev, void* stream);

/* Synchronise `stream`, then return and clear the device-side error latch of
 * `m`: I6G_ETOKEN, I6G_EBYTES, I6G_EUNSUPPORTED or I6G_OK.  I6G_EUNSUPPORTED
 * (I6G_FLAG_RANGE): the scoring pass holds its GEMM inputs, q, k, v, the
 * attention probabilities and output and the MLP hidden values in binary16
 * (fp32 accumulation; the residual stream itself is fp32), and a residual
 * row whose sum of squares reached 65504^2 or an MLP hidden value of 65504
 * or more was met; the nats of that call are not valid. */
int i6g_model_status(i6g_model* m, void* stream);

/* Release a model and its scratch.  NULL is ignored.  The caller must have
 * synchronised every stream that used it. */
void i6g_free_model(i6g_model* m);

/* Text of the last failure on this thread ("" if none). */
const char* i6g_last_error(void);

/*
 * i6g_plan_windows -- the window plan of i6g_score_tokens, on the host
 * (no GPU needed).  Writes min(K, capacity) entries of starts/ends/score_from
 * (each may be NULL) and the window count K to *n_windows.
 * Errors: I6G_EINVAL as for i6g_score_tokens.
 */
int i6g_plan_windows(int64_t n_tokens, int32_t window, int32_t stride, int64_t* n_windows,
                     int64_t* starts, int64_t* ends, int64_t* score_from, int64_t capacity);

/* Model options (tuning and testing; results do not depend on them beyond
 * floating-point rounding):
 *   I6G_OPT_BATCH_WINDOWS  windows per batch in i6g_score_tokens (0 = the
 *                          default: about 131072 rows per batch with the
 *                          fused block tail, 49152 without); an upper
 *                          bound: a batch is also kept within the rows
 *                          i6g_score_tokens can index (at most 2^24 - 1);
 *   I6G_OPT_PRUNE_LAST     1 (default): the final layer computes queries,
 *                          the output projection and the MLP only for the
 *                          scored rows; 0: for every row.
 *   I6G_OPT_STREAMS        1 (default): every batch on the caller's
 *                          stream.  2: consecutive batches alternate between
 *                          the caller's stream and a second stream the
 *                          model owns (default priority), each with its own
 *                          scratch, so their kernels can overlap; the
 *                          second stream waits for the caller's earlier work
 *                          and the caller's stream waits for it before the
 *                          totals are reduced.  Results are identical.
 *   I6G_OPT_REGISTER_CODES 1 (default): the fc and proj GEMMs load their
 *                          weight codes, rearranged into fragment order when
 *                          the model is loaded, straight into registers; 0:
 *                          they stage the row-major codes through LDS like
 *                          the q/k/v and output projections.  The
 *                          MFMAs are the same; the per-row sums of squares
 *                          for the next norm are added in another order, so
 *                          results agree to fp32 rounding.
 *   I6G_OPT_FUSED_TAIL     1 (default): for d_model = 512 (and streams of
 *                          fewer than 2^31 tokens) each block's output
 *                          projection, norm and MLP run as one kernel per
 *                          128-row tile, the hidden activations never
 *                          leaving the chip; 0: as three GEMM launches.  The
 *                          same products in another rounding order: results
 *                          agree to fp32 rounding of the residual.
 *   I6G_OPT_QKV_TILE       1 (default): for d_model = 512, head size 64 and
 *                          no LoRA (and windows of at least 128 positions
 *                          after padding to 64), the q/k/v projection runs as
 *                          one kernel per 128-row tile computing every head
 *                          of it, with the codes rearranged into per-head
 *                          fragment order when the model is loaded; with
 *                          the fused block tail on, each tail but the last
 *                          (and one whose rows are pruned) runs the same
 *                          per-head loop on its own output rows for the
 *                          next layer, so only the first layer's q/k/v has a
 *                          launch of its own; 0: the LDS-staged GEMM.  The
 *                          same products accumulated in the same order:
 *                          results are identical.
 * Errors: I6G_EINVAL for an unknown option or a value out of range. */
enum {
  I6G_OPT_BATCH_WINDOWS = 0, I6G_OPT_PRUNE_LAST = 1, I6G_OPT_STREAMS = 2, I6G_OPT_REGISTER_CODES = 3,
  I6G_OPT_FUSED_TAIL = 4, I6G_OPT_QKV_TILE = 5
};
int i6g_set_option(i6g_model* m, int option, int64_t value);

/* Per-launch kernel timing with HIP events, for measurement.  Kernel
 * classes: */
enum {
  I6G_K_EMBED = 0, I6G_K_QKV = 1, I6G_K_ATTN = 2, I6G_K_OPROJ = 3, I6G_K_FC = 4,
  I6G_K_PROJ = 5, I6G_K_HEAD = 6, I6G_K_REDUCE = 7, I6G_K_LORA = 8, I6G_K_TAIL = 9, I6G_K_COUNT = 10
};
/* enable != 0 records an event pair around every launch of the classes in
 * `class_mask` (bit i = class i) in later i6g_score_tokens calls; counters
 * are reset.  Event timestamps are collected when the stream is synchronised
 * by i6g_get_timing. */
int i6g_set_timing(i6g_model* m, int enable, uint32_t class_mask);
/* Synchronise the timed stream and report, for one kernel class, the summed
 * launch durations (ms), the number of launches, and the algorithmic FLOPs
 * and bytes of those launches. */
int i6g_get_timing(i6g_model* m, int kernel_class, double* total_ms, int64_t* launches,
                   double* flops, double* bytes);

/*
 * Export side.  [363] timeline and run notes: the codes are sized by their
 * entropy in bits per value, compressed (bit packing among the methods
 * tried) into an artifact of at most 16,000,000 bytes, then dequantised and
 * evaluated again; its run commands export int5 matrices (MLP_INT5,
 * ATTN_INT5).  [11L] 后训练量化导出: int6 codes are int8 multiples of 4 in
 * [-128, 124] with one binary16 scale per row.
 *
 * Packed formats (bits), least significant bit first:
 *   6: code c -> u = c/4 + 32 in [0, 63]; four codes u0..u3 make the 24-bit
 *      word u0 | u1 << 6 | u2 << 12 | u3 << 18, stored as 3 bytes;
 *      n codes take 3 * ceil(n / 4) bytes;
 *   5: code c -> u = c + 16 in [0, 31]; eight codes make the 40-bit word
 *      sum u_i << 5i, stored as 5 bytes; n codes take 5 * ceil(n / 8) bytes;
 * a tail shorter than a word is padded with code 0.  Code buffers and
 * fp32/bf16 outputs must be 16-byte aligned and packed buffers 4-byte
 * aligned (I6G_EUNSUPPORTED otherwise); n = 0 enqueues nothing.
 */

/* i6g_pack_codes -- n codes (int8) -> their packed bytes (bits 5 or 6).  A
 * byte that is not a code of the format (int6: not a multiple of 4; int5:
 * outside [-16, 15]) is packed from its low bits and I6G_FLAG_CODE is OR-ed
 * into *flags_dev (may be NULL).  Errors: I6G_EINVAL for bits not in {5, 6},
 * n < 0 or a NULL buffer with n > 0. */
int i6g_pack_codes(const int8_t* codes_dev, int64_t n, int bits, uint8_t* packed_dev, int32_t* flags_dev,
                   void* stream);

/* i6g_unpack_codes -- the inverse: the first n codes held in packed_dev ->
 * codes_dev [n] int8.  Errors as i6g_pack_codes. */
int i6g_unpack_codes(const uint8_t* packed_dev, int64_t n, int bits, int8_t* codes_dev, void* stream);

/* i6g_dequantize_rows -- out[r, c] = code[r, c] * scale[r] for a [rows, cols]
 * matrix of int8 codes (int8, int6 or int5) and binary16 row scales.
 * out_dtype I6G_DTYPE_F32: the exact product (an int8 times a binary16 has at
 * most 19 significant bits); I6G_DTYPE_BF16: that product rounded to
 * bfloat16, nearest with ties to even (a NaN stays a NaN).  out_dev [rows, cols].
 * Errors: I6G_EINVAL for rows or cols < 0, an unknown dtype or a NULL
 * buffer; I6G_EUNSUPPORTED for misaligned buffers. */
int i6g_dequantize_rows(const int8_t* codes_dev, const uint16_t* scales_dev, int64_t rows, int64_t cols,
                        int out_dtype, void* out_dev, void* stream);

/* i6g_dequantize_packed -- i6g_dequantize_rows with the codes read from their
 * packed form (bits 5 or 6: the rows * cols codes of the matrix, row-major,
 * packed by i6g_pack_codes): the decode step of loading an artifact, without
 * the unpacked codes ever reaching memory.  Same results; errors as
 * i6g_dequantize_rows, and I6G_EINVAL for bits not in {5, 6}. */
int i6g_dequantize_packed(const uint8_t* packed_dev, int bits, const uint16_t* scales_dev, int64_t rows,
                          int64_t cols, int out_dtype, void* out_dev, void* stream);

/* i6g_code_histogram -- counts of each int8 value among n codes:
 * hist_dev[v + 128] (int64 [256]).  accumulate = 0 overwrites the
 * histogram; 1 adds to it, so several matrices can share one histogram.
 * Uses 128 KiB of stream-ordered temporary device memory (hipMallocAsync /
 * hipFreeAsync on `stream`).  Errors: I6G_EINVAL for n < 0 or NULL buffers;
 * I6G_ENOMEM if the temporary memory cannot be had; I6G_EUNSUPPORTED for n
 * beyond the codes one call covers (2^31 - 1 workgroups of 8,192 codes). */
int i6g_code_histogram(const int8_t* codes_dev, int64_t n, int accumulate, int64_t* hist_dev,
                       void* stream);

/* i6g_code_histogram_noalloc -- i6g_code_histogram (same counts) for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation.  It allocates
 * nothing: its 64 partial histograms (128 KiB) live in a static device array
 * of the library, one per device, held until the process ends; the first
 * call on a device resolves that array's address on it.  Every call on one
 * device shares the array and clears it first (with a kernel), so calls that
 * overlap on one device -- on different streams or host threads -- race and
 * must be serialised by the caller.  Errors: as i6g_code_histogram
 * (I6G_EUNSUPPORTED for n beyond the codes one call covers: 2^31 - 1
 * workgroups of 8,192 codes). */
int i6g_code_histogram_noalloc(const int8_t* codes_dev, int64_t n, int accumulate, int64_t* hist_dev,
                               void* stream);

/* i6g_code_entropy -- Shannon entropy in bits per value of a 256-bin
 * histogram of non-negative counts: -sum p log2 p over the bins with a
 * positive count, p = count / total (fp64); 0 if the total is 0.  Writes one
 * double to bits_dev.  Errors: I6G_EINVAL for NULL buffers. */
int i6g_code_entropy(const int64_t* hist_dev, double* bits_dev, void* stream);

/* i6g_artifact_bytes -- host only: bytes of a packed artifact holding
 * n_mats matrices (shapes[2 i] rows, shapes[2 i + 1] cols, bits[i] in
 * {5, 6, 8}; bits may be NULL for all-int6): each its packed codes (int8 at
 * one byte per code) plus 2 bytes per row scale, and passthrough_elements
 * binary16 values (2 bytes each).  Compare the result with
 * I6G_ARTIFACT_LIMIT.  Errors: I6G_EINVAL for a negative count or size, a
 * bit width outside {5, 6, 8}, or NULL shapes with n_mats > 0. */
#define I6G_ARTIFACT_LIMIT 16000000LL
int i6g_artifact_bytes(const int64_t* shapes, const int32_t* bits, int32_t n_mats,
                       int64_t passthrough_elements, int64_t* bytes);

#ifdef __cplusplus
}
#endif

#endif /* I6G_H */
