// Per-row int8 / int6 / int5 quantiser: a wavefront takes one row, or a
// unit of up to four short rows; rows of up to 2048 columns stay in
// registers between the quantile and the codes, so each weight is read from
// memory once.
//
// pwwt.cn "parameter-golf 16MB 极限压缩实战 …", sections 训练时的模拟量化 and
// 后训练量化导出: scale = clipped |w| maximum / 127 per row, stored binary16;
// codes round(w/scale), in int6 mode round(code/4)*4 clamped to [-128, 124].
// The clip value is the linear-interpolation quantile of |w| over the row
// (at q = 0.99999 84 only the top two order statistics matter for rows up to
// 625,000 long); kwkr.cn PR #363 Noisy-QAT block: floor 1e-12.  int5 (the
// same write-up's MLP_INT5 / ATTN_INT5 export, step amax / 15): scale = c/15,
// codes round(w/scale) clamped to [-16, 15].
//
// Every fp32 operation is rounded on its own (contraction into FMA is off in
// this file) and the codes and scales are bit-identical to a plain binary32
// evaluation.  The quotient w / scale is only rounded to an integer, so the
// register-resident path forms it as w * (1 / scale) and divides only rows
// where that product lies near a half-integer (fast_code).
#include "common.h"

#pragma clang fp contract(off)

namespace i6g {
namespace {

constexpr int kTop = 8;  // most largest |w| a row's quantile may need

template <int KT>
__device__ __attribute__((always_inline)) void insert_top(float (&t)[KT], float a) {
  // t is sorted descending; insert a and drop the smallest.
#pragma unroll
  for (int i = 0; i < KT; ++i) {
    float hi = fmaxf(t[i], a);
    float lo = fminf(t[i], a);
    t[i] = hi;
    a = lo;
  }
}

// Clip value, scale and reciprocal of a row.
struct RowScale {
  float c, scale, inv;
};

// s_hi >= s_lo are the order statistics next to the quantile position.
__device__ inline RowScale row_scale(float s_hi, float s_lo, float frac, int bits) {
  float diff = s_hi - s_lo;
  float step = frac * diff;
  float c = s_lo + step;
  c = fmaxf(c, 1e-12f);
  RowScale r;
  r.c = c;
  r.scale = c / (bits == 5 ? 15.0f : 127.0f);
  // v_rcp_f32 (1 ulp; scale >= 1e-12 / 127 is a normal number): only the
  // register-resident path uses it, with the error bound of fast_code
  r.inv = __builtin_amdgcn_rcpf(r.scale);
  return r;
}

// The code of one weight: clip to [-c, c], divide by the scale (correctly
// rounded), round half to even; int8 clamps to [-127, 127], int5 to
// [-16, 15], int6 rounds again to a multiple of 4 and clamps to [-128, 124].
__device__ inline float quant_code(float w, const RowScale& s, int bits) {
  const float v = fminf(fmaxf(w, -s.c), s.c);
  const float r = v / s.scale;
  const float k = rintf(r);
  if (bits == 8) return fminf(fmaxf(k, -127.0f), 127.0f);
  if (bits == 5) return fminf(fmaxf(k, -16.0f), 15.0f);
  const float k4 = rintf(k * 0.25f);
  return fminf(fmaxf(k4 * 4.0f, -128.0f), 124.0f);
}

// Codes (or fake-quantised values) of columns col .. col + 3.
template <bool FQ>
__device__ inline void store4(float4 x, int col, const RowScale& s, int bits, int8_t* codes, void* fq,
                              int fq_bf16) {
  const float k0 = quant_code(x.x, s, bits), k1 = quant_code(x.y, s, bits);
  const float k2 = quant_code(x.z, s, bits), k3 = quant_code(x.w, s, bits);
  if (FQ) {
    // the codes as integers: a zero code gives +0, as the straight-through
    // sum w + (w_q - w) does
    const float q0 = (float)(int)k0 * s.scale, q1 = (float)(int)k1 * s.scale;
    const float q2 = (float)(int)k2 * s.scale, q3 = (float)(int)k3 * s.scale;
    if (fq_bf16) {
      typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
      typedef float f32x4_t __attribute__((ext_vector_type(4)));
      const f32x4_t f = {q0, q1, q2, q3};
      *reinterpret_cast<bf16x4_t*>(static_cast<__bf16*>(fq) + col) = __builtin_convertvector(f, bf16x4_t);
    } else {
      *reinterpret_cast<float4*>(static_cast<float*>(fq) + col) = make_float4(q0, q1, q2, q3);
    }
  } else {
    const uint32_t packed = ((uint32_t)(uint8_t)(int)k0) | ((uint32_t)(uint8_t)(int)k1 << 8) |
                            ((uint32_t)(uint8_t)(int)k2 << 16) | ((uint32_t)(uint8_t)(int)k3 << 24);
    *reinterpret_cast<uint32_t*>(codes + col) = packed;
  }
}

template <bool FQ>
__device__ inline void store1(float x, int col, const RowScale& s, int bits, int8_t* codes, void* fq,
                              int fq_bf16) {
  const float code = quant_code(x, s, bits);
  if (FQ) {
    const float q = (float)(int)code * s.scale;
    if (fq_bf16) static_cast<__bf16*>(fq)[col] = (__bf16)q;   // v_cvt_pk_bf16_f32: nearest even
    else static_cast<float*>(fq)[col] = q;
  } else {
    codes[col] = (int8_t)(int)code;
  }
}

template <bool FQ>
__device__ inline void store_scale(const RowScale& s, uint16_t* scale_out, int lane) {
  if (!FQ && lane == 0) {
    _Float16 h = (_Float16)s.scale;   // v_cvt_f16_f32: round to nearest even
    *scale_out = __builtin_bit_cast(uint16_t, h);
  }
}

// A row with a NaN or an infinity: codes 0 and a NaN scale (or NaN
// outputs), and bit 0 of *flags.
template <bool FQ>
__device__ void bad_row(int cols, int lane, int8_t* codes, uint16_t* scale_out, int32_t* flags, void* fq,
                        int fq_bf16) {
  for (int c = lane; c < cols; c += kWave) {
    if (FQ) {
      if (fq_bf16) static_cast<uint16_t*>(fq)[c] = 0x7FC0;
      else static_cast<float*>(fq)[c] = __builtin_nanf("");
    } else {
      codes[c] = 0;
    }
  }
  if (lane == 0) {
    if (!FQ) *scale_out = 0x7e00;
    if (flags) atomicOr(flags, 1);
  }
}

// The topk (<= KT) largest of the wave's per-lane sorted lists, extracted
// one at a time; returns the last two extracted as (s_hi, s_lo).
template <int KT>
__device__ __attribute__((always_inline)) void extract_top(float (&top)[KT], int topk, int lane, float& s_hi, float& s_lo) {
  float lo = 0.0f, prev = 0.0f;
  for (int r = 0; r < topk; ++r) {
    float best = top[0];
    int who = lane;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      float ob = __shfl_xor(best, off);
      int ow = __shfl_xor(who, off);
      if (ob > best || (ob == best && ow < who)) { best = ob; who = ow; }
    }
    if (lane == who) {
#pragma unroll
      for (int i = 0; i < KT - 1; ++i) top[i] = top[i + 1];
      top[KT - 1] = -1.0f;
    }
    prev = lo;
    lo = best;
  }
  s_lo = lo;
  s_hi = (topk >= 2) ? prev : lo;
}

// One row of `cols` fp32 weights in two passes over memory, on one
// wavefront (every lane must call it): the KT >= topk largest |w| per lane,
// then the codes.  VEC (cols a multiple of 4, 16-byte aligned rows): a lane
// handles four consecutive columns at a time, so a wavefront moves 1 KiB
// per load and writes four codes per 32-bit store; otherwise one column per
// lane.  FQ: instead of codes and the binary16 scale, write the
// fake-quantised row code * scale (fp32 scale, one rounding) to fq as fp32
// or bfloat16.
template <int KT, bool FQ, bool VEC>
__device__ __attribute__((noinline)) void quantize_row_k(const float* w, int cols, int topk, float frac, int bits, int8_t* codes,
                               uint16_t* scale_out, int32_t* flags, int lane, void* fq, int fq_bf16) {
  // The row is read in chunks of kU elements per lane whose loads are all
  // issued before any is used, so their latencies overlap.
  constexpr int kU = 8;
  constexpr int kV = kU / 4;            // float4 loads per lane per chunk (VEC)
  float top[KT];
#pragma unroll
  for (int i = 0; i < KT; ++i) top[i] = -1.0f;
  int bad = 0;
  for (int c0 = 0; c0 < cols; c0 += kU * kWave) {
    float v[kU];
    if (VEC) {
#pragma unroll
      for (int u = 0; u < kV; ++u) {
        const int c = c0 + 4 * (u * kWave + lane);
        const float4 x = c < cols ? *reinterpret_cast<const float4*>(w + c) : make_float4(0.f, 0.f, 0.f, 0.f);
        v[4 * u] = x.x; v[4 * u + 1] = x.y; v[4 * u + 2] = x.z; v[4 * u + 3] = x.w;
      }
    } else {
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int c = c0 + u * kWave + lane;
        v[u] = c < cols ? w[c] : 0.0f;
      }
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      bad |= !isfinite(v[u]);
      insert_top<KT>(top, fabsf(v[u]));   // a 0 past the row end never displaces a |w|
    }
  }
  if (__any(bad)) {
    bad_row<FQ>(cols, lane, codes, scale_out, flags, fq, fq_bf16);
    return;
  }
  float s_hi, s_lo;
  extract_top<KT>(top, topk, lane, s_hi, s_lo);
  const RowScale rs = row_scale(s_hi, s_lo, frac, bits);

  for (int c0 = 0; c0 < cols; c0 += kU * kWave) {
    if (VEC) {
      float4 wv[kV];
#pragma unroll
      for (int u = 0; u < kV; ++u) {
        const int col = c0 + 4 * (u * kWave + lane);
        wv[u] = col < cols ? *reinterpret_cast<const float4*>(w + col) : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int u = 0; u < kV; ++u) {
        const int col = c0 + 4 * (u * kWave + lane);
        if (col < cols) store4<FQ>(wv[u], col, rs, bits, codes, fq, fq_bf16);
      }
    } else {
      float wv[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int col = c0 + u * kWave + lane;
        wv[u] = col < cols ? w[col] : 0.0f;
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int col = c0 + u * kWave + lane;
        if (col < cols) store1<FQ>(wv[u], col, rs, bits, codes, fq, fq_bf16);
      }
    }
  }
  store_scale<FQ>(rs, scale_out, lane);
}

// The code of a weight in the register-resident path, from p = w * inv
// with inv ~ 1 / scale instead of fl(w / scale), and without clipping w
// to [-c, c] first.
//
// Division: for |w| <= c the quotient t = w / scale has |t| <= 127 (1 +
// 2^-23).  inv (v_rcp_f32) is within 1 ulp of 1 / scale, so p is within
// |t| (2^-23 + 2^-24) (1 + 2^-23) < 2^-15 of t, and fl(t) within 2^-17 of
// t.  When p is at least 2^-14 > 2^-15 + 2^-17 from every half-integer, p,
// t and fl(t) lie strictly between the same two half-integers and round to
// the same integer.  dist keeps the largest |p - rint(p)|; above 1/2 - 2^-14
// the caller redoes the row with quant_code (about one int6 row of 512 in
// seventeen).
// Clipping: |w| > c gives |t| > 127 (int8, int6) or > 15 (int5), so the
// clamps below yield the code of +-c, which is what clipping gives: +-127,
// +-15, or 124 / -128 for int6 (rint(127 / 4) * 4 = 128).  Clipping keeps
// int5 codes in [-15, 15], so that is the clamp here.
// BIAS: the code + 128 (the byte the packed store wants), in as few
// operations as the width allows.
template <int BITS, bool BIAS = false>
__device__ __attribute__((always_inline)) float fast_code(float w, float inv, float& dist) {
  const float r = w * inv;
  const float k = rintf(r);
  dist = fmaxf(dist, fabsf(r - k));
  if (BITS == 8) return BIAS ? __builtin_amdgcn_fmed3f(k + 128.0f, 1.0f, 255.0f) : __builtin_amdgcn_fmed3f(k, -127.0f, 127.0f);
  if (BITS == 5) return BIAS ? __builtin_amdgcn_fmed3f(k + 128.0f, 113.0f, 143.0f) : __builtin_amdgcn_fmed3f(k, -15.0f, 15.0f);
  const float k4 = rintf(k * 0.25f);
  // 4 k4 + 128 is exact (|k4| is small, or the clamp takes over)
  return BIAS ? __builtin_amdgcn_fmed3f(__builtin_fmaf(k4, 4.0f, 128.0f), 0.0f, 252.0f)
              : __builtin_amdgcn_fmed3f(k4 * 4.0f, -128.0f, 124.0f);
}

// Four columns from the register-resident path: fake-quantised values
// (FQ, from codes) or packed codes (from code + 128).
template <bool FQ>
__device__ __attribute__((always_inline)) void put4(float k0, float k1, float k2, float k3, int col, float scale,
                                                    int8_t* codes, void* fq, int fq_bf16) {
  if (FQ) {
    const float q0 = (float)(int)k0 * scale, q1 = (float)(int)k1 * scale;
    const float q2 = (float)(int)k2 * scale, q3 = (float)(int)k3 * scale;
    if (fq_bf16) {
      typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
      typedef float f32x4_t __attribute__((ext_vector_type(4)));
      const f32x4_t f = {q0, q1, q2, q3};
      *reinterpret_cast<bf16x4_t*>(static_cast<__bf16*>(fq) + col) = __builtin_convertvector(f, bf16x4_t);
    } else {
      *reinterpret_cast<float4*>(static_cast<float*>(fq) + col) = make_float4(q0, q1, q2, q3);
    }
  } else {
    // k0 .. k3 are code + 128 (fast_code BIAS): v_cvt_pk_u8_f32 packs each
    // into its byte, the xor takes the bias back off
    uint32_t b = __builtin_amdgcn_cvt_pk_u8_f32(k0, 0, 0u);
    b = __builtin_amdgcn_cvt_pk_u8_f32(k1, 1, b);
    b = __builtin_amdgcn_cvt_pk_u8_f32(k2, 2, b);
    b = __builtin_amdgcn_cvt_pk_u8_f32(k3, 3, b);
    *reinterpret_cast<uint32_t*>(codes + col) = b ^ 0x80808080u;
  }
}

// ---------------------------------------------------------------------------
// Register-resident units (quant_unit_shape 0 .. 3): nr <= R consecutive
// rows of at most 512 NCH columns (a multiple of 4, 16-byte aligned rows)
// and topk <= 2, on one wavefront.  Slot s of the unit's eight float4 per
// lane holds row s / (2 NCH), columns 512 ((s / 2) % NCH) + 4 (64 (s % 2) +
// lane) .. + 3.  Every load of the unit is issued before any is used, so
// R NCH KiB are in flight per wave, and the rows are quantised from
// registers: each weight is read from memory once.

template <int NCH, int R>
__device__ __attribute__((always_inline)) void load_unit(const float* w, int cols, int nr, int lane,
                                                         float4 (&x)[8]) {
#pragma unroll
  for (int s = 0; s < 2 * NCH * R; ++s) {
    const int r = s / (2 * NCH), ch = (s / 2) % NCH, u = s & 1;
    const int c = 512 * ch + 4 * (u * kWave + lane);
    // rows past nr re-read the unit's last row, columns past the end the
    // row's last four; neither is written
    const float* wr = w + (int64_t)min(r, nr - 1) * cols;
    x[s] = *reinterpret_cast<const float4*>(wr + min(c, cols - 4));
  }
}

// The two largest |w| of each row are tracked as bit patterns: for |w|
// (sign cleared) unsigned order is float order, and every NaN or infinity
// is at least 0x7f800000, so the row maximum also tells whether the row is
// finite.  A butterfly of pair merges combines the lanes' pairs, all rows
// at once.
template <int NCH, int R, bool FQ, int BITS>
__device__ __attribute__((always_inline)) void process_unit(float4 (&x)[8], int cols, int nr, int topk, float frac,
                                                            int8_t* codes, uint16_t* scales, int32_t* flags,
                                                            int lane, void* fq, int fq_bf16) {
  if (cols != 512 * NCH) {
    // ragged rows: the lanes past the end hold copies; make them zeros,
    // which never displace a |w| from the top two
#pragma unroll
    for (int s = 0; s < 2 * NCH * R; ++s) {
      const int c = 512 * ((s / 2) % NCH) + 4 * ((s & 1) * kWave + lane);
      if (c >= cols) x[s] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  uint32_t t0[R], t1[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    t0[r] = 0u;
    t1[r] = 0u;
#pragma unroll
    for (int q = 0; q < 2 * NCH; ++q) {
      const float4 f = x[2 * NCH * r + q];
      const float v[4] = {f.x, f.y, f.z, f.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t a = __builtin_bit_cast(uint32_t, v[e]) & 0x7fffffffu;
        t1[r] = max(t1[r], min(t0[r], a));
        t0[r] = max(t0[r], a);
      }
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1)
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const uint32_t u0 = __shfl_xor(t0[r], off), u1 = __shfl_xor(t1[r], off);
      const uint32_t second = max(min(t0[r], u0), max(t1[r], u1));
      t0[r] = max(t0[r], u0);
      t1[r] = second;
    }
  // Clip value, scale and reciprocal of all R rows in one pass: lane r takes
  // row r's pair, and the results are read back from lanes 0 .. R - 1.
  uint32_t m0 = t0[0], m1 = t1[0];
#pragma unroll
  for (int r = 1; r < R; ++r)
    if (lane == r) { m0 = t0[r]; m1 = t1[r]; }
  const float m_hi = __builtin_bit_cast(float, m0);
  const RowScale lane_rs = row_scale(m_hi, topk >= 2 ? __builtin_bit_cast(float, m1) : m_hi, frac, BITS);
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (r >= nr) break;
    int8_t* cr = FQ ? nullptr : codes + (int64_t)r * cols;
    uint16_t* sr = FQ ? nullptr : scales + r;
    void* fr = nullptr;
    if (FQ) fr = fq_bf16 ? (void*)(static_cast<uint16_t*>(fq) + (int64_t)r * cols)
                         : (void*)(static_cast<float*>(fq) + (int64_t)r * cols);
    if (t0[r] >= 0x7f800000u) {   // a NaN or an infinity (uniform: every lane holds the row's pair)
      bad_row<FQ>(cols, lane, cr, sr, flags, fr, fq_bf16);
      continue;
    }
    RowScale rs;
    rs.c = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, lane_rs.c), r));
    rs.scale = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, lane_rs.scale), r));
    rs.inv = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, lane_rs.inv), r));
    float dist = 0.0f;
#pragma unroll
    for (int q = 0; q < 2 * NCH; ++q) {
      const int col = 512 * (q / 2) + 4 * ((q & 1) * kWave + lane);
      const float4 v = x[2 * NCH * r + q];
      const float k0 = fast_code<BITS, !FQ>(v.x, rs.inv, dist), k1 = fast_code<BITS, !FQ>(v.y, rs.inv, dist);
      const float k2 = fast_code<BITS, !FQ>(v.z, rs.inv, dist), k3 = fast_code<BITS, !FQ>(v.w, rs.inv, dist);
      if (col < cols) put4<FQ>(k0, k1, k2, k3, col, rs.scale, cr, fr, fq_bf16);
      // folded into one register here: left to itself the compiler keeps
      // every product and its rounding alive to the end of the row
      asm volatile("" : "+v"(dist));
    }
    if (__builtin_expect(__any(dist > 0.5f - 0x1p-14f), 0)) {
      // a quotient near a half-integer somewhere in the row: the row again
      // with the correctly rounded division (these stores follow the ones
      // above from the same lanes, so they win)
#pragma unroll
      for (int q = 0; q < 2 * NCH; ++q) {
        const int col = 512 * (q / 2) + 4 * ((q & 1) * kWave + lane);
        if (col < cols) store4<FQ>(x[2 * NCH * r + q], col, rs, BITS, cr, fr, fq_bf16);
      }
    }
    store_scale<FQ>(rs, sr, lane);
  }
}

// One unit of a matrix: rows [r0, r0 + nr), r0 = unit * quant_unit_rows.
struct Unit {
  const float* w;
  int8_t* codes;
  uint16_t* scales;
  void* fq;        // fake quantisation output rows (FQ)
  int cols, nr, topk, shape;
  float frac;
};

// The vector path needs 16-byte aligned weight rows and 4-byte aligned code
// rows (or 16 / 8 bytes for fake-quantised fp32 / bf16 rows).
__device__ inline bool vec_ok(const float* w, const void* out, int cols, int out_align) {
  return (cols & 3) == 0 && ((uintptr_t)w & 15) == 0 && ((uintptr_t)out & (out_align - 1)) == 0;
}

// Rows of a kShapeRowwise unit, one by one in two passes over memory.
template <bool FQ>
__device__ __attribute__((always_inline)) void rowwise_unit(const Unit& U, int bits, int32_t* flags, int lane, int fq_bf16) {
  const bool vec = vec_ok(U.w, FQ ? U.fq : (const void*)U.codes, U.cols, FQ ? (fq_bf16 ? 8 : 16) : 4);
  for (int r = 0; r < U.nr; ++r) {
    const float* wr = U.w + (int64_t)r * U.cols;
    int8_t* cr = FQ ? nullptr : U.codes + (int64_t)r * U.cols;
    uint16_t* sr = FQ ? nullptr : U.scales + r;
    void* fr = nullptr;
    if (FQ) fr = fq_bf16 ? (void*)(static_cast<uint16_t*>(U.fq) + (int64_t)r * U.cols)
                         : (void*)(static_cast<float*>(U.fq) + (int64_t)r * U.cols);
    if (U.topk <= 2) {
      if (vec) quantize_row_k<2, FQ, true>(wr, U.cols, U.topk, U.frac, bits, cr, sr, flags, lane, fr, fq_bf16);
      else quantize_row_k<2, FQ, false>(wr, U.cols, U.topk, U.frac, bits, cr, sr, flags, lane, fr, fq_bf16);
    } else {
      if (vec) quantize_row_k<kTop, FQ, true>(wr, U.cols, U.topk, U.frac, bits, cr, sr, flags, lane, fr, fq_bf16);
      else quantize_row_k<kTop, FQ, false>(wr, U.cols, U.topk, U.frac, bits, cr, sr, flags, lane, fr, fq_bf16);
    }
  }
}

// One unit, whatever its shape (a wave-uniform branch; loads and work of a
// shape sit in one case, so its registers never meet another shape's).
template <bool FQ, int BITS>
__device__ __attribute__((always_inline)) void work_unit(const Unit& U, int32_t* flags, int lane, int fq_bf16) {
  float4 x[8];
  switch (U.shape) {
#define I6G_CASE(S, NCH, R)                                                                                  \
  case S:                                                                                                    \
    load_unit<NCH, R>(U.w, U.cols, U.nr, lane, x);                                                           \
    process_unit<NCH, R, FQ, BITS>(x, U.cols, U.nr, U.topk, U.frac, U.codes, U.scales, flags, lane, U.fq,    \
                                   fq_bf16);                                                                 \
    break;
    I6G_CASE(0, 1, 4)
    I6G_CASE(1, 2, 2)
    I6G_CASE(2, 3, 1)
    I6G_CASE(3, 4, 1)
#undef I6G_CASE
    default: rowwise_unit<FQ>(U, BITS, flags, lane, fq_bf16); break;
  }
}

// The wave's index in its workgroup, as a value the compiler knows to be
// uniform, so that row addresses and job lookups stay in scalar registers.
__device__ inline int wave_in_block() { return __builtin_amdgcn_readfirstlane(threadIdx.x / kWave); }

// One matrix, one unit per wave (quantiser: FQ false; fake quantisation:
// the straight-through forward value code * scale of each row, FQ true).
template <bool FQ, int BITS>
__device__ __attribute__((always_inline)) void one_matrix_unit(const QuantArgs& a, int lane) {
  const int per = quant_unit_rows(a.shape);
  const int64_t r0 = ((int64_t)blockIdx.x * (blockDim.x / kWave) + wave_in_block()) * per;
  if (r0 >= a.rows) return;
  Unit U;
  U.w = a.w + r0 * a.cols;
  U.codes = FQ ? nullptr : a.codes + r0 * a.cols;
  U.scales = FQ ? nullptr : a.scales + r0;
  U.fq = nullptr;
  if (FQ) U.fq = a.fq_bf16 ? (void*)(static_cast<uint16_t*>(a.fq) + r0 * a.cols)
                           : (void*)(static_cast<float*>(a.fq) + r0 * a.cols);
  U.cols = a.cols;
  U.nr = (int)min((int64_t)per, a.rows - r0);
  U.topk = a.topk;
  U.shape = a.shape;
  U.frac = a.frac;
  work_unit<FQ, BITS>(U, a.flags, lane, a.fq_bf16);
}

__global__ __launch_bounds__(256) void quantize_rows_kernel(QuantArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  if (a.bits == 6) one_matrix_unit<false, 6>(a, lane);
  else if (a.bits == 8) one_matrix_unit<false, 8>(a, lane);
  else one_matrix_unit<false, 5>(a, lane);
}

__global__ __launch_bounds__(256) void fake_quant_kernel(QuantArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  if (a.bits == 6) one_matrix_unit<true, 6>(a, lane);
  else if (a.bits == 8) one_matrix_unit<true, 8>(a, lane);
  else one_matrix_unit<true, 5>(a, lane);
}

// Units of several matrices, one per wave.  The job of unit u is the number
// of jobs j >= 1 with unit0[j] <= u: lane l tests unit0[l + 1] and
// unit0[l + 65], so two loads and ballots replace a search.
template <int BITS>
__device__ __attribute__((always_inline)) void many_unit(const QuantManyArgs& a, int lane) {
  const int64_t unit = (int64_t)blockIdx.x * (blockDim.x / kWave) + wave_in_block();
  if (unit >= a.unit0[a.n]) return;
  static_assert(kQuantJobs <= 2 * kWave, "two ballots cover the job table");
  const int64_t n1 = lane + 1 < a.n ? a.unit0[lane + 1] : INT64_MAX;
  const int64_t n2 = lane + 1 + kWave < a.n ? a.unit0[lane + 1 + kWave] : INT64_MAX;
  const int j = __popcll(__ballot(n1 <= unit)) + __popcll(__ballot(n2 <= unit));
  const QuantJob& q = a.job[j];
  const int per = quant_unit_rows(q.shape);
  const int64_t r0 = (unit - a.unit0[j]) * per;
  Unit U;
  U.w = q.w + r0 * q.cols;
  U.codes = q.codes + r0 * q.cols;
  U.scales = q.scales + r0;
  U.fq = nullptr;
  U.cols = q.cols;
  U.nr = unit == a.unit0[j + 1] - 1 ? (int)q.last : per;
  U.topk = q.topk;
  U.shape = q.shape;
  U.frac = q.frac;
  work_unit<false, BITS>(U, a.flags, lane, 0);
}

__global__ __launch_bounds__(256) void quantize_many_kernel(QuantManyArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  if (a.bits == 6) many_unit<6>(a, lane);
  else if (a.bits == 8) many_unit<8>(a, lane);
  else many_unit<5>(a, lane);
}

}  // namespace

hipError_t launch_quantize(const QuantArgs& a, hipStream_t s) {
  const int64_t rows_per_block = 4 * (int64_t)quant_unit_rows(a.shape);
  int64_t blocks = (a.rows + rows_per_block - 1) / rows_per_block;
  hipLaunchKernelGGL(quantize_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_fake_quantize(const QuantArgs& a, hipStream_t s) {
  const int64_t rows_per_block = 4 * (int64_t)quant_unit_rows(a.shape);
  int64_t blocks = (a.rows + rows_per_block - 1) / rows_per_block;
  hipLaunchKernelGGL(fake_quant_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_quantize_many(const QuantManyArgs& a, hipStream_t s) {
  const int units_per_block = 4;
  int64_t blocks = (a.unit0[a.n] + units_per_block - 1) / units_per_block;
  hipLaunchKernelGGL(quantize_many_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace i6g
