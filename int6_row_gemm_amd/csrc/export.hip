// Export side of the int6 / int5 formats: bit packing, unpacking,
// dequantisation and code statistics.
//
// kwkr.cn write-up of parameter-golf PR #363, timeline and run notes: the
// codes are measured by their entropy (bits per value) and compressed (bit
// packing among the methods tried) into an artifact of at most 16,000,000
// bytes, which is dequantised and evaluated again; its run commands export
// int5 matrices (MLP_INT5, ATTN_INT5).  pwwt.cn "parameter-golf 16MB 极限压缩
// 实战 …", 后训练量化导出: int6 codes are int8 multiples of 4 in
// [-128, 124] with one binary16 scale per row.
//
// Packed formats, least significant bit first:
//   int6: code c -> u = c/4 + 32 (6 bits); 4 codes -> 3 bytes;
//   int5: code c -> u = c + 16 (5 bits);   8 codes -> 5 bytes;
// a tail shorter than a word is padded with code 0.
//
// All kernels are bound by HBM traffic.  A thread moves one group of codes
// per step (16 int6 codes = one 16-byte load and 12 packed bytes; 32 int5
// codes = two 16-byte loads and 20 packed bytes; 16 int8 codes for the
// dequantisation of unpacked codes) and issues its kU groups' loads before
// using any, so that enough bytes are in flight to cover HBM latency (the
// registers are zeroed first: without that the compiler waits for each
// group's load before issuing the next).  The
// last, partial group of a buffer is done one word at a time by the thread
// whose group index is the group count.
#include "common.h"

#include <mutex>

namespace i6g {
namespace {

constexpr int kU = 2;           // groups per thread
constexpr int kThreads = 256;   // threads per workgroup
constexpr int64_t kGroupsPerBlock = (int64_t)kU * kThreads;
constexpr int kHistParts = 64;  // partial histograms (see hist_kernel)

// Group and word geometry of each code format (8: unpacked int8 codes).
template <int BITS> struct Fmt;
template <> struct Fmt<6> { static constexpr int G = 16, PB = 12, WC = 4, WB = 3; };
template <> struct Fmt<5> { static constexpr int G = 32, PB = 20, WC = 8, WB = 5; };
template <> struct Fmt<8> { static constexpr int G = 16, PB = 16, WC = 1, WB = 1; };

// --- int6: four codes, one per byte of x, <-> a 24-bit packed word.  For a
// code c = 4t (t in [-32, 31]) bits 2..7 of the byte are t in 6-bit two's
// complement, and t + 32 mod 64 flips its top bit.
__device__ inline uint32_t pack6x4(uint32_t x) {
  const uint32_t y = ((x >> 2) & 0x3F3F3F3Fu) ^ 0x20202020u;
  return (y & 0x3Fu) | ((y >> 2) & 0xFC0u) | ((y >> 4) & 0x3F000u) | ((y >> 6) & 0xFC0000u);
}
__device__ inline uint32_t unpack6x4(uint32_t w) {
  const uint32_t y = (w & 0x3Fu) | ((w << 2) & 0x3F00u) | ((w << 4) & 0x3F0000u) | ((w << 6) & 0x3F000000u);
  return (y ^ 0x20202020u) << 2;
}
// a byte is an int6 code iff its low two bits are clear
__device__ inline bool bad6(uint32_t x) { return (x & 0x03030303u) != 0; }

// --- int5: four codes <-> a 20-bit word.  The low 5 bits of a code in
// [-16, 15] are its 5-bit two's complement; + 16 mod 32 flips bit 4.
__device__ inline uint32_t pack5x4(uint32_t x) {
  const uint32_t y = (x ^ 0x10101010u) & 0x1F1F1F1Fu;
  return (y & 0x1Fu) | ((y >> 3) & 0x3E0u) | ((y >> 6) & 0x7C00u) | ((y >> 9) & 0xF8000u);
}
__device__ inline uint32_t unpack5x4(uint32_t w) {
  const uint32_t y = (w & 0x1Fu) | ((w << 3) & 0x1F00u) | ((w << 6) & 0x1F0000u) | ((w << 9) & 0x1F000000u);
  const uint32_t v = y ^ 0x10101010u;       // 5-bit two's complement per byte
  return v | ((v & 0x10101010u) * 14u);     // sign-extend: bit 4 -> bits 5..7
}
// a byte is an int5 code iff its bits 4..7 are equal
__device__ inline bool bad5(uint32_t x) { return ((x ^ (x << 1)) & 0xE0E0E0E0u) != 0; }

// A group's codes (G/4 words of 4 codes) -> its packed words (PB/4).
__device__ inline void pack_group(const uint32_t (&c)[4], uint32_t (&p)[3]) {
  const uint32_t w0 = pack6x4(c[0]), w1 = pack6x4(c[1]), w2 = pack6x4(c[2]), w3 = pack6x4(c[3]);
  p[0] = w0 | (w1 << 24);
  p[1] = (w1 >> 8) | (w2 << 16);
  p[2] = (w2 >> 16) | (w3 << 8);
}
__device__ inline void unpack_group(const uint32_t (&p)[3], uint32_t (&c)[4]) {
  c[0] = unpack6x4(p[0] & 0xFFFFFFu);
  c[1] = unpack6x4((p[0] >> 24) | ((p[1] & 0xFFFFu) << 8));
  c[2] = unpack6x4((p[1] >> 16) | ((p[2] & 0xFFu) << 16));
  c[3] = unpack6x4(p[2] >> 8);
}
__device__ inline uint64_t pack5x8(uint32_t lo, uint32_t hi) {
  return (uint64_t)pack5x4(lo) | ((uint64_t)pack5x4(hi) << 20);
}
__device__ inline void pack_group(const uint32_t (&c)[8], uint32_t (&p)[5]) {
  const uint64_t q0 = pack5x8(c[0], c[1]), q1 = pack5x8(c[2], c[3]);
  const uint64_t q2 = pack5x8(c[4], c[5]), q3 = pack5x8(c[6], c[7]);
  p[0] = (uint32_t)q0;
  p[1] = (uint32_t)(q0 >> 32) | (uint32_t)(q1 << 8);
  p[2] = (uint32_t)(q1 >> 24) | (uint32_t)(q2 << 16);
  p[3] = (uint32_t)(q2 >> 16) | (uint32_t)(q3 << 24);
  p[4] = (uint32_t)(q3 >> 8);
}
__device__ inline void unpack_group(const uint32_t (&p)[5], uint32_t (&c)[8]) {
  const uint64_t q[4] = {
      (uint64_t)p[0] | ((uint64_t)(p[1] & 0xFFu) << 32),
      (uint64_t)(p[1] >> 8) | ((uint64_t)(p[2] & 0xFFFFu) << 24),
      (uint64_t)(p[2] >> 16) | ((uint64_t)(p[3] & 0xFFFFFFu) << 16),
      (uint64_t)(p[3] >> 24) | ((uint64_t)p[4] << 8)};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    c[2 * j] = unpack5x4((uint32_t)q[j] & 0xFFFFFu);
    c[2 * j + 1] = unpack5x4((uint32_t)(q[j] >> 20) & 0xFFFFFu);
  }
}

// One word (WC codes in the low bytes of a uint64, WB packed bytes) of the
// tail, for formats 6 and 5.
template <int BITS> __device__ inline uint64_t pack_word(uint64_t codes);
template <> __device__ inline uint64_t pack_word<6>(uint64_t c) { return pack6x4((uint32_t)c); }
template <> __device__ inline uint64_t pack_word<5>(uint64_t c) { return pack5x8((uint32_t)c, (uint32_t)(c >> 32)); }
template <int BITS> __device__ inline uint64_t unpack_word(uint64_t w);
template <> __device__ inline uint64_t unpack_word<6>(uint64_t w) { return unpack6x4((uint32_t)w); }
template <> __device__ inline uint64_t unpack_word<5>(uint64_t w) {
  return (uint64_t)unpack5x4((uint32_t)w & 0xFFFFFu) | ((uint64_t)unpack5x4((uint32_t)(w >> 20) & 0xFFFFFu) << 32);
}
template <int BITS> __device__ inline bool bad_word(uint32_t x);
template <> __device__ inline bool bad_word<6>(uint32_t x) { return bad6(x); }
template <> __device__ inline bool bad_word<5>(uint32_t x) { return bad5(x); }

// Tail word j: codes idx0 .. idx0 + WC - 1 (those below n), zero padded.
template <int BITS>
__device__ inline uint64_t gather_codes(const int8_t* codes, int64_t idx0, int64_t n) {
  uint64_t x = 0;
  for (int b = 0; b < Fmt<BITS>::WC; ++b)
    if (idx0 + b < n) x |= (uint64_t)(uint8_t)codes[idx0 + b] << (8 * b);
  return x;
}
template <int BITS>
__device__ inline uint64_t gather_packed(const uint8_t* p) {
  uint64_t w = 0;
  for (int b = 0; b < Fmt<BITS>::WB; ++b) w |= (uint64_t)p[b] << (8 * b);
  return w;
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// bfloat16 bits of (a, b) in the low / high half, round to nearest with
// ties to even (one v_cvt_pk_bf16_f32); a NaN stays a NaN.
__device__ inline uint32_t bf16x2_rne(float a, float b) {
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ inline float f16_bits_to_float(uint16_t s) { return (float)__builtin_bit_cast(_Float16, s); }

// Loads of group g: NW 32-bit words at byte offset NW * 4 * g (16-byte loads
// where NW is a multiple of 4).
template <int NW>
__device__ inline void load_words(const void* base, int64_t g, uint32_t (&d)[NW]) {
  const uint32_t* p = reinterpret_cast<const uint32_t*>(base) + NW * g;
  if (NW % 4 == 0) {
#pragma unroll
    for (int i = 0; i < NW / 4; ++i) {
      const uint4 v = reinterpret_cast<const uint4*>(p)[i];
      d[4 * i] = v.x; d[4 * i + 1] = v.y; d[4 * i + 2] = v.z; d[4 * i + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < NW; ++i) d[i] = p[i];
  }
}
template <int NW>
__device__ inline void store_words(void* base, int64_t g, const uint32_t (&d)[NW]) {
  uint32_t* p = reinterpret_cast<uint32_t*>(base) + NW * g;
  if (NW % 4 == 0) {
#pragma unroll
    for (int i = 0; i < NW / 4; ++i)
      reinterpret_cast<uint4*>(p)[i] = make_uint4(d[4 * i], d[4 * i + 1], d[4 * i + 2], d[4 * i + 3]);
  } else {
#pragma unroll
    for (int i = 0; i < NW; ++i) p[i] = d[i];
  }
}

template <int BITS>
__global__ __launch_bounds__(kThreads) void pack_kernel(const int8_t* codes, int64_t n, uint8_t* packed,
                                                        int32_t* flags) {
  using F = Fmt<BITS>;
  const int64_t ng = n / F::G;
  const int64_t gb = blockIdx.x * kGroupsPerBlock + threadIdx.x;
  bool bad = false;
  uint32_t c[kU][F::G / 4];
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    const int64_t g = gb + u * kThreads;
#pragma unroll
    for (int i = 0; i < F::G / 4; ++i) c[u][i] = 0;
    if (g < ng) load_words<F::G / 4>(codes, g, c[u]);
  }
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    const int64_t g = gb + u * kThreads;
    if (g < ng) {
      uint32_t p[F::PB / 4];
#pragma unroll
      for (int i = 0; i < F::G / 4; ++i) bad |= bad_word<BITS>(c[u][i]);
      pack_group(c[u], p);
      store_words<F::PB / 4>(packed, g, p);
    } else if (g == ng && n % F::G) {
      for (int64_t j = 0; F::G * ng + F::WC * j < n; ++j) {
        const int64_t idx0 = F::G * ng + F::WC * j;
        const uint64_t x = gather_codes<BITS>(codes, idx0, n);
        bad |= bad_word<BITS>((uint32_t)x) || bad_word<BITS>((uint32_t)(x >> 32));
        const uint64_t w = pack_word<BITS>(x);
        uint8_t* o = packed + F::PB * ng + F::WB * j;
        for (int b = 0; b < F::WB; ++b) o[b] = (uint8_t)(w >> (8 * b));
      }
    }
  }
  if (bad && flags) atomicOr(flags, kFlagCode);
}

template <int BITS>
__global__ __launch_bounds__(kThreads) void unpack_kernel(const uint8_t* packed, int64_t n, int8_t* codes) {
  using F = Fmt<BITS>;
  const int64_t ng = n / F::G;
  const int64_t gb = blockIdx.x * kGroupsPerBlock + threadIdx.x;
  uint32_t p[kU][F::PB / 4];
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    const int64_t g = gb + u * kThreads;
#pragma unroll
    for (int i = 0; i < F::PB / 4; ++i) p[u][i] = 0;
    if (g < ng) load_words<F::PB / 4>(packed, g, p[u]);
  }
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    const int64_t g = gb + u * kThreads;
    if (g < ng) {
      uint32_t c[F::G / 4];
      unpack_group(p[u], c);
      store_words<F::G / 4>(codes, g, c);
    } else if (g == ng && n % F::G) {
      for (int64_t j = 0; F::G * ng + F::WC * j < n; ++j) {
        const uint64_t x = unpack_word<BITS>(gather_packed<BITS>(packed + F::PB * ng + F::WB * j));
        for (int b = 0; b < F::WC; ++b) {
          const int64_t idx = F::G * ng + F::WC * j + b;
          if (idx < n) codes[idx] = (int8_t)(x >> (8 * b));
        }
      }
    }
  }
}

// out[i] = code[i] * scale[i / cols] for the G codes of group g (four per
// word of c), written as fp32 or bfloat16.  ROWG: cols is a multiple of G,
// so the whole group lies in one row, and rows * cols < 2^32.
template <int G, bool BF16, bool ROWG>
__device__ inline void dequant_group(const uint32_t (&c)[G / 4], int64_t g, int64_t cols, const uint16_t* scales,
                                     void* out) {
  float v[G];
  if (ROWG) {
    // 32-bit division: a few instructions where 64-bit division is a long sequence
    const float s = f16_bits_to_float(scales[(uint32_t)(G * g) / (uint32_t)cols]);
#pragma unroll
    for (int i = 0; i < G; ++i) v[i] = (float)(int8_t)((c[i >> 2] >> (8 * (i & 3))) & 0xFF) * s;
  } else {
    int64_t r = (G * g) / cols, col = G * g - r * cols;
#pragma unroll
    for (int i = 0; i < G; ++i) {
      while (col >= cols) { col -= cols; ++r; }
      v[i] = (float)(int8_t)((c[i >> 2] >> (8 * (i & 3))) & 0xFF) * f16_bits_to_float(scales[r]);
      ++col;
    }
  }
  if (BF16) {
    uint32_t p[G / 2];
#pragma unroll
    for (int i = 0; i < G / 2; ++i) p[i] = bf16x2_rne(v[2 * i], v[2 * i + 1]);
    store_words<G / 2>(out, g, p);
  } else {
    float4* o = reinterpret_cast<float4*>(static_cast<float*>(out) + G * g);
#pragma unroll
    for (int i = 0; i < G / 4; ++i) o[i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
  }
}

template <bool BF16>
__device__ inline void dequant_one(int8_t code, int64_t idx, int64_t cols, const uint16_t* scales, void* out) {
  const float v = (float)code * f16_bits_to_float(scales[idx / cols]);
  if (BF16) static_cast<uint16_t*>(out)[idx] = (uint16_t)(bf16x2_rne(v, 0.0f) & 0xFFFF);
  else static_cast<float*>(out)[idx] = v;
}

// BITS 6 / 5: src holds packed codes; BITS 8: int8 codes.
template <int BITS, bool BF16, bool ROWG>
__global__ __launch_bounds__(kThreads) void dequant_kernel(const void* src, const uint16_t* scales, int64_t n,
                                                           int64_t cols, void* out) {
  using F = Fmt<BITS>;
  const int64_t ng = n / F::G;
  const int64_t gb = blockIdx.x * kGroupsPerBlock + threadIdx.x;
  uint32_t p[kU][F::PB / 4];
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    const int64_t g = gb + u * kThreads;
#pragma unroll
    for (int i = 0; i < F::PB / 4; ++i) p[u][i] = 0;
    if (g < ng) load_words<F::PB / 4>(src, g, p[u]);
  }
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    const int64_t g = gb + u * kThreads;
    if (g < ng) {
      if constexpr (BITS == 8) {
        dequant_group<F::G, BF16, ROWG>(p[u], g, cols, scales, out);
      } else {
        uint32_t c[F::G / 4];
        unpack_group(p[u], c);
        dequant_group<F::G, BF16, ROWG>(c, g, cols, scales, out);
      }
    } else if (g == ng && n % F::G) {
      for (int64_t idx0 = F::G * ng; idx0 < n; idx0 += F::WC) {
        uint64_t x;
        if constexpr (BITS == 8) {
          x = (uint64_t)(uint8_t) static_cast<const int8_t*>(src)[idx0];
        } else {
          const int64_t j = (idx0 - F::G * ng) / F::WC;
          x = unpack_word<BITS>(gather_packed<BITS>(static_cast<const uint8_t*>(src) + F::PB * ng + F::WB * j));
        }
        for (int b = 0; b < F::WC; ++b)
          if (idx0 + b < n) dequant_one<BF16>((int8_t)(x >> (8 * b)), idx0 + b, cols, scales, out);
      }
    }
  }
}

__global__ __launch_bounds__(256) void zero_parts_kernel(unsigned long long* parts) {
  parts[256 * blockIdx.x + threadIdx.x] = 0;
}

// out[b] (+)= sum of the partial histograms' bin b.
__global__ __launch_bounds__(256) void hist_finish_kernel(const unsigned long long* parts, int accumulate,
                                                          long long* out) {
  const int b = threadIdx.x;
  unsigned long long s = 0;
  for (int p = 0; p < kHistParts; ++p) s += parts[256 * p + b];
  out[b] = (accumulate ? out[b] : 0) + (long long)s;
}

// Histogram of int8 values.  Each wavefront counts into four LDS copies of
// the 256 bins (lane & 3 picks one), so that fewer lanes of one atomic
// instruction meet on one address; the copies start in different banks
// (257 words apart), and bin b sits at word (b >> 2) | (b & 3) << 6, so the
// int6 levels (every fourth value) fill 64 consecutive words instead of
// every fourth bank.  At the end each workgroup adds its counts to one of
// kHistParts partial histograms (blockIdx % kHistParts): device-scope
// atomics on one address are applied one after another, and a thousand
// workgroups adding into the same 256 bins queued for longer than the
// counting took; a one-workgroup kernel then sums the partial histograms.
constexpr int kCopies = 4 * (kThreads / kWave);
constexpr int kCopyWords = 256 + 1;
__device__ inline int hist_word(uint32_t b) { return (int)((b >> 2) | ((b & 3u) << 6)); }

__global__ __launch_bounds__(kThreads) void hist_kernel(const int8_t* codes, int64_t n,
                                                        unsigned long long* parts) {
  __shared__ uint32_t h[kCopies * kCopyWords];
  for (int i = threadIdx.x; i < kCopies * kCopyWords; i += kThreads) h[i] = 0;
  __syncthreads();
  uint32_t* hc = h + (4 * (threadIdx.x / kWave) + (threadIdx.x & 3)) * kCopyWords;
  const int64_t n16 = n >> 4;
  const int64_t gb = blockIdx.x * kGroupsPerBlock + threadIdx.x;
  uint4 x[kU];
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    const int64_t g = gb + u * kThreads;
    x[u] = g < n16 ? reinterpret_cast<const uint4*>(codes)[g] : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    const int64_t g = gb + u * kThreads;
    if (g < n16) {
      const uint32_t w[4] = {x[u].x, x[u].y, x[u].z, x[u].w};
#pragma unroll
      for (int i = 0; i < 16; ++i) atomicAdd(&hc[hist_word(((w[i >> 2] >> (8 * (i & 3))) & 0xFF) ^ 0x80)], 1u);
    } else if (g == n16 && (n & 15)) {
      for (int64_t idx = 16 * n16; idx < n; ++idx) atomicAdd(&hc[hist_word((uint8_t)codes[idx] ^ 0x80)], 1u);
    }
  }
  __syncthreads();
  unsigned long long* hist = parts + 256 * (blockIdx.x % kHistParts);
  for (int b = threadIdx.x; b < 256; b += kThreads) {
    uint32_t s = 0;
    for (int k = 0; k < kCopies; ++k) s += h[k * kCopyWords + hist_word(b)];
    if (s) atomicAdd(&hist[b], (unsigned long long)s);
  }
}

// Shannon entropy (bits per value) of a 256-bin histogram: -sum p log2 p
// over bins with a positive count, p = count / total; 0 for a zero total.
__global__ __launch_bounds__(256) void entropy_kernel(const int64_t* hist, double* out) {
  __shared__ double red[256];
  __shared__ long long tot[256];
  const int t = threadIdx.x;
  const long long h = hist[t];
  tot[t] = h;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (t < s) tot[t] += tot[t + s];
    __syncthreads();
  }
  const long long n = tot[0];
  double term = 0.0;
  if (h > 0 && n > 0) {
    const double p = (double)h / (double)n;
    term = -p * log2(p);
  }
  red[t] = term;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (t < s) red[t] += red[t + s];
    __syncthreads();
  }
  if (t == 0) *out = red[0];
}

// Workgroups covering the groups of G codes of n (a last partial group
// included).
inline unsigned grid_for(int64_t n, int G) {
  const int64_t groups = n / G + (n % G != 0);
  return (unsigned)((groups + kGroupsPerBlock - 1) / kGroupsPerBlock);
}

}  // namespace

hipError_t launch_pack_codes(const int8_t* codes, int64_t n, int bits, uint8_t* packed, int32_t* flags,
                             hipStream_t s) {
  if (bits == 6)
    hipLaunchKernelGGL(pack_kernel<6>, dim3(grid_for(n, 16)), dim3(kThreads), 0, s, codes, n, packed, flags);
  else
    hipLaunchKernelGGL(pack_kernel<5>, dim3(grid_for(n, 32)), dim3(kThreads), 0, s, codes, n, packed, flags);
  return hipGetLastError();
}

hipError_t launch_unpack_codes(const uint8_t* packed, int64_t n, int bits, int8_t* codes, hipStream_t s) {
  if (bits == 6)
    hipLaunchKernelGGL(unpack_kernel<6>, dim3(grid_for(n, 16)), dim3(kThreads), 0, s, packed, n, codes);
  else
    hipLaunchKernelGGL(unpack_kernel<5>, dim3(grid_for(n, 32)), dim3(kThreads), 0, s, packed, n, codes);
  return hipGetLastError();
}

hipError_t launch_dequantize(const void* src, int bits, const uint16_t* scales, int64_t rows, int64_t cols,
                             bool bf16_out, void* out, hipStream_t s) {
  const int64_t n = rows * cols;
  const int G = bits == 5 ? 32 : 16;
  const bool rowg = cols % G == 0 && n < (int64_t(1) << 32);
  const unsigned grid = grid_for(n, G);
#define I6G_DQ(B, O, R)                                                                                  \
  if (bits == B && bf16_out == O && rowg == R)                                                           \
    hipLaunchKernelGGL((dequant_kernel<B, O, R>), dim3(grid), dim3(kThreads), 0, s, src, scales, n, cols, out);
  I6G_DQ(8, true, true) I6G_DQ(8, true, false) I6G_DQ(8, false, true) I6G_DQ(8, false, false)
  I6G_DQ(6, true, true) I6G_DQ(6, true, false) I6G_DQ(6, false, true) I6G_DQ(6, false, false)
  I6G_DQ(5, true, true) I6G_DQ(5, true, false) I6G_DQ(5, false, true) I6G_DQ(5, false, false)
#undef I6G_DQ
  return hipGetLastError();
}

namespace {

// The three launches of a histogram into the given partial histograms
// (cleared by a kernel, not a memset, so the sequence can be captured).
hipError_t histogram_with_parts(const int8_t* codes, int64_t n, bool accumulate, int64_t* hist,
                                unsigned long long* parts, hipStream_t s) {
  hipLaunchKernelGGL(zero_parts_kernel, dim3(kHistParts), dim3(256), 0, s, parts);
  if (n > 0) hipLaunchKernelGGL(hist_kernel, dim3(grid_for(n, 16)), dim3(kThreads), 0, s, codes, n, parts);
  hipLaunchKernelGGL(hist_finish_kernel, dim3(1), dim3(256), 0, s, parts, (int)accumulate,
                     reinterpret_cast<long long*>(hist));
  return hipGetLastError();
}

}  // namespace

// Scratch of launch_code_histogram_noalloc: the kHistParts partial
// histograms (128 KiB).  Every device holds its own copy of this array for
// as long as the library stays loaded; host code reaches it only through the
// address hipGetSymbolAddress returns with that device current.
static __device__ __align__(256) unsigned long long scratch[256 * kHistParts];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
unsigned long long* g_scratch[kMaxDevices] = {};
}  // namespace

hipError_t launch_code_histogram(const int8_t* codes, int64_t n, bool accumulate, int64_t* hist, hipStream_t s) {
  // the partial histograms live in stream-ordered memory, so calls on
  // different streams never share them
  unsigned long long* parts = nullptr;
  hipError_t e = hipMallocAsync(reinterpret_cast<void**>(&parts), sizeof(unsigned long long) * 256 * kHistParts, s);
  if (e != hipSuccess) return e;
  e = histogram_with_parts(codes, n, accumulate, hist, parts, s);
  const hipError_t f = hipFreeAsync(parts, s);
  return e != hipSuccess ? e : f;
}

hipError_t code_histogram_scratch(unsigned long long** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch[dev] = static_cast<unsigned long long*>(p);
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

hipError_t launch_code_histogram_noalloc(const int8_t* codes, int64_t n, bool accumulate, int64_t* hist,
                                         hipStream_t s) {
  unsigned long long* parts = nullptr;
  hipError_t e = code_histogram_scratch(&parts);
  if (e != hipSuccess) return e;
  return histogram_with_parts(codes, n, accumulate, hist, parts, s);
}

int64_t code_histogram_max_codes() {
  // hist_kernel's workgroups: one per kGroupsPerBlock groups of 16 codes,
  // at most 2^31 - 1 of them in one launch
  return (int64_t)INT32_MAX * kGroupsPerBlock * 16;
}

hipError_t launch_code_entropy(const int64_t* hist, double* out, hipStream_t s) {
  hipLaunchKernelGGL(entropy_kernel, dim3(1), dim3(256), 0, s, hist, out);
  return hipGetLastError();
}

}  // namespace i6g
