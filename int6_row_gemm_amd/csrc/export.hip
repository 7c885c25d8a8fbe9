// Export side of the int6 format: 6-bit packing, unpacking, dequantisation
// and code statistics.
//
// kwkr.cn write-up of parameter-golf PR #363, timeline and run notes: the
// int6 codes are measured by their entropy (bits per value) and compressed
// (bit packing among the methods tried) into an artifact of at most
// 16,000,000 bytes, which is dequantised and evaluated again.  pwwt.cn
// "parameter-golf 16MB 极限压缩实战 …", 后训练量化导出: codes are int8
// multiples of 4 in [-128, 124] with one binary16 scale per row.
//
// Packed format: code c -> u = c/4 + 32 in [0, 63]; four codes u0..u3 make
// the 24-bit word u0 | u1 << 6 | u2 << 12 | u3 << 18, stored as 3 bytes,
// least significant first; a tail of fewer than four codes is padded with
// code 0.
//
// All kernels are bound by HBM traffic.  A thread moves 16 codes (one 16-byte
// load or store of codes, 12 bytes of packed data) per group and each thread
// issues its kU groups' loads before using any, so that enough bytes are in
// flight to cover HBM latency.  The last, partial group of a buffer is done
// by the thread whose group index is the group count.
#include "common.h"

namespace i6g {
namespace {

constexpr int kU = 2;           // groups per thread
constexpr int kThreads = 256;   // threads per workgroup
constexpr int64_t kGroupsPerBlock = (int64_t)kU * kThreads;
constexpr int kHistParts = 64;  // partial histograms (see hist_kernel)

// Four codes, one per byte of x, -> their 24-bit packed word.  For a code
// c = 4t (t in [-32, 31]) bits 2..7 of the byte are t in 6-bit two's
// complement, and t + 32 mod 64 flips its top bit.
__device__ inline uint32_t pack4(uint32_t x) {
  const uint32_t y = ((x >> 2) & 0x3F3F3F3Fu) ^ 0x20202020u;
  return (y & 0x3Fu) | ((y >> 2) & 0xFC0u) | ((y >> 4) & 0x3F000u) | ((y >> 6) & 0xFC0000u);
}

// The inverse: a 24-bit packed word -> four codes, one per byte.
__device__ inline uint32_t unpack4(uint32_t w) {
  const uint32_t y = (w & 0x3Fu) | ((w << 2) & 0x3F00u) | ((w << 4) & 0x3F0000u) | ((w << 6) & 0x3F000000u);
  return (y ^ 0x20202020u) << 2;
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

// Codes of a partial last group (idx0 .. n-1, fewer than 16), padded with 0.
__device__ inline uint32_t tail_word(const int8_t* codes, int64_t idx0, int64_t n, int& bad) {
  uint32_t x = 0;
  for (int b = 0; b < 4; ++b) {
    if (idx0 + b < n) {
      const uint32_t byte = (uint8_t)codes[idx0 + b];
      bad |= (byte & 3u) != 0;
      x |= byte << (8 * b);
    }
  }
  return x;
}

__device__ inline uint32_t load_packed_word(const uint8_t* p) {
  return (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16);
}

__global__ __launch_bounds__(kThreads) void pack_kernel(const int8_t* codes, int64_t n, uint8_t* packed,
                                                        int32_t* flags) {
  const int64_t n16 = n >> 4;
  const int64_t gb = blockIdx.x * kGroupsPerBlock + threadIdx.x;
  int bad = 0;
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
      bad |= ((x[u].x | x[u].y | x[u].z | x[u].w) & 0x03030303u) != 0;
      const uint32_t w0 = pack4(x[u].x), w1 = pack4(x[u].y), w2 = pack4(x[u].z), w3 = pack4(x[u].w);
      uint32_t* o = reinterpret_cast<uint32_t*>(packed + 12 * g);
      o[0] = w0 | (w1 << 24);
      o[1] = (w1 >> 8) | (w2 << 16);
      o[2] = (w2 >> 16) | (w3 << 8);
    } else if (g == n16 && (n & 15)) {
      for (int64_t j = 0; 16 * n16 + 4 * j < n; ++j) {
        const uint32_t w = pack4(tail_word(codes, 16 * n16 + 4 * j, n, bad));
        uint8_t* o = packed + 12 * n16 + 3 * j;
        o[0] = w & 0xFF;
        o[1] = (w >> 8) & 0xFF;
        o[2] = w >> 16;
      }
    }
  }
  if (bad && flags) atomicOr(flags, kFlagCode);
}

__global__ __launch_bounds__(kThreads) void unpack_kernel(const uint8_t* packed, int64_t n, int8_t* codes) {
  const int64_t n16 = n >> 4;
  const int64_t gb = blockIdx.x * kGroupsPerBlock + threadIdx.x;
  uint32_t d[kU][3];
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    const int64_t g = gb + u * kThreads;
    d[u][0] = d[u][1] = d[u][2] = 0;
    if (g < n16) {
      const uint32_t* p = reinterpret_cast<const uint32_t*>(packed + 12 * g);
      d[u][0] = p[0]; d[u][1] = p[1]; d[u][2] = p[2];
    }
  }
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    const int64_t g = gb + u * kThreads;
    if (g < n16) {
      uint4 x;
      x.x = unpack4(d[u][0] & 0xFFFFFFu);
      x.y = unpack4((d[u][0] >> 24) | ((d[u][1] & 0xFFFFu) << 8));
      x.z = unpack4((d[u][1] >> 16) | ((d[u][2] & 0xFFu) << 16));
      x.w = unpack4(d[u][2] >> 8);
      reinterpret_cast<uint4*>(codes)[g] = x;
    } else if (g == n16 && (n & 15)) {
      for (int64_t j = 0; 16 * n16 + 4 * j < n; ++j) {
        const uint32_t x = unpack4(load_packed_word(packed + 12 * n16 + 3 * j));
        for (int b = 0; b < 4; ++b) {
          const int64_t idx = 16 * n16 + 4 * j + b;
          if (idx < n) codes[idx] = (int8_t)((x >> (8 * b)) & 0xFF);
        }
      }
    }
  }
}

// out[i] = code[i] * scale[i / cols] for the 16 codes of group g (four per
// word of x), written as fp32 or bfloat16.  ROW16: cols is a multiple of 16,
// so the whole group lies in one row, and rows * cols < 2^32.
template <bool BF16, bool ROW16>
__device__ inline void dequant_group(const uint32_t (&x)[4], int64_t g, int64_t cols, const uint16_t* scales,
                                     void* out) {
  float v[16];
  if (ROW16) {
    // every index fits 32 bits (checked on the host), and 32-bit division
    // is a few instructions where 64-bit division is a long sequence
    const float s = f16_bits_to_float(scales[(uint32_t)(16 * g) / (uint32_t)cols]);
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = (float)(int8_t)((x[i >> 2] >> (8 * (i & 3))) & 0xFF) * s;
  } else {
    int64_t r = (16 * g) / cols, c = 16 * g - r * cols;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      while (c >= cols) { c -= cols; ++r; }
      v[i] = (float)(int8_t)((x[i >> 2] >> (8 * (i & 3))) & 0xFF) * f16_bits_to_float(scales[r]);
      ++c;
    }
  }
  if (BF16) {
    uint4* o = reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + 16 * g);
    uint32_t p[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) p[i] = bf16x2_rne(v[2 * i], v[2 * i + 1]);
    o[0] = make_uint4(p[0], p[1], p[2], p[3]);
    o[1] = make_uint4(p[4], p[5], p[6], p[7]);
  } else {
    float4* o = reinterpret_cast<float4*>(static_cast<float*>(out) + 16 * g);
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
  }
}

template <bool BF16>
__device__ inline void dequant_one(int8_t code, int64_t idx, int64_t cols, const uint16_t* scales, void* out) {
  const float v = (float)code * f16_bits_to_float(scales[idx / cols]);
  if (BF16) static_cast<uint16_t*>(out)[idx] = (uint16_t)(bf16x2_rne(v, 0.0f) & 0xFFFF);
  else static_cast<float*>(out)[idx] = v;
}

// PACKED: src holds the packed bytes, else int8 codes.
template <bool PACKED, bool BF16, bool ROW16>
__global__ __launch_bounds__(kThreads) void dequant_kernel(const void* src, const uint16_t* scales, int64_t n,
                                                           int64_t cols, void* out) {
  const int64_t n16 = n >> 4;
  const int64_t gb = blockIdx.x * kGroupsPerBlock + threadIdx.x;
  uint32_t x[kU][4];
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    const int64_t g = gb + u * kThreads;
    x[u][0] = x[u][1] = x[u][2] = x[u][3] = 0;
    if (g < n16) {
      if (PACKED) {
        const uint32_t* p = reinterpret_cast<const uint32_t*>(static_cast<const uint8_t*>(src) + 12 * g);
        x[u][0] = p[0]; x[u][1] = p[1]; x[u][2] = p[2];
      } else {
        const uint4 c = reinterpret_cast<const uint4*>(src)[g];
        x[u][0] = c.x; x[u][1] = c.y; x[u][2] = c.z; x[u][3] = c.w;
      }
    }
  }
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    const int64_t g = gb + u * kThreads;
    if (g < n16) {
      if (PACKED) {
        const uint32_t d0 = x[u][0], d1 = x[u][1], d2 = x[u][2];
        x[u][0] = unpack4(d0 & 0xFFFFFFu);
        x[u][1] = unpack4((d0 >> 24) | ((d1 & 0xFFFFu) << 8));
        x[u][2] = unpack4((d1 >> 16) | ((d2 & 0xFFu) << 16));
        x[u][3] = unpack4(d2 >> 8);
      }
      dequant_group<BF16, ROW16>(x[u], g, cols, scales, out);
    } else if (g == n16 && (n & 15)) {
      for (int64_t j = 0; 16 * n16 + 4 * j < n; ++j) {
        uint32_t w;
        if (PACKED) {
          w = unpack4(load_packed_word(static_cast<const uint8_t*>(src) + 12 * n16 + 3 * j));
        } else {
          int unused = 0;
          w = tail_word(static_cast<const int8_t*>(src), 16 * n16 + 4 * j, n, unused);
        }
        for (int b = 0; b < 4; ++b) {
          const int64_t idx = 16 * n16 + 4 * j + b;
          if (idx < n) dequant_one<BF16>((int8_t)((w >> (8 * b)) & 0xFF), idx, cols, scales, out);
        }
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

inline unsigned grid_for(int64_t n) {
  const int64_t groups = (n >> 4) + ((n & 15) != 0);
  return (unsigned)((groups + kGroupsPerBlock - 1) / kGroupsPerBlock);
}

}  // namespace

hipError_t launch_pack_int6(const int8_t* codes, int64_t n, uint8_t* packed, int32_t* flags, hipStream_t s) {
  hipLaunchKernelGGL(pack_kernel, dim3(grid_for(n)), dim3(kThreads), 0, s, codes, n, packed, flags);
  return hipGetLastError();
}

hipError_t launch_unpack_int6(const uint8_t* packed, int64_t n, int8_t* codes, hipStream_t s) {
  hipLaunchKernelGGL(unpack_kernel, dim3(grid_for(n)), dim3(kThreads), 0, s, packed, n, codes);
  return hipGetLastError();
}

hipError_t launch_dequantize(const void* src, bool packed, const uint16_t* scales, int64_t rows, int64_t cols,
                             bool bf16_out, void* out, hipStream_t s) {
  const int64_t n = rows * cols;
  const bool row16 = cols % 16 == 0 && n < (int64_t(1) << 32);
#define I6G_DQ(P, B, R)                                                                               \
  if (packed == P && bf16_out == B && row16 == R)                                                     \
    hipLaunchKernelGGL((dequant_kernel<P, B, R>), dim3(grid_for(n)), dim3(kThreads), 0, s, src, scales, \
                       n, cols, out);
  I6G_DQ(true, true, true) I6G_DQ(true, true, false) I6G_DQ(true, false, true) I6G_DQ(true, false, false)
  I6G_DQ(false, true, true) I6G_DQ(false, true, false) I6G_DQ(false, false, true) I6G_DQ(false, false, false)
#undef I6G_DQ
  return hipGetLastError();
}

hipError_t launch_code_histogram(const int8_t* codes, int64_t n, bool accumulate, int64_t* hist, hipStream_t s) {
  // the partial histograms live in stream-ordered memory, so calls on
  // different streams never share them
  unsigned long long* parts = nullptr;
  hipError_t e = hipMallocAsync(reinterpret_cast<void**>(&parts), sizeof(unsigned long long) * 256 * kHistParts, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(zero_parts_kernel, dim3(kHistParts), dim3(256), 0, s, parts);
  if (n > 0) hipLaunchKernelGGL(hist_kernel, dim3(grid_for(n)), dim3(kThreads), 0, s, codes, n, parts);
  hipLaunchKernelGGL(hist_finish_kernel, dim3(1), dim3(256), 0, s, parts, (int)accumulate,
                     reinterpret_cast<long long*>(hist));
  e = hipGetLastError();
  const hipError_t f = hipFreeAsync(parts, s);
  return e != hipSuccess ? e : f;
}

hipError_t launch_code_entropy(const int64_t* hist, double* out, hipStream_t s) {
  hipLaunchKernelGGL(entropy_kernel, dim3(1), dim3(256), 0, s, hist, out);
  return hipGetLastError();
}

}  // namespace i6g
