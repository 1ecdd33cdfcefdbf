// Comparison packings of the same ternary matrix, for measuring the pages'
// central claim on this GPU: padded 2-bit, and three weights in 5 bits (the
// 1.67-bit width the pages time as "TL2") -- "Sherry: Hardware-Efficient
// 1.25-Bit Ternary Quantization via Fine-grained Sparsification", agihunt
// digest, problem paragraph and results table.
//
// Layouts (this implementation's readings; the pages give none):
//   2-bit   value 0 / +1 / -1 -> code 0 / 1 / 2.  Superblocks of 128 weights;
//           the 32-byte record of (superblock g, row n) sits at (g*N + n)*32
//           and byte j holds the 4 weights of block j, weight i in bits 2i.
//   3-in-5  digits d = v + 1; the triple code d0 + 3 d1 + 9 d2 (0..26) takes
//           5 bits.  Superblocks of 192 weights (64 triples), K zero-padded to
//           a multiple of 192; the 40-byte record of (superblock g, row n)
//           sits at (g*N + n)*40 and holds code t in bits [5t, 5t+5).
//
// Both GEMV kernels follow the batch-1 Sherry kernel's plan -- per workgroup
// and window, tables of partial sums built from the activations in LDS, then
// one lookup per code -- so the three formats differ in what they must:
// bytes per weight (0.156 / 0.208+ / 0.25) and lookups per weight (1/4, 1/3,
// 1/2: a 2-bit pair is a 4-bit index into a 16-entry table, a triple a 5-bit
// index into a 32-entry table).  Scales are per output channel for all three
// (a triple can straddle a 128-weight group), applied once at the end.
#include "sherry_internal.h"

namespace sherry {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr int kSb2 = 128, kSb3 = 192;
constexpr int kWin2 = 4;  // 2-bit superblocks per table window: 256 pairs x 16 floats = 16 KB
constexpr int kWin3 = 2;  // 3-in-5 superblocks per window: 128 triples x 32 floats = 16 KB

__device__ inline float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

template <typename T>
__device__ inline T nt_load(const T* p) {
  return __builtin_nontemporal_load(p);
}

__device__ inline uint32_t code2(int v) { return v == 0 ? 0u : (v > 0 ? 1u : 2u); }

// ternary value of weight col of row (0 past k) from the Sherry planes
__device__ inline int sherry_weight(const uint8_t* __restrict__ packed, int64_t n, int64_t k, int64_t row,
                                    int64_t col) {
  if (col >= k) return 0;
  int t[4];
  decode_block(load_code(packed, n, k, row, col >> 2), t);
  return t[col & 3];
}

// one thread per (superblock, row) record
__global__ void repack_2bit_kernel(const uint8_t* __restrict__ packed, uint8_t* __restrict__ out, int64_t n,
                                   int64_t k) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t nsb = k / kSb2;
  if (idx >= nsb * n) return;
  const int64_t g = idx / n, row = idx % n;
  uint32_t w[8];
#pragma unroll
  for (int d = 0; d < 8; ++d) {
    uint32_t v = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      int t[4];
      decode_block(load_code(packed, n, k, row, g * 32 + d * 4 + b), t);
      const uint32_t byte = code2(t[0]) | (code2(t[1]) << 2) | (code2(t[2]) << 4) | (code2(t[3]) << 6);
      v |= byte << (8 * b);
    }
    w[d] = v;
  }
  u32x4* dst = reinterpret_cast<u32x4*>(out + (g * n + row) * 32);
  dst[0] = u32x4{w[0], w[1], w[2], w[3]};
  dst[1] = u32x4{w[4], w[5], w[6], w[7]};
}

__global__ void repack_tl2_kernel(const uint8_t* __restrict__ packed, uint8_t* __restrict__ out, int64_t n,
                                  int64_t k) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t nsb = (k + kSb3 - 1) / kSb3;
  if (idx >= nsb * n) return;
  const int64_t g = idx / n, row = idx % n;
  uint32_t w[10] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
  for (int tri = 0; tri < 64; ++tri) {
    const int64_t col = g * kSb3 + 3 * tri;
    const uint32_t code = (uint32_t)(sherry_weight(packed, n, k, row, col) + 1) +
                          3u * (uint32_t)(sherry_weight(packed, n, k, row, col + 1) + 1) +
                          9u * (uint32_t)(sherry_weight(packed, n, k, row, col + 2) + 1);
    const int bit = 5 * tri, d = bit >> 5, s = bit & 31;
    w[d] |= code << s;
    if (s > 27) w[d + 1] |= code >> (32 - s);
  }
  u32x2* dst = reinterpret_cast<u32x2*>(out + (g * n + row) * 40);
#pragma unroll
  for (int i = 0; i < 5; ++i) dst[i] = u32x2{w[2 * i], w[2 * i + 1]};
}

// Entries [16 H, 16 H + 16) of a triple's table: code = d0 + 3 d1 + 9 d2,
// value (v(d0) + v(d1)) + v(d2) with v(d) = (d - 1) x_i, from the nine sums
// of the first two digits (every index below is a compile-time constant).
template <int H>
__device__ inline void tl2_table_half(float* t, const float xs[3]) {
  const float a[3] = {-xs[0], 0.f, xs[0]}, b[3] = {-xs[1], 0.f, xs[1]}, c[3] = {-xs[2], 0.f, xs[2]};
  float p[9];
#pragma unroll
  for (int i = 0; i < 9; ++i) p[i] = a[i % 3] + b[i / 3];
  float e[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int code = 16 * H + j;
    e[j] = code < 27 ? p[code % 9] + c[code / 9] : 0.f;
  }
  float4* d = reinterpret_cast<float4*>(t);
#pragma unroll
  for (int q = 0; q < 4; ++q) d[q] = make_float4(e[4 * q], e[4 * q + 1], e[4 * q + 2], e[4 * q + 3]);
}

template <bool YBF16>
__device__ inline void store_out(void* y, int64_t i, float v) {
  if constexpr (YBF16) {
    reinterpret_cast<uint16_t*>(y)[i] = f32_to_bf16_rne(v);
  } else {
    reinterpret_cast<float*>(y)[i] = v;
  }
}

// Batch-1 GEMV over 2-bit planes.  Table of pair p: entry e = v(e & 3) x[2p]
// + v(e >> 2) x[2p+1], v = (0, +1, -1, 0).  TH threads (one row each) share
// the tables: 256, or 512 on launches with workgroups to spare (as the
// Sherry kernel's 512-row panels).
template <int TH>
__global__ __launch_bounds__(TH) void gemv_2bit_kernel(const uint8_t* __restrict__ planes,
                                                             const float* __restrict__ alpha,
                                                             const uint16_t* __restrict__ x,
                                                             uint16_t* __restrict__ y, int64_t n, int64_t k,
                                                             int64_t planes_stride, int64_t alpha_stride,
                                                             int64_t y_stride) {
  __shared__ __attribute__((aligned(16))) float tbl[kWin2 * 64 * 16];
  const int tid = threadIdx.x;
  const int64_t c = blockIdx.y;
  const uint8_t* pl = planes + c * planes_stride;
  const int64_t row = (int64_t)blockIdx.x * TH + tid;
  const uint32_t rr = (uint32_t)(row < n ? row : n - 1);  // clamped rows are not stored
  const int64_t nsb = k / kSb2;
  float acc = 0.f;
  for (int64_t g0 = 0; g0 < nsb; g0 += kWin2) {
    const int wn = (int)(nsb - g0 < kWin2 ? nsb - g0 : kWin2);
    __syncthreads();
    {
      // thread tid builds pair tid of the window (256 pairs = 4 superblocks)
      if (tid < kWin2 * 64) {
        const int64_t kk = g0 * kSb2 + 2 * tid;
        float x0 = 0.f, x1 = 0.f;
        if (tid < wn * 64) {
          const uint32_t xv = *reinterpret_cast<const uint32_t*>(x + kk);
          x0 = bf16_to_f32((uint16_t)(xv & 0xFFFF));
          x1 = bf16_to_f32((uint16_t)(xv >> 16));
        }
        const float v0[4] = {0.f, x0, -x0, 0.f};
        const float v1[4] = {0.f, x1, -x1, 0.f};
        float* t = tbl + tid * 16;
#pragma unroll
        for (int e = 0; e < 16; ++e) t[e] = v0[e & 3] + v1[e >> 2];
      }
    }
    __syncthreads();
    u32x4 rec[kWin2][2];
#pragma unroll
    for (int gi = 0; gi < kWin2; ++gi) {
      const int64_t g = g0 + (gi < wn ? gi : 0);
      const u32x4* src = reinterpret_cast<const u32x4*>(pl + (g * n + rr) * 32);
      rec[gi][0] = nt_load(src);
      rec[gi][1] = nt_load(src + 1);
    }
    const char* tb = reinterpret_cast<const char*>(tbl);
#pragma unroll
    for (int gi = 0; gi < kWin2; ++gi) {
      if (gi >= wn) break;
      float s[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        const uint32_t w = rec[gi][d >> 2][d & 3];
#pragma unroll
        for (int h = 0; h < 8; ++h) {
          const int p = gi * 64 + d * 8 + h;  // pair index in the window
          const uint32_t off = h == 0 ? (w << 2) & 0x3Cu : (w >> (4 * h - 2)) & 0x3Cu;
          s[h & 3] += *reinterpret_cast<const float*>(tb + p * 64 + off);
        }
      }
      acc += (s[0] + s[1]) + (s[2] + s[3]);
    }
  }
  if (row < n) store_out<true>(y + c * y_stride, row, acc * alpha[c * alpha_stride + row]);
}

// Batch-1 GEMV over 3-in-5 planes.  Table of triple t: entry code =
// sum_i (digit_i(code) - 1) x[3t + i] (entries 27..31 unused), built with
// adds of +-x / 0 only (with the digit products computed from the code at run
// time the build took 75 VGPRs and ran the layer pass 14% slower).  TH
// threads as in the 2-bit kernel.
template <int TH>
__global__ __launch_bounds__(TH) void gemv_tl2_kernel(const uint8_t* __restrict__ planes,
                                                            const float* __restrict__ alpha,
                                                            const uint16_t* __restrict__ x,
                                                            uint16_t* __restrict__ y, int64_t n, int64_t k,
                                                            int64_t planes_stride, int64_t alpha_stride,
                                                            int64_t y_stride) {
  __shared__ __attribute__((aligned(16))) float tbl[kWin3 * 64 * 32];
  const int tid = threadIdx.x;
  const int64_t c = blockIdx.y;
  const uint8_t* pl = planes + c * planes_stride;
  const int64_t row = (int64_t)blockIdx.x * TH + tid;
  const uint32_t rr = (uint32_t)(row < n ? row : n - 1);
  const int64_t nsb = (k + kSb3 - 1) / kSb3;
  float acc = 0.f;
  for (int64_t g0 = 0; g0 < nsb; g0 += kWin3) {
    const int wn = (int)(nsb - g0 < kWin3 ? nsb - g0 : kWin3);
    __syncthreads();
    if (tid < kWin3 * 64 * 2) {
      // thread tid builds half tid & 1 of triple tid >> 1 (128 triples = 2 superblocks)
      const int tri = tid >> 1, half = tid & 1;
      float xs[3];
#pragma unroll
      for (int i = 0; i < 3; ++i) {
        const int64_t kk = g0 * kSb3 + 3 * tri + i;
        xs[i] = (tri < wn * 64 && kk < k) ? bf16_to_f32(x[kk]) : 0.f;
      }
      float* t = tbl + tri * 32 + half * 16;
      if (half == 0) tl2_table_half<0>(t, xs);
      else tl2_table_half<1>(t, xs);
    }
    __syncthreads();
    // both superblocks' records at once: their 8-byte loads share cache lines
    // (loaded one superblock at a time, 5% more bytes were fetched)
    uint32_t rec[kWin3][10];
#pragma unroll
    for (int gi = 0; gi < kWin3; ++gi) {
      const int64_t g = g0 + (gi < wn ? gi : 0);
      const u32x2* src = reinterpret_cast<const u32x2*>(pl + (g * n + rr) * 40);
#pragma unroll
      for (int i = 0; i < 5; ++i) {
        const u32x2 v = nt_load(src + i);
        rec[gi][2 * i] = v[0];
        rec[gi][2 * i + 1] = v[1];
      }
    }
    const char* tb = reinterpret_cast<const char*>(tbl);
#pragma unroll
    for (int gi = 0; gi < kWin3; ++gi) {
      if (gi >= wn) break;
      float s[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < 64; ++t) {
        const int bit = 5 * t, d = bit >> 5, sh = bit & 31;
        uint32_t code;
        if (sh <= 27) {
          code = __builtin_amdgcn_ubfe(rec[gi][d], sh, 5);
        } else {
          code = __builtin_amdgcn_alignbit(rec[gi][d + 1], rec[gi][d], sh) & 31u;
        }
        s[t & 3] += *reinterpret_cast<const float*>(tb + (gi * 64 + t) * 128 + code * 4);
      }
      acc += (s[0] + s[1]) + (s[2] + s[3]);
    }
  }
  if (row < n) store_out<true>(y + c * y_stride, row, acc * alpha[c * alpha_stride + row]);
}

}  // namespace

int64_t compare_k_padded(int fmt, int64_t k) {
  const int64_t sb = fmt == 0 ? kSb2 : kSb3;
  return (k + sb - 1) / sb * sb;
}

size_t compare_bytes(int fmt, int64_t n, int64_t k) {
  if (fmt == 0) return (size_t)(n * compare_k_padded(fmt, k) / 4);
  return (size_t)(n * (compare_k_padded(fmt, k) / kSb3) * 40);
}

hipError_t launch_compare_repack(int fmt, int64_t n, int64_t k, const uint8_t* packed, uint8_t* out,
                                 hipStream_t s) {
  const int64_t items = (fmt == 0 ? k / kSb2 : compare_k_padded(fmt, k) / kSb3) * n;
  const dim3 grid((unsigned)((items + 255) / 256));
  if (fmt == 0) {
    hipLaunchKernelGGL(repack_2bit_kernel, grid, dim3(256), 0, s, packed, out, n, k);
  } else {
    hipLaunchKernelGGL(repack_tl2_kernel, grid, dim3(256), 0, s, packed, out, n, k);
  }
  return hipGetLastError();
}

hipError_t launch_compare_gemv(int fmt, int64_t n, int64_t k, const uint8_t* planes, const float* alpha,
                               const uint16_t* x, uint16_t* y, int count, int64_t planes_stride,
                               int64_t alpha_stride, int64_t y_stride, hipStream_t s) {
  // 2-bit: 512-row workgroups where the launch still has >= 2048 of them
  // (1-2% faster); the 3-in-5 kernel keeps 256 (with 512, its 40-byte
  // records fetched 4.6% more than their bytes and the pass ran 1% slower)
  const bool wide = fmt == 0 && (n + 511) / 512 * 512 * 8 <= n * 9 && (n + 511) / 512 * count >= 2048;
  const int th = wide ? 512 : kThreads;
  const dim3 grid((unsigned)((n + th - 1) / th), (unsigned)count);
#define SHERRY_CMP(KER)                                                                                        \
  if (wide) hipLaunchKernelGGL(KER<512>, grid, dim3(512), 0, s, planes, alpha, x, y, n, k, planes_stride,       \
                               alpha_stride, y_stride);                                                       \
  else hipLaunchKernelGGL(KER<kThreads>, grid, dim3(kThreads), 0, s, planes, alpha, x, y, n, k, planes_stride, \
                          alpha_stride, y_stride);
  if (fmt == 0) {
    SHERRY_CMP(gemv_2bit_kernel)
  } else {
    SHERRY_CMP(gemv_tl2_kernel)
  }
#undef SHERRY_CMP
  return hipGetLastError();
}

}  // namespace sherry
