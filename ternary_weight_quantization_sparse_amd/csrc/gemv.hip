// Decode-time product y[b, n] = sum_k x[b, k] * T[n, k] * alpha(n, k).
//
// Method: "Sherry, Tequila and Fairies in Python", section 1.1 (SherryLinear
// runs F.linear with the quantized weight) and the agihunt digest, inference
// paragraph (weights packed offline as index + sign; tables built from the
// activations online; accumulate; apply the scale).  The pages' kernel is an
// x86 AVX2 byte-shuffle table; here the same idea is mapped to a CDNA4
// workgroup.
//
// Batch 1 (gemv_b1_lut_kernel): HBM-bound streaming.  Each workgroup builds,
// in LDS, a 32-entry fp32 table per block of 4 activations: the signed sum of
// the three kept activations for every code (sign bit folded in).  Each lane
// owns one weight row; per superblock it reads 16 bytes of nibbles (dwordx4)
// and one sign dword, turns 4 blocks at a time into 4 byte offsets with 4
// VALU ops (a nibble shift, a sign shift, a mask and an and-or), and then per
// block does one byte extract, one ds_read_b32 and one fp32 add.  All 64 lanes
// of a wave read the same block's 128-byte table, which spans the 32 LDS
// banks once, so the lookups are conflict-free (equal entries broadcast).
// The scale is applied once per group in fp32.
//
// Batch 2..16 (gemv_mfma_kernel): the contraction is no longer HBM-bound on
// VALU (batch x 3 adds per block), so blocks are decoded to bf16 and fed to
// v_mfma_f32_16x16x32_bf16 with the batch as the M dimension.  Decode: the
// same 4-block byte offsets index a 128-byte LDS table whose 32 dword entries
// hold the high bytes of the four bf16 weights (+-0.5 or 0, so the low bytes
// are 0 and the result is rescaled by 2, exactly); two v_perm_b32 spread a
// dword into the two bf16x2 operand registers.
#include <type_traits>

#include "sherry_internal.h"

namespace sherry {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kLutThreads = 256;
#ifndef SHERRY_GEMV_SPLIT_TARGET
#define SHERRY_GEMV_SPLIT_TARGET 2048
#endif
#ifndef SHERRY_LUT_WIN_MAX
#define SHERRY_LUT_WIN_MAX 4  // superblocks per LDS table window (4 -> 16 KB)
#endif
#ifndef SHERRY_LUT_NT
#define SHERRY_LUT_NT 1       // non-temporal loads for the packed stream
#endif
#ifndef SHERRY_LUT_ROWS
#define SHERRY_LUT_ROWS 1     // row slots per thread on large launches
#endif
constexpr int kTableFloatsPerSb = kBlocksPerSb * 32;  // 32 entries per block

// The 4 byte offsets (entry*4 into a block's 32-entry fp32 table, or into the
// 128-byte decode table) of the blocks in quad q of a superblock record.
// Quad q = 2d + h holds blocks q + 8b (b = 0..3): nibble dword d, nibble half
// h, and sign bits q + 8b, which a shift moves to bit 6 of byte b.
__device__ inline uint32_t quad_offsets(uint32_t nib_dword, uint32_t sign_word, int q) {
  const uint32_t nq = (q & 1) ? (nib_dword >> 2) : (nib_dword << 2);
  const uint32_t sq = ((q <= 6) ? (sign_word << (6 - q)) : (sign_word >> 1)) & 0x40404040u;
  // (nq & 0x3C3C3C3C) | sq as one 3-input bit operation
  return __builtin_amdgcn_bitop3_b32(nq, sq, 0x3C3C3C3Cu, 0xEC);
}

// Table of one block of 4 activations, half h: entries for zero positions
// z = 2h, 2h+1 with both sign bits.  Entry index = s<<4 | z<<2 | p1<<1 | p0;
// value = (x_k0 +- x_k1) +- x_k2 over the kept positions k0 < k1 < k2 (all
// but z), negated when s = 1.  Writes entries [8h, 8h+8) and [16+8h, 24+8h).
__device__ inline void build_block_half(float* blk_tbl, const uint16_t* __restrict__ xblk, int h) {
  const uint2 xv = *reinterpret_cast<const uint2*>(xblk);
  const float xs[4] = {__uint_as_float(xv.x << 16), __uint_as_float(xv.x & 0xFFFF0000u),
                       __uint_as_float(xv.y << 16), __uint_as_float(xv.y & 0xFFFF0000u)};
  float e[8];
#pragma unroll
  for (int zz = 0; zz < 2; ++zz) {
    const int z = 2 * h + zz;
    const float a = xs[z == 0 ? 1 : 0];
    const float b = xs[z <= 1 ? 2 : 1];
    const float c = xs[z <= 2 ? 3 : 2];
    const float apb = a + b, amb = a - b;
    e[4 * zz + 0] = apb + c;
    e[4 * zz + 1] = amb + c;
    e[4 * zz + 2] = apb - c;
    e[4 * zz + 3] = amb - c;
  }
  float4* pos = reinterpret_cast<float4*>(blk_tbl + 8 * h);
  float4* neg = reinterpret_cast<float4*>(blk_tbl + 16 + 8 * h);
  pos[0] = make_float4(e[0], e[1], e[2], e[3]);
  pos[1] = make_float4(e[4], e[5], e[6], e[7]);
  neg[0] = make_float4(-e[0], -e[1], -e[2], -e[3]);
  neg[1] = make_float4(-e[4], -e[5], -e[6], -e[7]);
}

template <bool BF16>
__device__ inline void store_y(void* y, int64_t idx, float v) {
  if constexpr (BF16) {
    reinterpret_cast<uint16_t*>(y)[idx] = f32_to_bf16_rne(v);
  } else {
    reinterpret_cast<float*>(y)[idx] = v;
  }
}

// Scale handling of the batch-1 kernel.
enum LutMode { kGroup1 = 0, kGroupN = 1, kChannel = 2, kTensor = 3 };

// The packed data of one row over one window of WIN superblocks.
template <int MODE, int WIN>
struct RowWindow {
  uint4 nb[WIN];
  uint32_t sg[WIN];
  float al[(MODE == kGroup1 || MODE == kGroupN) ? WIN : 1];
};

// Packed weights and scales are read once per launch: streaming loads.
template <typename T>
__device__ inline T stream_load(const T* p) {
#if SHERRY_LUT_NT
  return __builtin_nontemporal_load(p);
#else
  return *p;
#endif
}

// Loads of one row-window.  The per-superblock bases are wave-uniform (SGPR)
// and the per-lane part is a 32-bit byte offset, so every load is a
// saddr + voffset global load.
template <int MODE, int WIN>
__device__ inline void load_row_window(RowWindow<MODE, WIN>& r, const uint8_t* __restrict__ nib_base,
                                       const uint8_t* __restrict__ sgn_base, const float* __restrict__ al,
                                       int64_t n, uint32_t row, int64_t g0, int group_sbs) {
#pragma unroll
  for (int gi = 0; gi < WIN; ++gi) {
    const int64_t g = g0 + gi;
    const u32x4 v = stream_load(reinterpret_cast<const u32x4*>(nib_base + g * n * 16 + row * 16u));
    r.nb[gi] = make_uint4(v[0], v[1], v[2], v[3]);
    r.sg[gi] = stream_load(reinterpret_cast<const uint32_t*>(sgn_base + g * n * 4 + row * 4u));
    if constexpr (MODE == kGroup1) r.al[gi] = stream_load(al + g * n + row);
    if constexpr (MODE == kGroupN) r.al[gi] = stream_load(al + (g / group_sbs) * n + row);
  }
}

// Sum of the 32 table lookups of superblock slot GI (4 partial sums for ILP).
// Every LDS offset is a compile-time immediate, GI*4096 + (q + 8b)*128, added
// to the byte taken from the quad's offsets.
template <int GI>
__device__ inline float superblock_sum(const float* tbl, const uint4 nb, const uint32_t sg) {
  const uint32_t nd[4] = {nb.x, nb.y, nb.z, nb.w};
  const char* t = reinterpret_cast<const char*>(tbl) + GI * kTableFloatsPerSb * 4;
  float s[4];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const uint32_t off = quad_offsets(nd[q >> 1], sg, q);
    const uint32_t o[4] = {off & 0xFFu, __builtin_amdgcn_ubfe(off, 8, 8), __builtin_amdgcn_ubfe(off, 16, 8),
                           off >> 24};
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const float v = *reinterpret_cast<const float*>(t + (q + 8 * b) * 128 + o[b]);
      s[b] = q == 0 ? v : s[b] + v;
    }
  }
  return (s[0] + s[1]) + (s[2] + s[3]);
}

template <int MODE, int WIN, int GI = 0>
__device__ inline void window_accumulate(const float* tbl, const RowWindow<MODE, WIN>& r, float& acc,
                                         float& accg, int& gpos, int group_sbs) {
  if constexpr (GI < WIN) {
    const float sb = superblock_sum<GI>(tbl, r.nb[GI], r.sg[GI]);
    if constexpr (MODE == kGroup1) {
      acc += r.al[GI] * sb;
    } else if constexpr (MODE == kGroupN) {
      accg += sb;
      if (++gpos == group_sbs) {
        acc += r.al[GI] * accg;
        accg = 0.f;
        gpos = 0;
      }
    } else {
      acc += sb;
    }
    window_accumulate<MODE, WIN, GI + 1>(tbl, r, acc, accg, gpos, group_sbs);
  }
}

// Batch-1 GEMV.  Workgroup = 256 threads = 256 rows x M row slots; K range =
// one split; LDS holds the tables of WIN superblocks at a time (WIN*4 KB).
// For each window: build the tables, then per row slot issue the whole
// row-window of loads (WIN x 24 bytes per lane, non-temporal: read once) and
// consume it.  Latency is hidden by occupancy: at ~55 VGPRs and 16 KB of LDS
// per workgroup, 8 waves share each SIMD.
template <int MODE, int WIN, int M, bool YBF16>
__global__ __launch_bounds__(kLutThreads) void gemv_b1_lut_kernel(
    const uint8_t* __restrict__ packed, const float* __restrict__ alpha,
    const uint16_t* __restrict__ x, void* __restrict__ y, float* __restrict__ partial, int64_t n,
    int64_t k, int group_sbs, int ksplit, int64_t packed_stride, int64_t alpha_stride,
    int64_t y_stride) {
  __shared__ __attribute__((aligned(16))) float tbl[WIN * kTableFloatsPerSb];
  const int tid = threadIdx.x;
  const int64_t c = blockIdx.y;
  const int kz = blockIdx.z;
  const int64_t nsb = k / kSuperblock;
  const int64_t sb_per_split = nsb / ksplit;
  const int64_t sb_begin = kz * sb_per_split;
  const int nwin = (int)(sb_per_split / WIN);

  const uint8_t* pk = packed + c * packed_stride;
  const uint8_t* __restrict__ sgn_base = pk + nibble_plane_bytes(n, k);
  const float* __restrict__ al = alpha + c * alpha_stride;
  const int64_t row_base = (int64_t)blockIdx.x * (kLutThreads * M) + tid;

  // rows past the end are clamped for loads (their results are not stored)
  uint32_t rows[M];
#pragma unroll
  for (int i = 0; i < M; ++i) {
    const int64_t r = row_base + (int64_t)i * kLutThreads;
    rows[i] = (uint32_t)(r < n ? r : n - 1);
  }

  float acc[M], accg[M];
  int gpos[M];
#pragma unroll
  for (int i = 0; i < M; ++i) {
    acc[i] = accg[i] = 0.f;
    gpos[i] = 0;
  }

  for (int w = 0; w < nwin; ++w) {
    const int64_t g0 = sb_begin + (int64_t)w * WIN;
    __syncthreads();  // previous window's lookups are done
    for (int task = tid; task < WIN * kBlocksPerSb * 2; task += kLutThreads) {
      const int blk = task >> 1;
      build_block_half(tbl + blk * 32, x + g0 * kSuperblock + blk * 4, task & 1);
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < M; ++i) {
      RowWindow<MODE, WIN> rw;
      load_row_window<MODE, WIN>(rw, pk, sgn_base, al, n, rows[i], g0, group_sbs);
      window_accumulate<MODE, WIN>(tbl, rw, acc[i], accg[i], gpos[i], group_sbs);
    }
  }

#pragma unroll
  for (int i = 0; i < M; ++i) {
    const int64_t row = row_base + (int64_t)i * kLutThreads;
    if (row >= n) continue;
    float v = acc[i];
    if (ksplit == 1) {
      if constexpr (MODE == kChannel) v *= al[row];
      if constexpr (MODE == kTensor) v *= al[0];
      store_y<YBF16>(y, c * y_stride + row, v);
    } else {
      partial[(c * ksplit + kz) * n + row] = v;
    }
  }
}

// Decode table entry for a code: the high bytes of the 4 bf16 weights, with
// +-0.5 (0x3F / 0xBF) for kept weights and 0 for the pruned one.
__device__ inline uint32_t decode_table_entry(uint32_t code) {
  const uint32_t z = (code >> 2) & 3;
  const uint32_t neg0 = (code >> 4) & 1;
  const uint32_t neg1 = neg0 ^ (code & 1);
  const uint32_t neg2 = neg0 ^ ((code >> 1) & 1);
  uint32_t e = 0;
  uint32_t rank = 0;
  for (uint32_t pos = 0; pos < 4; ++pos) {
    if (pos == z) continue;
    const uint32_t neg = rank == 0 ? neg0 : (rank == 1 ? neg1 : neg2);
    e |= (neg ? 0xBFu : 0x3Fu) << (8 * pos);
    ++rank;
  }
  return e;
}

// Batch 2..16.  Workgroup = 4 waves; a wave owns 4 tiles of 16 rows (64
// rows) so every activation fragment feeds 4 MFMAs.  The K loop walks one
// superblock at a time through a ring of kMfmaDepth register sets: while the
// MFMAs of superblock g run, the lane's records (nibble dword q and sign dword
// of its 4 rows, and the group scales) for g + kMfmaDepth - 1 and the
// activation fragments for g + 1 are already on their way, so the weight
// stream never waits for a compute phase.  Lane (r, q) supplies blocks 2q+8t
// and 2q+1+8t (t = 0..3) of row r, i.e. k = 32t + 8q .. +7 of the
// superblock, and the activations of batch row r at the same k.
constexpr int kMfmaTiles = 4;
constexpr int kMfmaDepth = 4;

template <int J>
using RingSlot = std::integral_constant<int, J>;

template <int MODE, bool YBF16>
__global__ __launch_bounds__(256) void gemv_mfma_kernel(
    const uint8_t* __restrict__ packed, const float* __restrict__ alpha,
    const uint16_t* __restrict__ x, void* __restrict__ y, float* __restrict__ partial, int64_t n,
    int64_t k, int group_sbs, int batch, int ksplit, int64_t packed_stride, int64_t alpha_stride,
    int64_t y_stride) {
  __shared__ uint32_t dtbl[32];
  if (threadIdx.x < 32) dtbl[threadIdx.x] = decode_table_entry(threadIdx.x);
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane & 15;  // weight row inside a 16-row tile / batch row of x
  const int q = lane >> 4;  // nibble dword q of each superblock record
  const int64_t row0 = (int64_t)blockIdx.x * (64 * kMfmaTiles) + wave * (16 * kMfmaTiles) + r;
  const int64_t c = blockIdx.y;
  const int kz = blockIdx.z;
  const int64_t nsb = k / kSuperblock;
  const int64_t sb_per_split = nsb / ksplit;
  const int64_t sb_begin = kz * sb_per_split;
  const int64_t sb_end = sb_begin + sb_per_split;

  const uint8_t* pk = packed + c * packed_stride;
  const uint8_t* __restrict__ sgn_base = pk + nibble_plane_bytes(n, k);
  const float* __restrict__ al = alpha + c * alpha_stride;
  // lanes past the batch read row 0: they only feed output rows that are not
  // stored, and an unconditional load needs no branch
  const uint16_t* xrow = x + (int64_t)(r < batch ? r : 0) * k;
  const char* dt = reinterpret_cast<const char*>(dtbl);
  constexpr bool kGroup = MODE == kGroup1 || MODE == kGroupN;

  uint32_t rows[kMfmaTiles];
#pragma unroll
  for (int i = 0; i < kMfmaTiles; ++i) {
    const int64_t rr = row0 + i * 16;
    rows[i] = (uint32_t)(rr < n ? rr : n - 1);  // clamped rows are not stored
  }

  f32x4 acc[kMfmaTiles], accg[kMfmaTiles];
#pragma unroll
  for (int i = 0; i < kMfmaTiles; ++i) {
    acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    accg[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  int gpos = 0;

  uint32_t nd[kMfmaDepth][kMfmaTiles], sg[kMfmaDepth][kMfmaTiles];
  float av[kMfmaDepth][kGroup ? kMfmaTiles : 1];
  u32x4 xf[2][4];
  // fetches past the split's end repeat its last superblock (never used)
  auto fetch = [&](auto J, int64_t g) {
    constexpr int j = decltype(J)::value;
    g = g < sb_end ? g : sb_end - 1;
#pragma unroll
    for (int i = 0; i < kMfmaTiles; ++i) {
      nd[j][i] = stream_load(reinterpret_cast<const uint32_t*>(pk + g * n * 16 + rows[i] * 16u + q * 4u));
      sg[j][i] = stream_load(reinterpret_cast<const uint32_t*>(sgn_base + g * n * 4 + rows[i] * 4u));
      if constexpr (MODE == kGroup1) av[j][i] = stream_load(al + g * n + rows[i]);
      if constexpr (MODE == kGroupN) av[j][i] = stream_load(al + (g / group_sbs) * n + rows[i]);
    }
  };
  auto fetch_x = [&](auto X, int64_t g) {
    constexpr int xs = decltype(X)::value;
    g = g < sb_end ? g : sb_end - 1;
#pragma unroll
    for (int t = 0; t < 4; ++t) xf[xs][t] = *reinterpret_cast<const u32x4*>(xrow + g * kSuperblock + 32 * t + 8 * q);
  };
  auto compute = [&](auto J, auto X) {
    constexpr int j = decltype(J)::value;
    constexpr int xs = decltype(X)::value;
    uint32_t off_lo[kMfmaTiles], off_hi[kMfmaTiles];
#pragma unroll
    for (int i = 0; i < kMfmaTiles; ++i) {
      off_lo[i] = quad_offsets(nd[j][i], sg[j][i], 2 * q);      // blocks 2q + 8t
      off_hi[i] = quad_offsets(nd[j][i], sg[j][i], 2 * q + 1);  // blocks 2q + 1 + 8t
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const bf16x8 xv = __builtin_bit_cast(bf16x8, xf[xs][t]);
#pragma unroll
      for (int i = 0; i < kMfmaTiles; ++i) {
        const uint32_t e0 = *reinterpret_cast<const uint32_t*>(dt + __builtin_amdgcn_ubfe(off_lo[i], 8 * t, 8));
        const uint32_t e1 = *reinterpret_cast<const uint32_t*>(dt + __builtin_amdgcn_ubfe(off_hi[i], 8 * t, 8));
        u32x4 wv;
        wv[0] = __builtin_amdgcn_perm(0u, e0, 0x010C000Cu);
        wv[1] = __builtin_amdgcn_perm(0u, e0, 0x030C020Cu);
        wv[2] = __builtin_amdgcn_perm(0u, e1, 0x010C000Cu);
        wv[3] = __builtin_amdgcn_perm(0u, e1, 0x030C020Cu);
        if constexpr (kGroup) {
          accg[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xv, __builtin_bit_cast(bf16x8, wv), accg[i], 0, 0, 0);
        } else {
          acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xv, __builtin_bit_cast(bf16x8, wv), acc[i], 0, 0, 0);
        }
      }
    }
    if constexpr (kGroup) {
      if (++gpos == group_sbs) {
#pragma unroll
        for (int i = 0; i < kMfmaTiles; ++i) {
          const float a2 = 2.f * av[j][i];
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[i][e] += a2 * accg[i][e];
          accg[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        gpos = 0;
      }
    }
  };
  // one superblock: prefetch, then compute slot J with activations X
  auto step = [&](auto J, auto X, int64_t g) {
    constexpr int j = decltype(J)::value;
    constexpr int xs = decltype(X)::value;
    fetch(RingSlot<(j + kMfmaDepth - 1) % kMfmaDepth>{}, g + kMfmaDepth - 1);
    fetch_x(RingSlot<1 - xs>{}, g + 1);
    compute(J, X);
  };

  static_assert(kMfmaDepth == 4, "the loop below is unrolled by the ring depth");
  fetch(RingSlot<0>{}, sb_begin);
  fetch(RingSlot<1>{}, sb_begin + 1);
  fetch(RingSlot<2>{}, sb_begin + 2);
  fetch_x(RingSlot<0>{}, sb_begin);
  // (every early exit leaves the loop, so each path into a step passes
  // through the step before it and the compiler's waits stay exact)
  for (int64_t g = sb_begin;; g += 4) {
    step(RingSlot<0>{}, RingSlot<0>{}, g);
    if (g + 1 >= sb_end) break;
    step(RingSlot<1>{}, RingSlot<1>{}, g + 1);
    if (g + 2 >= sb_end) break;
    step(RingSlot<2>{}, RingSlot<0>{}, g + 2);
    if (g + 3 >= sb_end) break;
    step(RingSlot<3>{}, RingSlot<1>{}, g + 3);
    if (g + 4 >= sb_end) break;
  }

  // lane holds D[batch 4q + e][row r] of each tile
#pragma unroll
  for (int i = 0; i < kMfmaTiles; ++i) {
    const int64_t row = row0 + i * 16;
    if (row >= n) continue;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int b = 4 * q + e;
      if (b >= batch) continue;
      float v = acc[i][e];
      if constexpr (!kGroup) v *= 2.f;
      if (ksplit == 1) {
        if constexpr (MODE == kChannel) v *= al[row];
        if constexpr (MODE == kTensor) v *= al[0];
        store_y<YBF16>(y, c * y_stride + (int64_t)b * n + row, v);
      } else {
        partial[((c * ksplit + kz) * batch + b) * n + row] = v;
      }
    }
  }
}

// Split-K second stage: fixed-order sum of the partials, then the per-channel
// or per-tensor scale and the output conversion.
template <int GRAN, bool YBF16>
__global__ void gemv_split_reduce(const float* __restrict__ partial, const float* __restrict__ alpha,
                                  void* __restrict__ y, int64_t n, int batch, int ksplit, int count,
                                  int64_t alpha_stride, int64_t y_stride) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per = (int64_t)batch * n;
  if (idx >= per * count) return;
  const int64_t c = idx / per;
  const int64_t bn = idx % per;
  const int64_t row = bn % n;
  float v = 0.f;
  for (int s = 0; s < ksplit; ++s) v += partial[(c * ksplit + s) * per + bn];
  const float* al = alpha + c * alpha_stride;
  if constexpr (GRAN == SHERRY_PER_CHANNEL) v *= al[row];
  if constexpr (GRAN == SHERRY_PER_TENSOR) v *= al[0];
  store_y<YBF16>(y, c * y_stride + bn, v);
}

template <int MODE, int WIN, int M, bool YBF16>
void launch_lut_one(dim3 grid, size_t lds, hipStream_t s, const uint8_t* packed, const float* alpha,
                    const uint16_t* x, void* y, float* ws, int64_t n, int64_t k, int group_sbs, int ksplit,
                    int64_t ps, int64_t as, int64_t ys) {
  hipLaunchKernelGGL((gemv_b1_lut_kernel<MODE, WIN, M, YBF16>), grid, dim3(kLutThreads), lds, s, packed,
                     alpha, x, y, ws, n, k, group_sbs, ksplit, ps, as, ys);
}

template <int MODE, int WIN, bool YBF16>
void launch_lut_m(int m, dim3 grid, size_t lds, hipStream_t s, const uint8_t* packed, const float* alpha,
                  const uint16_t* x, void* y, float* ws, int64_t n, int64_t k, int group_sbs, int ksplit,
                  int64_t ps, int64_t as, int64_t ys) {
  if (m >= 4) launch_lut_one<MODE, WIN, 4, YBF16>(grid, lds, s, packed, alpha, x, y, ws, n, k, group_sbs, ksplit, ps, as, ys);
  else if (m == 2) launch_lut_one<MODE, WIN, 2, YBF16>(grid, lds, s, packed, alpha, x, y, ws, n, k, group_sbs, ksplit, ps, as, ys);
  else launch_lut_one<MODE, WIN, 1, YBF16>(grid, lds, s, packed, alpha, x, y, ws, n, k, group_sbs, ksplit, ps, as, ys);
}

template <int MODE, bool YBF16>
void launch_lut_w(int win, int m, dim3 grid, size_t lds, hipStream_t s, const uint8_t* packed,
                  const float* alpha, const uint16_t* x, void* y, float* ws, int64_t n, int64_t k,
                  int group_sbs, int ksplit, int64_t ps, int64_t as, int64_t ys) {
  switch (win) {
    case 16: launch_lut_m<MODE, 16, YBF16>(m, grid, lds, s, packed, alpha, x, y, ws, n, k, group_sbs, ksplit, ps, as, ys); break;
    case 8: launch_lut_m<MODE, 8, YBF16>(m, grid, lds, s, packed, alpha, x, y, ws, n, k, group_sbs, ksplit, ps, as, ys); break;
    case 4: launch_lut_m<MODE, 4, YBF16>(m, grid, lds, s, packed, alpha, x, y, ws, n, k, group_sbs, ksplit, ps, as, ys); break;
    case 2: launch_lut_m<MODE, 2, YBF16>(m, grid, lds, s, packed, alpha, x, y, ws, n, k, group_sbs, ksplit, ps, as, ys); break;
    default: launch_lut_m<MODE, 1, YBF16>(m, grid, lds, s, packed, alpha, x, y, ws, n, k, group_sbs, ksplit, ps, as, ys); break;
  }
}

template <bool YBF16>
void launch_lut(int mode, int win, int m, dim3 grid, size_t lds, hipStream_t s, const uint8_t* packed,
                const float* alpha, const uint16_t* x, void* y, float* ws, int64_t n, int64_t k, int group_sbs,
                int ksplit, int64_t ps, int64_t as, int64_t ys) {
  switch (mode) {
    case kGroup1: launch_lut_w<kGroup1, YBF16>(win, m, grid, lds, s, packed, alpha, x, y, ws, n, k, group_sbs, ksplit, ps, as, ys); break;
    case kGroupN: launch_lut_w<kGroupN, YBF16>(win, m, grid, lds, s, packed, alpha, x, y, ws, n, k, group_sbs, ksplit, ps, as, ys); break;
    case kChannel: launch_lut_w<kChannel, YBF16>(win, m, grid, lds, s, packed, alpha, x, y, ws, n, k, group_sbs, ksplit, ps, as, ys); break;
    default: launch_lut_w<kTensor, YBF16>(win, m, grid, lds, s, packed, alpha, x, y, ws, n, k, group_sbs, ksplit, ps, as, ys); break;
  }
}

template <int GRAN, bool YBF16>
hipError_t launch_gemv_t(const GemvPlan& p, int64_t n, int64_t k, int group_size,
                         const uint8_t* packed, const float* alpha, const uint16_t* x, int batch,
                         void* y, int count, int64_t packed_stride, int64_t alpha_stride,
                         int64_t y_stride, float* ws, hipStream_t s) {
  const int group_sbs = GRAN == SHERRY_PER_GROUP ? group_size / kSuperblock : 1;
  const dim3 grid((unsigned)p.panels, (unsigned)count, (unsigned)p.ksplit);
  if (p.kind == 0) {
    const size_t lds = 0;  // the table is static LDS sized by the window
    const int mode = GRAN == SHERRY_PER_CHANNEL ? kChannel
                   : GRAN == SHERRY_PER_TENSOR  ? kTensor
                   : (group_sbs == 1 ? kGroup1 : kGroupN);
    launch_lut<YBF16>(mode, p.window_sbs, p.rows_per_thread, grid, lds, s, packed, alpha, x, y, ws, n, k,
                      group_sbs, p.ksplit, packed_stride, alpha_stride, y_stride);
  } else {
    const int mode = GRAN == SHERRY_PER_CHANNEL ? kChannel
                   : GRAN == SHERRY_PER_TENSOR  ? kTensor
                   : (group_sbs == 1 ? kGroup1 : kGroupN);
#define SHERRY_MFMA_CASE(MD)                                                                                \
  hipLaunchKernelGGL((gemv_mfma_kernel<MD, YBF16>), grid, dim3(256), 0, s, packed, alpha, x, y, ws, n, k, \
                     group_sbs, batch, p.ksplit, packed_stride, alpha_stride, y_stride)
    if (mode == kGroup1) SHERRY_MFMA_CASE(kGroup1);
    else if (mode == kGroupN) SHERRY_MFMA_CASE(kGroupN);
    else if (mode == kChannel) SHERRY_MFMA_CASE(kChannel);
    else SHERRY_MFMA_CASE(kTensor);
#undef SHERRY_MFMA_CASE
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.ksplit == 1) return e;
  const int64_t items = (int64_t)count * batch * n;
  hipLaunchKernelGGL((gemv_split_reduce<GRAN, YBF16>), dim3((unsigned)((items + 255) / 256)), dim3(256), 0,
                     s, ws, alpha, y, n, batch, p.ksplit, count, alpha_stride, y_stride);
  return hipGetLastError();
}

}  // namespace

GemvPlan plan_gemv(int64_t n, int64_t k, int gran, int group_size, int batch, int count) {
  GemvPlan p{};
  const int64_t nsb = k / kSuperblock;
  const int64_t group_sbs = gran == SHERRY_PER_GROUP ? group_size / kSuperblock : 1;
  p.kind = batch == 1 ? 0 : 1;
  int64_t rows_per_wg;
  if (p.kind == 0) {
    // four row slots per thread amortize the table build once the grid is large
    const int64_t wg1 = ((n + kLutThreads - 1) / kLutThreads) * count;
    p.rows_per_thread = wg1 >= 4096 ? SHERRY_LUT_ROWS : 1;
    rows_per_wg = (int64_t)kLutThreads * p.rows_per_thread;
  } else {
    p.rows_per_thread = 1;
    rows_per_wg = 64 * kMfmaTiles;
  }
  p.panels = (n + rows_per_wg - 1) / rows_per_wg;
  // Split K (in whole groups) until the launch has ~2048 workgroups (batch 1;
  // the table kernel keeps 8 per CU resident) or ~1024 (batch > 1).
  const int64_t wgs = p.panels * count;
  const int64_t groups = nsb / group_sbs;
  int64_t split = 1;
  const int64_t target = p.kind == 0 ? SHERRY_GEMV_SPLIT_TARGET : 1024;
  while (wgs * split * 2 <= target && groups % (split * 2) == 0) split *= 2;
  p.ksplit = (int)split;
  const int64_t sb_per_split = nsb / split;
  int win = SHERRY_LUT_WIN_MAX;
  while (sb_per_split % win != 0) win >>= 1;
  p.window_sbs = win;
  p.workspace_bytes = split > 1 ? (size_t)count * split * batch * n * sizeof(float) : 0;
  return p;
}

hipError_t launch_gemv(const GemvPlan& p, int64_t n, int64_t k, int gran, int group_size,
                       const uint8_t* packed, const float* alpha, const uint16_t* x, int batch,
                       void* y, bool y_bf16, int count, int64_t packed_stride,
                       int64_t alpha_stride, int64_t y_stride, float* ws, hipStream_t s) {
#define SHERRY_GEMV_CASE(G, B)                                                                        \
  return launch_gemv_t<G, B>(p, n, k, group_size, packed, alpha, x, batch, y, count, packed_stride, \
                             alpha_stride, y_stride, ws, s)
  if (gran == SHERRY_PER_GROUP) {
    if (y_bf16) SHERRY_GEMV_CASE(SHERRY_PER_GROUP, true);
    SHERRY_GEMV_CASE(SHERRY_PER_GROUP, false);
  } else if (gran == SHERRY_PER_CHANNEL) {
    if (y_bf16) SHERRY_GEMV_CASE(SHERRY_PER_CHANNEL, true);
    SHERRY_GEMV_CASE(SHERRY_PER_CHANNEL, false);
  } else {
    if (y_bf16) SHERRY_GEMV_CASE(SHERRY_PER_TENSOR, true);
    SHERRY_GEMV_CASE(SHERRY_PER_TENSOR, false);
  }
#undef SHERRY_GEMV_CASE
}

}  // namespace sherry
