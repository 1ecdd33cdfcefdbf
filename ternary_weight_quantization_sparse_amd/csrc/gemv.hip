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
// v_mfma_f32_16x16x32_bf16 with the batch as the M dimension; weight records
// and activations reach LDS by DMA copies (details at the kernel).
#include <type_traits>

#include "sherry_internal.h"

namespace sherry {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kLutThreads = 256;
#ifndef SHERRY_GEMV_SPLIT_TARGET
#define SHERRY_GEMV_SPLIT_TARGET 2048      // batch 1: split K until a launch has ~this many 256-row workgroups
#endif
#ifndef SHERRY_GEMV_MFMA_SPLIT_TARGET
#define SHERRY_GEMV_MFMA_SPLIT_TARGET 768  // batch 2..16: the same, for the MFMA kernel
#endif
#ifndef SHERRY_LUT_WIN_MAX
#define SHERRY_LUT_WIN_MAX 4  // superblocks per LDS table window (4 -> 16 KB)
#endif
#ifndef SHERRY_LUT_NT
#define SHERRY_LUT_NT 1       // non-temporal loads for the packed stream
#endif
#ifndef SHERRY_LUT_ONEWIN
#define SHERRY_LUT_ONEWIN 1  // batch-1 splits of one window: records and activations loaded together
#endif
#ifndef SHERRY_LUT_ROWS
#define SHERRY_LUT_ROWS 1     // row slots per thread on large launches
#endif
constexpr int kTableFloatsPerSb = kBlocksPerSb * 32;  // 32 entries per block

// The 4 byte offsets (entry * 4, into a block's 32-entry fp32 table of 128
// bytes) of the blocks in quad q of a superblock record.
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
__device__ inline void build_block_half_x(float* blk_tbl, const uint2 xv, int h) {
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

__device__ inline void build_block_half(float* blk_tbl, const uint16_t* __restrict__ xblk, int h) {
  build_block_half_x(blk_tbl, *reinterpret_cast<const uint2*>(xblk), h);
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

// Batch-1 GEMV.  Workgroup = RW x KW waves: RW row waves (64 rows each, M
// row slots per lane) times KW K-slices.  Slice s owns superblocks
// [s S, (s + 1) S) of the row range (S = K / 128 / KW, whole groups), and its
// RW waves share that slice's tables.  For each window of WIN superblocks:
// the workgroup builds every slice's tables (one 32-entry table per block of
// 4 activations, 4 KB per superblock), then each lane issues its row-window
// of loads (WIN x 24 bytes, non-temporal: read once) and consumes it.  With
// KW > 1 the slices' partial sums of a row are added in slice order through
// LDS at the end (deterministic): launches with few rows split K inside the
// workgroup instead of across workgroups, so a call is one kernel with no
// workspace.  Latency is hidden by occupancy: ~55 VGPRs and 16-64 KB of LDS
// per workgroup, 8 waves per SIMD.
template <int MODE, int WIN, int M, bool YBF16, int RW, int KW, bool ONEWIN = false>
__global__ __launch_bounds__(64 * RW * KW) void gemv_b1_lut_kernel(
    const uint8_t* __restrict__ packed, const float* __restrict__ alpha,
    const uint16_t* __restrict__ x, void* __restrict__ y, float* __restrict__ partial, int64_t n, int64_t k,
    int group_sbs, int ksplit, int64_t packed_stride, int64_t alpha_stride, int64_t y_stride) {
  constexpr int kRows = 64 * RW;  // rows per row slot
  constexpr int kThreadsWg = 64 * RW * KW;
  __shared__ __attribute__((aligned(16))) float tbl[KW][WIN * kTableFloatsPerSb];
  __shared__ float red[KW > 1 ? KW : 1][KW > 1 ? kRows * M : 1];
  const int tid = threadIdx.x;
  const int slice = tid / kRows;      // K-slice of this thread
  const int rtid = tid % kRows;       // row inside a row slot
  const int64_t c = blockIdx.y;
  const int kz = blockIdx.z;  // split across workgroups (KW == 1 only)
  const int64_t nsb = k / kSuperblock / ksplit;
  const int64_t per_slice = nsb / KW;
  const int64_t sb_begin = kz * nsb + slice * per_slice;
  const int nwin = (int)(per_slice / WIN);

  const uint8_t* pk = packed + c * packed_stride;
  const uint8_t* __restrict__ sgn_base = pk + nibble_plane_bytes(n, k);
  const float* __restrict__ al = alpha + c * alpha_stride;
  const int64_t row_base = (int64_t)blockIdx.x * (kRows * M) + rtid;

  // rows past the end are clamped for loads (their results are not stored)
  uint32_t rows[M];
#pragma unroll
  for (int i = 0; i < M; ++i) {
    const int64_t r = row_base + (int64_t)i * kRows;
    rows[i] = (uint32_t)(r < n ? r : n - 1);
  }

  float acc[M], accg[M];
  int gpos[M];
#pragma unroll
  for (int i = 0; i < M; ++i) {
    acc[i] = accg[i] = 0.f;
    gpos[i] = 0;
  }

  // Split launches (few workgroups, several windows per slice) issue window
  // w + 1's loads (packed data and the activations of the next tables)
  // before consuming window w, so their latency runs under the lookups and
  // the next table build.  Full launches keep one window of registers: their
  // occupancy (8 waves per SIMD) hides the latency.
  constexpr bool kAhead = KW > 1;
  if constexpr (ONEWIN) {
    // One window per workgroup (the launcher checks it): the activations of
    // the table and the row's records are loaded together before the table
    // build, so one memory latency is exposed per workgroup instead of two in
    // sequence.  The activations go first: the build waits only for them.
    static_assert(KW == 1 && M == 1, "one row slot, one slice");
    constexpr int kTasks = WIN * kBlocksPerSb * 2;
    static_assert(kTasks <= kThreadsWg, "one table task per thread");
    const bool has_task = tid < kTasks;
    const int blk = (tid >> 1) % (WIN * kBlocksPerSb);
    const uint2 xv = has_task ? *reinterpret_cast<const uint2*>(x + sb_begin * kSuperblock + blk * 4)
                              : make_uint2(0u, 0u);
    RowWindow<MODE, WIN> rw;
    load_row_window<MODE, WIN>(rw, pk, sgn_base, al, n, rows[0], sb_begin, group_sbs);
    if (has_task) build_block_half_x(tbl[0] + blk * 32, xv, tid & 1);
    __syncthreads();
    window_accumulate<MODE, WIN>(tbl[0], rw, acc[0], accg[0], gpos[0], group_sbs);
  } else if constexpr (kAhead) {
    // the plan gives every thread at most one table task per window
    // (KW * WIN * 64 <= threads), so each thread also prefetches the 8 bytes
    // of activations its next task needs
    constexpr int kTasks = KW * WIN * kBlocksPerSb * 2;
    static_assert(kTasks <= kThreadsWg, "one table task per thread and window");
    const bool has_task = tid < kTasks;
    const int ts = tid / (WIN * kBlocksPerSb * 2);
    const int blk = (tid >> 1) % (WIN * kBlocksPerSb);
    const uint16_t* xsrc = x + (has_task ? (kz * nsb + ts * per_slice) * kSuperblock + blk * 4 : 0);
    float* tdst = tbl[has_task ? ts : 0] + blk * 32;
    RowWindow<MODE, WIN> cur[M], nxt[M];
    uint2 xcur = has_task ? *reinterpret_cast<const uint2*>(xsrc) : make_uint2(0u, 0u), xnxt = xcur;
#pragma unroll
    for (int i = 0; i < M; ++i) load_row_window<MODE, WIN>(cur[i], pk, sgn_base, al, n, rows[i], sb_begin, group_sbs);
    for (int w = 0; w < nwin; ++w) {
      __syncthreads();  // previous window's lookups are done
      if (has_task) build_block_half_x(tdst, xcur, tid & 1);
      __syncthreads();
      if (w + 1 < nwin) {
        const int64_t g1 = sb_begin + (int64_t)(w + 1) * WIN;
#pragma unroll
        for (int i = 0; i < M; ++i) load_row_window<MODE, WIN>(nxt[i], pk, sgn_base, al, n, rows[i], g1, group_sbs);
        if (has_task) xnxt = *reinterpret_cast<const uint2*>(xsrc + (int64_t)(w + 1) * WIN * kSuperblock);
      }
#pragma unroll
      for (int i = 0; i < M; ++i) {
        window_accumulate<MODE, WIN>(tbl[slice], cur[i], acc[i], accg[i], gpos[i], group_sbs);
        cur[i] = nxt[i];
      }
      xcur = xnxt;
    }
  } else {
    for (int w = 0; w < nwin; ++w) {
      const int64_t g0 = sb_begin + (int64_t)w * WIN;
      __syncthreads();  // previous window's lookups are done
      for (int task = tid; task < WIN * kBlocksPerSb * 2; task += kThreadsWg) {
        const int blk = task >> 1;
        build_block_half(tbl[0] + blk * 32, x + g0 * kSuperblock + blk * 4, task & 1);
      }
      __syncthreads();
#pragma unroll
      for (int i = 0; i < M; ++i) {
        RowWindow<MODE, WIN> rw;
        load_row_window<MODE, WIN>(rw, pk, sgn_base, al, n, rows[i], g0, group_sbs);
        window_accumulate<MODE, WIN>(tbl[0], rw, acc[i], accg[i], gpos[i], group_sbs);
      }
    }
  }

  if constexpr (KW > 1) {
#pragma unroll
    for (int i = 0; i < M; ++i) red[slice][i * kRows + rtid] = acc[i];
    __syncthreads();
    if (slice != 0) return;
#pragma unroll
    for (int i = 0; i < M; ++i) {
      float v = red[0][i * kRows + rtid];
#pragma unroll
      for (int t = 1; t < KW; ++t) v += red[t][i * kRows + rtid];
      acc[i] = v;
    }
  }
#pragma unroll
  for (int i = 0; i < M; ++i) {
    const int64_t row = row_base + (int64_t)i * kRows;
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

// Batch 2..16.  Workgroup = 4 waves; a wave owns 64 rows as 4 tiles of 16,
// so every activation fragment feeds 4 MFMAs, and walks the split's K range
// one superblock at a time.  Lane (r, q) supplies blocks 2q+8t and 2q+1+8t
// (t = 0..3) of row r of each tile, i.e. k = 32t + 8q .. +7 of the
// superblock -- exactly nibble dword q of the row's record -- and the
// activations of batch row r at the same k.
//
// Every load of the K loop is an LDS-DMA copy, which holds no registers in
// flight, with explicit vmcnt waits (vmcnt counts in issue order, so a
// register load issued a step ahead would force every copy issued before it
// to land, and the ring would collapse):
// * weights: each wave copies its own rows' records (1 KB of nibble records,
//   256 B of sign dwords and, for per_group, 256 B of scales per superblock)
//   into a private ring kMfmaRing superblocks deep, kMfmaRing - 1 ahead.  No
//   barrier: no wave reads another's records.
// * activations: chunks of kXChunk superblocks x XR batch rows (the batch
//   rounded up; extra rows copy row 0), double-buffered and shared by the
//   workgroup: the next chunk's copy is issued when a chunk starts and
//   published by one barrier when it ends.  Rows are padded by 16 bytes so
//   16 lanes reading 16 rows touch every bank once.
//
// Decode: a 32-entry LDS table holds each code's four bf16 weights (+-1, 0)
// as one 8-byte entry; one ds_read_b64 per block gives both operand dwords
// (a table of 4-byte high-byte entries plus two v_perm_b32 per block moves
// half that LDS traffic to the VALU and measured slower).  The byte offsets
// (code * 8) of four blocks come out of one nibble dword and the sign dword
// with four bit operations.  A tile's lookups are issued one tile ahead of
// its MFMAs so their latencies overlap.
//
// Per wave and superblock: 1.5 KB of weight records from HBM, ~42 LDS
// instructions (of which 32 table lookups, ~16 KB), ~85 VALU and 16 MFMA.
// The decode, not HBM, bounds this kernel: the issue and latency of the
// table lookups and the VALU; the lookups' bytes run at about half of what
// 8-byte lookups into this table sustain on gfx950.
constexpr int kMfmaTiles = 4;
#ifndef SHERRY_REDUCE4
#define SHERRY_REDUCE4 1  // split-K sums four outputs per thread where the shape allows
#endif
#ifndef SHERRY_MFMA_RING
#define SHERRY_MFMA_RING 3  // record ring slots per wave (superblocks in flight + 1)
#endif
constexpr int kMfmaRing = SHERRY_MFMA_RING;
#ifndef SHERRY_XCHUNK_SMALL
#define SHERRY_XCHUNK_SMALL 8  // superblocks per activation chunk at batch <= 4
#endif
// superblocks per activation chunk (a multiple of 4: one 1 KB copy per row
// and 4 superblocks) and bytes per chunk row (padded by 16)
template <int XR> constexpr int kXChunkOf = XR == 4 ? SHERRY_XCHUNK_SMALL : 4;
template <int XR> constexpr int kXPitchOf = kXChunkOf<XR> * kSuperblock * 2 + 16;
constexpr int kMRecNib = 0, kMRecSgn = 1024, kMRecAlpha = 1280;

template <int MODE, int XR, bool YBF16>
__global__ __launch_bounds__(256) void gemv_mfma_kernel(
    const uint8_t* packed, const float* alpha, const uint16_t* __restrict__ x, void* __restrict__ y,
    float* __restrict__ partial, int64_t n, int64_t k, int group_sbs, int batch, int ksplit,
    int64_t packed_stride, int64_t alpha_stride, int64_t y_stride) {
  constexpr bool kGroup = MODE == kGroup1 || MODE == kGroupN;
  constexpr int kRec = kGroup ? 1536 : 1280;  // record bytes per wave per superblock
  constexpr int kOps = kGroup ? 3 : 2;        // record copies per wave per superblock
  constexpr int kXChunk = kXChunkOf<XR>, kXPitch = kXPitchOf<XR>;
  constexpr int kXPieces = kXChunk / 4;       // 1 KB copies per activation row per chunk
  static_assert(kXChunk % 4 == 0, "chunks are whole 1 KB copies");
  static_assert(kMfmaRing - 2 <= kXChunk, "the chunk-end wait must not cover records still ahead");
  __shared__ __attribute__((aligned(16))) char ring[4][kMfmaRing * kRec];
  __shared__ __attribute__((aligned(16))) char xbuf[2][XR * kXPitch];
  __shared__ __attribute__((aligned(16))) uint2 dtab[32];
  if (threadIdx.x < 32) dtab[threadIdx.x] = decode_bf16(threadIdx.x);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15;  // weight row inside a 16-row tile / batch row of x
  const int q = lane >> 4;  // nibble dword q of each superblock record
  const int64_t wrow0 = (int64_t)blockIdx.x * (64 * kMfmaTiles) + wave * (16 * kMfmaTiles);
  const int64_t c = blockIdx.y;
  const int kz = blockIdx.z;
  const int64_t nsb = k / kSuperblock;
  const int sb_per_split = (int)(nsb / ksplit);
  const int64_t sb_begin = kz * (int64_t)sb_per_split;

  // (no __restrict__ on the record planes: the copies must stay where they
  // are issued)
  const uint8_t* pk = packed + c * packed_stride;
  const uint8_t* sgn_base = pk + nibble_plane_bytes(n, k);
  const float* al = alpha + c * alpha_stride;
  char* my_ring = ring[wave];
  const uint32_t ring_lds = (uint32_t)(size_t)(__attribute__((address_space(3))) char*)my_ring;

  // row whose records this lane copies (clamped rows are not stored)
  int64_t crow = wrow0 + lane;
  crow = crow < n ? crow : n - 1;

  // Copies of the records, in superblock order: each call copies superblock
  // `iss` of the split into ring slot `slot` and moves on to the next one
  // (past the end it copies the last one again; those are never used).  The
  // copies are buffer loads from resources based at the superblock's slice
  // of each plane (uniform bases advanced per copy, per-lane row offsets
  // fixed): with flat-encoded global_load_lds copies in flight the compiler
  // cannot count LDS reads in order and would wait for every table lookup
  // in flight before each tile's MFMAs, including the next tile's.  (The
  // shape checks keep n below 2^22, so a slice's byte range fits 32 bits.)
  int iss = 0, apos = 0;
  const uint8_t* nib_s = pk + sb_begin * n * 16;
  const uint8_t* sgn_s = sgn_base + sb_begin * n * 4;
  const float* al_s = al + (kGroup ? (sb_begin / group_sbs) * n : 0);
  const uint32_t v16 = (uint32_t)crow * 16u, v4 = (uint32_t)crow * 4u;
  auto issue = [&](int slot) {
    char* rb = my_ring + slot * kRec;
    const __amdgpu_buffer_rsrc_t nr =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(nib_s), (short)0, (int)(n * 16), kBufferWord3);
    const __amdgpu_buffer_rsrc_t sr =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(sgn_s), (short)0, (int)(n * 4), kBufferWord3);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(nr, (lds_void*)(rb + kMRecNib), 16, v16, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(sr, (lds_void*)(rb + kMRecSgn), 4, v4, 0, 0, 0);
    if constexpr (kGroup) {
      const __amdgpu_buffer_rsrc_t ar =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(al_s), (short)0, (int)(n * 4), kBufferWord3);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ar, (lds_void*)(rb + kMRecAlpha), 4, v4, 0, 0, 0);
    }
    if (iss + 1 < sb_per_split) {
      ++iss;
      nib_s += n * 16;
      sgn_s += n * 4;
      if constexpr (MODE == kGroup1) al_s += n;
      if constexpr (MODE == kGroupN) {
        if (++apos == group_sbs) { apos = 0; al_s += n; }
      }
    }
  };

  // activation chunk ch (superblocks kXChunk*ch .. of the split) into buffer
  // b: wave w copies rows w, w + 4, ...; each row is one 1 KB copy.  Reads
  // past the activations' end (a short last chunk) fall outside the buffer
  // resource and return zeros.
  const uint32_t xbytes = (uint32_t)(batch * k * 2);
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(x), (short)0, (int)xbytes, kBufferWord3);
  auto issue_x = [&](int ch, int b) {
    ch = ch * kXChunk < sb_per_split ? ch : (sb_per_split - 1) / kXChunk;
    const uint32_t col = (uint32_t)((sb_begin + (int64_t)ch * kXChunk) * (kSuperblock * 2)) + lane * 16u;
#pragma unroll
    for (int i = 0; i < XR / 4; ++i) {
      const int row = wave + 4 * i;
      const uint32_t src = (uint32_t)(row < batch ? row : 0) * (uint32_t)(k * 2);
#pragma unroll
      for (int pc = 0; pc < kXPieces; ++pc)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_void*)(xbuf[b] + row * kXPitch + pc * 1024), 16,
                                                 src + col + pc * 1024u, 0, 0, 0);
    }
  };

  // This lane's operands of one superblock: from its ring slot, nibble dword
  // q and the sign dword of rows r + 16 i (and for per_group their scales);
  // from the activation chunk, the four 16-byte fragments of batch row r.
  // One asm block that waits for its own results: the compiler cannot tell
  // these reads from ones that might overlap copies still in flight and
  // would wait for every copy first.
  uint32_t nd[kMfmaTiles], sg[kMfmaTiles];
  float av[kGroup ? kMfmaTiles : 1];
  u32x4 xf[4];
  const uint32_t xbuf_lds = (uint32_t)(size_t)(__attribute__((address_space(3))) char*)&xbuf[0][0];
  const uint32_t xrow_off = (uint32_t)((r < batch ? r : 0) * kXPitch + 16 * q);
  auto read_operands = [&](int slot, int b, int s) {
    const uint32_t rb = ring_lds + (uint32_t)(slot * kRec);
    const uint32_t a_nib = rb + kMRecNib + r * 16 + q * 4;
    const uint32_t a_sgn = rb + kMRecSgn + r * 4;
    const uint32_t a_x = xbuf_lds + (uint32_t)(b * XR * kXPitch + s * (kSuperblock * 2)) + xrow_off;
    u32x2 n01, n23, s01, s23;  // tiles (0, 1) and (2, 3)
    u32x4 x0, x1, x2, x3;
    if constexpr (kGroup) {
      const uint32_t a_al = rb + kMRecAlpha + r * 4;
      u32x2 a01, a23;
      asm volatile(
          "ds_read2st64_b32 %0, %10 offset1:1\n"
          "ds_read2st64_b32 %1, %10 offset0:2 offset1:3\n"
          "ds_read2_b32 %2, %11 offset1:16\n"
          "ds_read2_b32 %3, %11 offset0:32 offset1:48\n"
          "ds_read2_b32 %4, %12 offset1:16\n"
          "ds_read2_b32 %5, %12 offset0:32 offset1:48\n"
          "ds_read_b128 %6, %13\n"
          "ds_read_b128 %7, %13 offset:64\n"
          "ds_read_b128 %8, %13 offset:128\n"
          "ds_read_b128 %9, %13 offset:192\n"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(n01), "=&v"(n23), "=&v"(s01), "=&v"(s23), "=&v"(a01), "=&v"(a23),
            "=&v"(x0), "=&v"(x1), "=&v"(x2), "=&v"(x3)
          : "v"(a_nib), "v"(a_sgn), "v"(a_al), "v"(a_x)
          : "memory");
      av[0] = __uint_as_float(a01[0]);
      av[kGroup ? 1 : 0] = __uint_as_float(a01[1]);
      av[kGroup ? 2 : 0] = __uint_as_float(a23[0]);
      av[kGroup ? 3 : 0] = __uint_as_float(a23[1]);
    } else {
      asm volatile(
          "ds_read2st64_b32 %0, %8 offset1:1\n"
          "ds_read2st64_b32 %1, %8 offset0:2 offset1:3\n"
          "ds_read2_b32 %2, %9 offset1:16\n"
          "ds_read2_b32 %3, %9 offset0:32 offset1:48\n"
          "ds_read_b128 %4, %10\n"
          "ds_read_b128 %5, %10 offset:64\n"
          "ds_read_b128 %6, %10 offset:128\n"
          "ds_read_b128 %7, %10 offset:192\n"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(n01), "=&v"(n23), "=&v"(s01), "=&v"(s23), "=&v"(x0), "=&v"(x1), "=&v"(x2), "=&v"(x3)
          : "v"(a_nib), "v"(a_sgn), "v"(a_x)
          : "memory");
    }
    nd[0] = n01[0]; nd[1] = n01[1]; nd[2] = n23[0]; nd[3] = n23[1];
    sg[0] = s01[0]; sg[1] = s01[1]; sg[2] = s23[0]; sg[3] = s23[1];
    xf[0] = x0; xf[1] = x1; xf[2] = x2; xf[3] = x3;
  };

  f32x4 acc[kMfmaTiles], accg[kGroup ? kMfmaTiles : 1];
#pragma unroll
  for (int i = 0; i < kMfmaTiles; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  int gpos = 0;

  auto compute = [&]() {
    uint32_t off_lo[kMfmaTiles], off_hi[kMfmaTiles];
#pragma unroll
    for (int i = 0; i < kMfmaTiles; ++i) {
      off_lo[i] = quad_offsets8(nd[i], sg[i], 2 * q);      // blocks 2q + 8t
      off_hi[i] = quad_offsets8(nd[i], sg[i], 2 * q + 1);  // blocks 2q + 1 + 8t
    }
    const bool first = MODE == kGroup1 || (MODE == kGroupN && gpos == 0);  // a group starts here
    // Tile by tile: tile i + 1's 8 table lookups are issued before tile i's 4
    // MFMAs, so about 8-16 lookups are in flight at a time (a wave can have at
    // most 15 LDS operations outstanding: issuing all 32 of the superblock
    // first stalled issue), and their latency runs under the MFMAs.
    auto lookups = [&](int i, u32x4 (&w)[4]) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint2 e0 = *reinterpret_cast<const uint2*>(
            reinterpret_cast<const char*>(dtab) + __builtin_amdgcn_ubfe(off_lo[i], 8 * t, 8));
        const uint2 e1 = *reinterpret_cast<const uint2*>(
            reinterpret_cast<const char*>(dtab) + __builtin_amdgcn_ubfe(off_hi[i], 8 * t, 8));
        w[t] = u32x4{e0.x, e0.y, e1.x, e1.y};
      }
    };
    u32x4 wa[4], wb[4];
    lookups(0, wa);
#pragma unroll
    for (int i = 0; i < kMfmaTiles; ++i) {
      u32x4 (&wc)[4] = (i & 1) ? wb : wa;
      u32x4 (&wn)[4] = (i & 1) ? wa : wb;
      if (i + 1 < kMfmaTiles) lookups(i + 1, wn);
      __builtin_amdgcn_sched_barrier(0);  // keep the next tile's lookups ahead of these MFMAs
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const bf16x8 xv = __builtin_bit_cast(bf16x8, xf[t]);
        const bf16x8 w8 = __builtin_bit_cast(bf16x8, wc[t]);
        if constexpr (kGroup) {
          // the group's first MFMA starts from zero instead of clearing accg
          const f32x4 cin = (t == 0 && first) ? f32x4{0.f, 0.f, 0.f, 0.f} : accg[i];
          accg[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xv, w8, cin, 0, 0, 0);
        } else {
          acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xv, w8, acc[i], 0, 0, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (kGroup) {
      if (++gpos == group_sbs) {
#pragma unroll
        for (int i = 0; i < kMfmaTiles; ++i)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[i][e] += av[i] * accg[i][e];
        gpos = 0;
      }
    }
  };

  // Prologue: activation chunk 0, records of superblocks 0 .. kMfmaRing - 2.
  issue_x(0, 0);
  for (int j = 0; j < kMfmaRing - 1; ++j) issue(j);
  wait_vmcnt<(kMfmaRing - 1) * kOps>();  // chunk 0 has landed
  lds_barrier();                          // ... for every wave, and the table is written

  // Chunk ch: issue chunk ch + 1, then per superblock j: copy the records of
  // j + kMfmaRing - 1, wait for those of j (issued kMfmaRing - 1 steps ago; at
  // most the later records and one activation chunk are in flight), compute.
  int slot = 0;
  const int chunks = (sb_per_split + kXChunk - 1) / kXChunk;
  for (int ch = 0; ch < chunks; ++ch) {
    issue_x(ch + 1, (ch + 1) & 1);
#pragma unroll
    for (int s = 0; s < kXChunk; ++s) {
      const int j = ch * kXChunk + s;
      issue(slot == 0 ? kMfmaRing - 1 : slot - 1);  // superblock j + kMfmaRing - 1
      wait_vmcnt<(kMfmaRing - 1) * kOps>();
      if (j < sb_per_split) {
        read_operands(slot, ch & 1, s);
        compute();
      }
      slot = slot == kMfmaRing - 1 ? 0 : slot + 1;
    }
    // the next chunk was issued before this chunk's kXChunk record copies
    wait_vmcnt<kXChunk * kOps>();
    lds_barrier();
  }
  wait_vmcnt<0>();  // the trailing copies have landed in LDS before the wave ends

  // lane holds D[batch 4q + e][row r] of each tile
#pragma unroll
  for (int i = 0; i < kMfmaTiles; ++i) {
    const int64_t row = wrow0 + i * 16 + r;
    if (row >= n) continue;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int b = 4 * q + e;
      if (b >= batch) continue;
      float v = acc[i][e];
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
  // loads 8 splits ahead of their adds (one memory latency per 8 splits, not
  // per split); the adds keep split order
  const float* p = partial + c * ksplit * per + bn;
  float v = 0.f;
  for (int s0 = 0; s0 < ksplit; s0 += 8) {
    float t[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) t[j] = s0 + j < ksplit ? p[(int64_t)(s0 + j) * per] : 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (s0 + j < ksplit) v += t[j];
  }
  const float* al = alpha + c * alpha_stride;
  if constexpr (GRAN == SHERRY_PER_CHANNEL) v *= al[row];
  if constexpr (GRAN == SHERRY_PER_TENSOR) v *= al[0];
  store_y<YBF16>(y, c * y_stride + bn, v);
}

// The same sum, four consecutive outputs per thread with 16-byte loads, for
// launches whose per-copy output count batch * n is a multiple of 4 and
// whose total output count is at least 2^16 and fits 31 bits (32-bit index
// arithmetic).  Same split order, so the same bits.
template <int GRAN, bool YBF16>
__global__ __launch_bounds__(256) void gemv_split_reduce4(const float* __restrict__ partial,
                                                          const float* __restrict__ alpha, void* __restrict__ y,
                                                          int64_t n, int batch, int ksplit, int count,
                                                          int64_t alpha_stride, int64_t y_stride) {
  typedef float f4 __attribute__((ext_vector_type(4)));
  const uint32_t per = (uint32_t)batch * (uint32_t)n;
  const uint32_t idx = (blockIdx.x * blockDim.x + threadIdx.x) * 4u;
  if (idx >= per * (uint32_t)count) return;
  const uint32_t c = idx / per;
  const uint32_t bn = idx - c * per;
  const float* p = partial + (size_t)c * (size_t)ksplit * per + bn;
  f4 v = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < ksplit; s0 += 8) {
    f4 t[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      t[j] = s0 + j < ksplit ? *reinterpret_cast<const f4*>(p + (size_t)(s0 + j) * per) : f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (s0 + j < ksplit) v += t[j];
  }
  const float* al = alpha + c * alpha_stride;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float ve = v[e];
    if constexpr (GRAN == SHERRY_PER_CHANNEL) ve *= al[(bn + e) % (uint32_t)n];
    if constexpr (GRAN == SHERRY_PER_TENSOR) ve *= al[0];
    store_y<YBF16>(y, c * y_stride + bn + e, ve);
  }
}

template <int MODE, int WIN, int M, bool YBF16, int RW, int KW>
void launch_lut_one(dim3 grid, hipStream_t s, const uint8_t* packed, const float* alpha, const uint16_t* x,
                    void* y, float* ws, int64_t n, int64_t k, int group_sbs, int ksplit, int64_t ps, int64_t as,
                    int64_t ys) {
  if constexpr (KW == 1 && M == 1) {
    // one window per workgroup (a split across workgroups into single windows,
    // or K of one window)
    if (SHERRY_LUT_ONEWIN && k / kSuperblock / ksplit == WIN) {
      hipLaunchKernelGGL((gemv_b1_lut_kernel<MODE, WIN, M, YBF16, RW, KW, true>), grid, dim3(64 * RW * KW), 0, s,
                         packed, alpha, x, y, ws, n, k, group_sbs, ksplit, ps, as, ys);
      return;
    }
  }
  hipLaunchKernelGGL((gemv_b1_lut_kernel<MODE, WIN, M, YBF16, RW, KW>), grid, dim3(64 * RW * KW), 0, s, packed,
                     alpha, x, y, ws, n, k, group_sbs, ksplit, ps, as, ys);
}

// (rw, kw, win, m) -> instantiation; the plan only produces these shapes
template <int MODE, bool YBF16>
hipError_t launch_lut(const GemvPlan& p, dim3 grid, hipStream_t s, const uint8_t* packed, const float* alpha,
                      const uint16_t* x, void* y, float* ws, int64_t n, int64_t k, int group_sbs, int64_t ps,
                      int64_t as, int64_t ys) {
#define SHERRY_LUT(W, M_, RW_, KW_) \
  launch_lut_one<MODE, W, M_, YBF16, RW_, KW_>(grid, s, packed, alpha, x, y, ws, n, k, group_sbs, p.ksplit, ps, as, ys)
#define SHERRY_LUT_WIN(M_, RW_, KW_)                 \
  do {                                               \
    if (p.window_sbs >= 4) SHERRY_LUT(4, M_, RW_, KW_); \
    else if (p.window_sbs == 2) SHERRY_LUT(2, M_, RW_, KW_); \
    else SHERRY_LUT(1, M_, RW_, KW_);                \
  } while (0)
  const int cfg = p.rw * 100 + p.kw;
  if (cfg == 401 && p.rows_per_thread == 4) SHERRY_LUT_WIN(4, 4, 1);
  else if (cfg == 401) SHERRY_LUT_WIN(1, 4, 1);
  else if (cfg == 801) SHERRY_LUT_WIN(1, 8, 1);
  else if (cfg == 402) SHERRY_LUT_WIN(1, 4, 2);
  else if (cfg == 404) SHERRY_LUT_WIN(1, 4, 4);
  else if (cfg == 208) {
    if (p.window_sbs >= 2) SHERRY_LUT(2, 1, 2, 8);
    else SHERRY_LUT(1, 1, 2, 8);
  } else if (cfg == 116) SHERRY_LUT(1, 1, 1, 16);
  else return hipErrorInvalidValue;
#undef SHERRY_LUT_WIN
#undef SHERRY_LUT
  return hipSuccess;
}

template <int GRAN, bool YBF16>
hipError_t launch_gemv_t(const GemvPlan& p, int64_t n, int64_t k, int group_size,
                         const uint8_t* packed, const float* alpha, const uint16_t* x, int batch,
                         void* y, int count, int64_t packed_stride, int64_t alpha_stride,
                         int64_t y_stride, float* ws, hipStream_t s) {
  const int group_sbs = GRAN == SHERRY_PER_GROUP ? group_size / kSuperblock : 1;
  const dim3 grid((unsigned)p.panels, (unsigned)count, (unsigned)p.ksplit);
  if (p.kind == 0) {
    const int mode = GRAN == SHERRY_PER_CHANNEL ? kChannel
                   : GRAN == SHERRY_PER_TENSOR  ? kTensor
                   : (group_sbs == 1 ? kGroup1 : kGroupN);
    hipError_t le;
    if (mode == kGroup1) le = launch_lut<kGroup1, YBF16>(p, grid, s, packed, alpha, x, y, ws, n, k, group_sbs, packed_stride, alpha_stride, y_stride);
    else if (mode == kGroupN) le = launch_lut<kGroupN, YBF16>(p, grid, s, packed, alpha, x, y, ws, n, k, group_sbs, packed_stride, alpha_stride, y_stride);
    else if (mode == kChannel) le = launch_lut<kChannel, YBF16>(p, grid, s, packed, alpha, x, y, ws, n, k, group_sbs, packed_stride, alpha_stride, y_stride);
    else le = launch_lut<kTensor, YBF16>(p, grid, s, packed, alpha, x, y, ws, n, k, group_sbs, packed_stride, alpha_stride, y_stride);
    if (le != hipSuccess) return le;
  } else {
    const int mode = GRAN == SHERRY_PER_CHANNEL ? kChannel
                   : GRAN == SHERRY_PER_TENSOR  ? kTensor
                   : (group_sbs == 1 ? kGroup1 : kGroupN);
#define SHERRY_MFMA_XR(MD, XR)                                                                           \
  hipLaunchKernelGGL((gemv_mfma_kernel<MD, XR, YBF16>), grid, dim3(256), 0, s, packed, alpha, x, y, ws, n, \
                     k, group_sbs, batch, p.ksplit, packed_stride, alpha_stride, y_stride)
#define SHERRY_MFMA_CASE(MD)                                 \
  do {                                                       \
    if (batch <= 4) SHERRY_MFMA_XR(MD, 4);                   \
    else if (batch <= 8) SHERRY_MFMA_XR(MD, 8);              \
    else SHERRY_MFMA_XR(MD, 16);                             \
  } while (0)
    if (mode == kGroup1) SHERRY_MFMA_CASE(kGroup1);
    else if (mode == kGroupN) SHERRY_MFMA_CASE(kGroupN);
    else if (mode == kChannel) SHERRY_MFMA_CASE(kChannel);
    else SHERRY_MFMA_CASE(kTensor);
#undef SHERRY_MFMA_CASE
#undef SHERRY_MFMA_XR
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.ksplit == 1) return e;
  const int64_t items = (int64_t)count * batch * n;
  // four outputs per thread only for large outputs: a single call (N <= 8192
  // outputs, often tens of splits) needs the thread count of one output per
  // thread to keep enough loads in flight
  if (SHERRY_REDUCE4 && ((int64_t)batch * n) % 4 == 0 && items >= ((int64_t)1 << 16) &&
      items < ((int64_t)1 << 31)) {
    const int64_t threads = items / 4;
    hipLaunchKernelGGL((gemv_split_reduce4<GRAN, YBF16>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                       s, ws, alpha, y, n, batch, p.ksplit, count, alpha_stride, y_stride);
  } else {
    hipLaunchKernelGGL((gemv_split_reduce<GRAN, YBF16>), dim3((unsigned)((items + 255) / 256)), dim3(256), 0,
                       s, ws, alpha, y, n, batch, p.ksplit, count, alpha_stride, y_stride);
  }
  return hipGetLastError();
}

}  // namespace

GemvPlan plan_gemv(int64_t n, int64_t k, int gran, int group_size, int batch, int count) {
  GemvPlan p{};
  const int64_t nsb = k / kSuperblock;
  const int64_t group_sbs = gran == SHERRY_PER_GROUP ? group_size / kSuperblock : 1;
  const int64_t groups = nsb / group_sbs;
  p.ksplit = 1;
  if (batch == 1) {
    // Batch 1: 256-row workgroups sharing one set of tables (four row slots
    // per thread on very large grids).  A launch with fewer than
    // SHERRY_GEMV_SPLIT_TARGET of them splits K: inside the workgroup (KW
    // K-slices of 64-256 rows each, partial sums added through LDS, one
    // kernel) when every slice then holds a single window of tables -- this
    // is what single calls with K up to 2048 get -- and otherwise across
    // workgroups into fp32 partials summed by a second kernel in split order
    // (measured faster for long K and for the batched launches, whose
    // workgroups then need no barrier coupling between slices).
    p.kind = 0;
    p.rw = 4;
    // Launches with workgroups to spare take 512-row panels (fewer, longer
    // lived workgroups, each table build shared by twice the rows) when the
    // last panel wastes at most an eighth of its rows and the launch still
    // has >= 2048 workgroups: +1-2% per shape on the 1B headline launches.
    {
      const int64_t panels8 = (n + 511) / 512;
      if (panels8 * 512 * 8 <= n * 9 && panels8 * count >= 2048) p.rw = 8;
    }
    p.kw = 1;
    const int64_t wg256 = (n + kLutThreads - 1) / kLutThreads * count;
    p.rows_per_thread = wg256 >= 4096 ? SHERRY_LUT_ROWS : 1;
    p.panels = (n + 64 * p.rw * p.rows_per_thread - 1) / (64 * p.rw * p.rows_per_thread);
    int64_t split = 1;
    while (p.panels * count * split * 2 <= SHERRY_GEMV_SPLIT_TARGET && groups % (split * 2) == 0) split *= 2;
    if (split > 1) {
      static const int cand[4][2] = {{1, 16}, {2, 8}, {4, 4}, {4, 2}};
      int64_t best_waves = 0;
      for (int i = 0; i < 4; ++i) {
        const int rw = cand[i][0], kw = cand[i][1];
        const int win_max = 16 / kw < 4 ? 16 / kw : 4;
        if (groups % kw != 0 || nsb / kw > win_max) continue;  // one window per slice
        const int64_t waves = (n + 64 * rw - 1) / (64 * rw) * count * rw * kw;
        if (waves > best_waves) {
          best_waves = waves;
          p.rw = rw;
          p.kw = kw;
        }
      }
      if (p.kw > 1) {
        split = 1;
        p.rows_per_thread = 1;
        p.panels = (n + 64 * p.rw - 1) / (64 * p.rw);
      }
    }
    if (split > 1 && p.kw == 1) {
      // Across workgroups the split need not be a power of two: take the
      // largest divisor of the groups that stays within the target and leaves
      // every split whole 4-superblock windows (the 3B launches: q / o and
      // k / v split 6 rather than 4 and 8 with 1-2 superblock windows; the
      // K = 8192 single call 16 rather than 64 one-superblock splits): +4% on
      // the 3B batch-1 sweep, the `down` single call 7.2 -> 6.4 us.
      int64_t best = 0;
      for (int64_t d = 2; d <= groups && p.panels * count * d <= SHERRY_GEMV_SPLIT_TARGET; ++d)
        if (groups % d == 0 && (nsb / d) % 4 == 0) best = d;
      if (best > 0) split = best;
    }
    p.ksplit = (int)split;
    const int64_t per_slice = nsb / split / p.kw;
    int win = SHERRY_LUT_WIN_MAX < 4 ? SHERRY_LUT_WIN_MAX : 4;
    while (win > 1 && (per_slice % win != 0 || win * p.kw > 16)) win >>= 1;
    p.window_sbs = win;
    p.workspace_bytes = split > 1 ? (size_t)count * split * n * sizeof(float) : 0;
    return p;
  }
  // Batch 2..16: split K (in whole groups) across workgroups until the
  // launch has ~768 of them (3-5 per CU resident); a second kernel sums the
  // partials.
  p.kind = 1;
  p.rows_per_thread = 1;
  p.rw = p.kw = 1;
  p.panels = (n + 64 * kMfmaTiles - 1) / (64 * kMfmaTiles);
  const int64_t wgs = p.panels * count;
  int64_t split = 1;
  while (wgs * split * 2 <= SHERRY_GEMV_MFMA_SPLIT_TARGET && groups % (split * 2) == 0) split *= 2;
  p.ksplit = (int)split;
  p.window_sbs = 1;
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
