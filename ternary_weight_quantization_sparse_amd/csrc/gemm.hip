// Prefill product Y[m, n] = sum_k X[m, k] * T[n, k] * alpha(n, k) on bf16 MFMA.
//
// Method: "Sherry, Tequila and Fairies in Python", section 1.1 (SherryLinear:
// F.linear with the dequantized ternary weight); activations stay bf16 (same
// section, and the agihunt digest's limits paragraph).
//
// Tiling: a workgroup of 4 waves owns a 64 (m) x 128 (n) output tile; wave w
// owns all 64 m and the 32 n starting at 32w, as 4 x 2 tiles of
// v_mfma_f32_16x16x32_bf16 with the weights as the A operand (MFMA row = n)
// and the activations as B (MFMA column = m), so each lane's four
// accumulators are four consecutive n of one output row.  Three workgroups
// share a CU and run out of step, so one's copies and barrier waits overlap
// the others' MFMAs.  Launches with enough tiles to fill the GPU at two per
// CU use 64 x 256 tiles instead (4 x 4 MFMA tiles per wave: each activation
// fragment read from LDS feeds four MFMAs, not two).
//
// K loop: stages of 128 k (one superblock) in a two-slot ring.  The
// activation tile of a stage (64 rows x 256 bytes) is copied straight from
// global memory into LDS by buffer loads (no registers) one stage ahead;
// 16-byte chunks are XOR-swizzled so MFMA operand reads are conflict-free.
// The weights never sit in LDS as bf16: each wave copies the nibble and sign
// records of its 32 weight rows into the slot, reads its lane's two nibble
// and sign dwords into registers at the end of the previous stage, and
// decodes its own A operands right before the MFMAs: byte cb of nibble dword
// q holds the lookup nibbles of two consecutive blocks (8 consecutive k), and
// each nibble with its block's sign bit indexes a 32-entry LDS table of the
// block's 4 bf16 weights {-1, 0, +1}.  One barrier per stage publishes the
// copied tile; a stage of a whole superblock gives each wave 32 MFMAs between
// barriers (stages of 64 k with a three-slot ring, the same LDS, ran 11-28%
// slower).
//
// Scales: per_group keeps an fp32 accumulator set per group (the group's first
// MFMA starts from zero) and adds alpha(n, group) * acc_g to the output
// accumulators when the group ends; the group's scales ride along with the
// activation copies into a small LDS ring.  per_channel / per_tensor
// accumulate directly and scale once at the end.
//
// Split K: launches with few tiles split K into `splits` ranges of whole
// groups; each writes fp32 partial tiles to the workspace, and a second
// kernel sums them in split order (deterministic), scales and rounds to bf16.
#include <cmath>
#include <type_traits>

#include "sherry_internal.h"

namespace sherry {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kStageK = 128;                // k per LDS stage: one superblock
constexpr int kRowBytes = kStageK * 2;      // one LDS row: 64 bf16
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
#ifndef SHERRY_GEMM_WIDE_TILES
#define SHERRY_GEMM_WIDE_TILES 512  // 256-wide weight tiles once a launch has this many of them
#endif
constexpr int kMaxBM = 128;                 // largest activation tile (rows) the host chunking allows for
#ifndef SHERRY_GEMM_SPLIT_TARGET
#define SHERRY_GEMM_SPLIT_TARGET 512  // split K until a launch has this many workgroups
#endif
constexpr int kGemmTM = 4;                  // MFMA tiles per wave along m: 64-row tiles
#ifndef SHERRY_AR_BAND_M
#define SHERRY_AR_BAND_M 8  // Arenas: m-tiles per band of the tile order
#endif
constexpr int kArBandM = SHERRY_AR_BAND_M;

// Activation LDS rows are 256 bytes = 16 chunks of 16 bytes; chunk c of row r
// sits at physical chunk c ^ (r & 15).  An MFMA operand read (a quarter wave:
// 16 rows, one chunk) then touches every bank once.
__device__ inline int swz_key(int row) { return row & 15; }
__device__ inline int swz(int row, int ch) { return row * kRowBytes + ((ch ^ swz_key(row)) << 4); }

// TM = MFMA tiles per wave along m (4: 64-row tiles); TN = MFMA tiles per
// wave along n (2: 32 weight rows per wave, 128 per workgroup; 4: 64 and
// 256, twice the MFMAs per activation fragment read, for launches with
// enough tiles to fill the GPU at two workgroups per CU).
// AR: the Arenas training forward, which adds lambda * X W^T over the dense
// bf16 latent weight W in the same K loop.
// MERGE (Arenas, per_group): the dense product accumulates into the output
// accumulators, and each group's sum is folded in scaled by alpha / lambda;
// the epilogue multiplies by lambda.  One accumulator set fewer, so the
// dense-weight operands fit in registers.  Needs lambda != 0 with alpha /
// lambda finite (the host picks it only then).
template <int GRAN, int TM, bool AR, int TN, bool MERGE = false>
struct GemmCfg {
  static constexpr bool kGroup = GRAN == SHERRY_PER_GROUP;
  static constexpr int kTN = TN;
  static constexpr int kWN = 16 * TN;              // weight rows per wave
  static constexpr int kBN = kWN * kWaves;         // weight rows per tile
  // Arenas dense-weight operands: loaded straight into registers one stage
  // ahead (no LDS tile, so two workgroups fit per CU), except for per_group
  // without MERGE, whose three accumulator sets leave no room: it copies a
  // dense tile into LDS like the activations.
  static constexpr bool kWReg = AR && (GRAN != SHERRY_PER_GROUP || MERGE);
  static constexpr int kWLoads = !AR ? 0
                               : kWReg ? TN * 4                                // 16-byte loads per lane per stage
                               : kBN * kRowBytes / 1024 / kWaves;              // 1 KB tile copies per wave per stage
  static constexpr int kTM = TM;
  static constexpr int kBM = 16 * TM;              // rows of X per tile
  static constexpr int kXLoads = kBM * kRowBytes / 1024 / kWaves;  // 1 KB activation copies per wave per stage
  // Per-wave record area of a ring slot: lane l < kWN copies the records of
  // weight row kWN wave + l: kWN nibble records (16 B), kWN sign dwords, and
  // for per_group kWN scales.
  static constexpr int kRecNib = 0, kRecSgn = kWN * 16, kRecAlpha = kRecSgn + kWN * 4;
  static constexpr int kRecWave = kRecAlpha + (kGroup ? kWN * 4 : 0);  // record bytes per wave
  // vector-memory operations per wave per stage: activation pieces, nibble
  // and sign records, and for per_group the scales
  static constexpr int VM_PER_STAGE = kXLoads + 2 + (kGroup ? 1 : 0) + kWLoads;
};

template <int J>
using Slot = std::integral_constant<int, J>;

// grid: x = tiles (tiles_m * tiles_n), y = K splits.  partial == nullptr:
// write bf16 Y; else write fp32 partial[split][m][n] (per_group already
// scaled, per_channel / per_tensor not yet; AR: fully scaled).
template <int GRAN, int TM, bool AR, int TN, bool MERGE>
__global__ __launch_bounds__(kThreads, AR ? (GRAN != SHERRY_PER_GROUP || MERGE ? 2 : 1) : (TN == 4 ? 2 : 3)) void gemm_kernel(const uint8_t* packed,
                                                     const float* __restrict__ alpha,
                                                     const uint16_t* __restrict__ x,
                                                     uint16_t* __restrict__ y, float* __restrict__ partial,
                                                     int64_t n, int64_t k, int64_t m, int group_sbs,
                                                     int tiles_m, int tiles_n, int sb_per_split,
                                                     const uint16_t* __restrict__ wd, float lam) {
  using C = GemmCfg<GRAN, TM, AR, TN, MERGE>;
  static_assert(!MERGE || (AR && GRAN == SHERRY_PER_GROUP), "MERGE is the per_group Arenas variant");
  constexpr int kTM = C::kTM, kBM = C::kBM, kXLoads = C::kXLoads, kRecWave = C::kRecWave;
  constexpr int kTN = C::kTN, kWN = C::kWN, kBN = C::kBN;
  constexpr int kRecNib = C::kRecNib, kRecSgn = C::kRecSgn, kRecAlpha = C::kRecAlpha;
  // one __shared__ object per ring slot: the compiler's wait insertion then
  // knows an LDS read of one slot never aliases the copies in flight into
  // another.  Slot: activation tile, records, and for AR the dense-weight tile.
  constexpr int kWOff = kBM * kRowBytes + kRecWave * kWaves;
  constexpr int kSlot = kWOff + ((AR && !C::kWReg) ? kBN * kRowBytes : 0);
  __shared__ __attribute__((aligned(16))) char sl0[kSlot], sl1[kSlot];
  __shared__ __attribute__((aligned(16))) uint2 dtab[32];

  auto XS = [&](auto J) -> char* {
    if constexpr (decltype(J)::value == 0) return sl0; else return sl1;
  };
  auto RC = [&](auto J) -> char* { return XS(J) + kBM * kRowBytes; };
  auto WT = [&](auto J) -> char* { return XS(J) + kWOff; };

  const float rlam = MERGE ? 1.0f / lam : 0.f;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, q = lane >> 4;

  // XCD-aware tile order: consecutive workgroup ids land on different XCDs;
  // give each XCD a contiguous range of tiles (m-major) so its L2 shares X.
  const int tiles = tiles_m * tiles_n;
  int bid = blockIdx.x;
  if ((tiles & 7) == 0) bid = (bid & 7) * (tiles >> 3) + (bid >> 3);
  int tm, tn;
  if constexpr (AR && kArBandM > 1) {
    // The Arenas variant also streams the bf16 latent weight: per n-tile
    // twice the bytes of an m-tile's activations.  Walking the range in bands
    // of kArBandM m-tiles, n-major inside a band, makes the tiles resident on
    // one XCD at a time a kArBandM x (64 / kArBandM) block that shares both
    // operands in L2, instead of one m-tile row that re-reads all of W.
    const int band = tiles_n * kArBandM;
    const int first = bid / band * kArBandM;
    const int rows = min(tiles_m - first, kArBandM);
    const int in = bid - first * tiles_n;
    tm = first + in % rows;
    tn = in / rows;
  } else {
    tm = bid / tiles_n;
    tn = bid % tiles_n;
  }
  const int64_t m0 = (int64_t)tm * kBM;
  const int64_t n0 = (int64_t)tn * kBN;
  const int kz = blockIdx.y;
  const int64_t sb0 = (int64_t)kz * sb_per_split;  // first superblock of this split
  const int stages = sb_per_split;

  if (tid < 32) dtab[tid] = decode_bf16(tid);

  // (no __restrict__ on the weight pointers: the record loads must stay where
  // they are issued, not float across the LDS barriers)
  const uint8_t* nib_plane = packed;
  const uint8_t* sgn_plane = packed + nibble_plane_bytes(n, k);

  // Activation copies: piece p (4 rows) of a stage goes to LDS bytes
  // [1024p, 1024p + 1024); lane l of the copy fetches physical chunk l%16 of
  // row 4p + l/16, i.e. logical chunk (l%16) ^ swz_key(row).  The key has a
  // period of 16 rows, so the lane part of the offset depends only on p % 4.
  // Rows past m fall outside the buffer resource's range and read zeros (the
  // host keeps (m + 128) * k * 2 below 2^31).
  constexpr int kRowsPerCopy = 1024 / kRowBytes;  // rows per 1 KB copy
  static_assert(kXLoads % 4 == 0 && 16 % kRowsPerCopy == 0, "piece phases repeat every 16 rows");
  uint32_t xlane[4];
#pragma unroll
  for (int p = 0; p < 4; ++p)
    xlane[p] = (uint32_t)((lane >> 4) * k * 2) +
               (uint32_t)(((lane & 15) ^ swz_key(p * kRowsPerCopy + (lane >> 4))) * 16);
  const uint32_t xbytes = (uint32_t)(m * k * 2);
  const uint32_t wbytes = AR ? (uint32_t)(n * k * 2) : 0u;

  // weight row whose records this lane copies: n0 + kWN wave + lane % kWN
  // (clamped rows feed only outputs that are not stored)
  int64_t crow = n0 + wave * kWN + (lane % kWN);
  crow = crow < n ? crow : n - 1;

  u32x4 wreg[C::kWReg ? 2 : 1][C::kWReg ? kTN : 1][4];  // dense-weight operands, one stage per slot
  auto issue = [&](auto J, int st) {
    const int64_t sb = sb0 + st;
    const uint32_t sbyte = (uint32_t)(sb * (kStageK * 2));
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(reinterpret_cast<const char*>(x)) + sbyte, (short)0, (int)(xbytes - sbyte), kBufferWord3);
    char* xb = XS(J);
#pragma unroll
    for (int i = 0; i < kXLoads; ++i) {
      const int piece = wave * kXLoads + i;
      const uint32_t voff = xlane[piece & 3] + (uint32_t)((m0 + piece * kRowsPerCopy) * k * 2);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_void*)(xb + piece * 1024), 16, voff, 0, 0, 0);
    }
    char* rb = RC(J) + wave * kRecWave;
    if (lane < kWN) {
      __builtin_amdgcn_global_load_lds(const_cast<uint8_t*>(nib_plane + sb * n * 16 + crow * 16),
                                       (lds_void*)(rb + kRecNib), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(const_cast<uint8_t*>(sgn_plane + sb * n * 4 + crow * 4),
                                       (lds_void*)(rb + kRecSgn), 4, 0, 0);
      if constexpr (C::kGroup)
        __builtin_amdgcn_global_load_lds(
            const_cast<float*>(alpha + (group_sbs == 1 ? sb : (int64_t)((int)sb / group_sbs)) * n + crow),
            (lds_void*)(rb + kRecAlpha), 4, 0, 0);
    }
    if constexpr (C::kWReg) {
      // dense-weight operands of this stage straight into registers: lane
      // (r, q) of tile i, k-step kk reads W[row][32 kk + 8q .. + 7] of this
      // superblock (rows past n are clamped: their outputs are not stored).
      // They land with the stage's copies (the wait at the end of the
      // previous stage).
#pragma unroll
      for (int i = 0; i < kTN; ++i) {
        int64_t row = n0 + wave * kWN + i * 16 + r;
        row = row < n ? row : n - 1;
        const uint16_t* src = wd + row * k + sb * kStageK + q * 8;
#pragma unroll
        for (int kk = 0; kk < kStageK / 32; ++kk)
          wreg[decltype(J)::value][i][kk] = *reinterpret_cast<const u32x4*>(src + kk * 32);
      }
    } else if constexpr (AR) {
      // dense-weight tile: rows n0 .. n0+127 of W, copied like X (rows past n
      // read zeros; the host keeps (n + 128) * k * 2 below 2^31)
      const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<char*>(reinterpret_cast<const char*>(wd)) + sbyte, (short)0, (int)(wbytes - sbyte), kBufferWord3);
      char* wb = WT(J);
#pragma unroll
      for (int i = 0; i < C::kWLoads; ++i) {
        const int piece = wave * C::kWLoads + i;
        const uint32_t voff = xlane[piece & 3] + (uint32_t)((n0 + piece * kRowsPerCopy) * k * 2);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (lds_void*)(wb + piece * 1024), 16, voff, 0, 0, 0);
      }
    }
  };

  // This lane's records of the next stage: nibble dword q and the sign dword
  // of rows r, 16 + r, ... of its wave's rows.  Each wave copies its own records, so
  // they are read right after its own wait for the copies, before the
  // barrier.  The reads are one asm block that waits for its own results:
  // the compiler cannot tell these LDS reads from ones that might overlap
  // copies still in flight and would otherwise wait for every copy.
  static_assert(kTN % 2 == 0, "the record reads below cover row tiles in pairs");
  uint32_t nd[kTN], sg[kTN];
  auto read_records = [&](auto J) {
    const uint32_t rb = (uint32_t)(size_t)(__attribute__((address_space(3))) char*)(RC(J) + wave * kRecWave);
#pragma unroll
    for (int pr = 0; pr < kTN / 2; ++pr) {
      // row tiles 2pr, 2pr + 1: 16 rows of 16 nibble bytes / 4 sign bytes each
      const uint32_t a_nib = rb + kRecNib + pr * 512 + r * 16 + q * 4;
      const uint32_t a_sgn = rb + kRecSgn + pr * 128 + r * 4;
      uint32_t n0v, n1v, s0v, s1v;
      asm volatile(
          "ds_read_b32 %0, %4\n"
          "ds_read_b32 %1, %4 offset:256\n"
          "ds_read_b32 %2, %5\n"
          "ds_read_b32 %3, %5 offset:64\n"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(n0v), "=&v"(n1v), "=&v"(s0v), "=&v"(s1v)
          : "v"(a_nib), "v"(a_sgn)
          : "memory");
      nd[2 * pr] = n0v; nd[2 * pr + 1] = n1v; sg[2 * pr] = s0v; sg[2 * pr + 1] = s1v;
    }
  };

  f32x4 acc[kTN][kTM];
  f32x4 accg[C::kGroup ? kTN : 1][C::kGroup ? kTM : 1];
  constexpr bool kAccD = AR && !MERGE;
  f32x4 accd[kAccD ? kTN : 1][kAccD ? kTM : 1];  // AR: X W^T over the dense weight
#pragma unroll
  for (int i = 0; i < kTN; ++i)
#pragma unroll
    for (int jj = 0; jj < kTM; ++jj) acc[i][jj] = f32x4{0.f, 0.f, 0.f, 0.f};
  if constexpr (AR) {
#pragma unroll
    for (int i = 0; i < kTN; ++i)
#pragma unroll
      for (int jj = 0; jj < kTM; ++jj) accd[i][jj] = f32x4{0.f, 0.f, 0.f, 0.f};  // (unused with MERGE)
  }
  int gpos = 0;  // superblocks done in the current group (its first stage zeroes accg)

  // One stage: stage st sits in slot J = st % 3.
  auto stage = [&](auto J, int st) {
    constexpr int j2 = (decltype(J)::value + 1) % 2;
    const bool group_end = C::kGroup && gpos + 1 == group_sbs;
    // copies one stage ahead into slot j2 (read in the previous stage, which
    // every wave has finished: it ended with a barrier).  Issued
    // unconditionally; past the end they repeat the last stage into a slot
    // nobody reads.
    issue(Slot<j2>{}, st + 1 < stages ? st + 1 : stages - 1);

    const char* xb = XS(J);
    const char* dt = reinterpret_cast<const char*>(dtab);
    // table offsets of the blocks this lane decodes, four per dword: byte cb
    // of off_lo / off_hi = blocks 8cb + 2q / 8cb + 2q + 1 of the superblock
    uint32_t off_lo[kTN], off_hi[kTN];
#pragma unroll
    for (int i = 0; i < kTN; ++i) {
      off_lo[i] = quad_offsets8(nd[i], sg[i], 2 * q);
      off_hi[i] = quad_offsets8(nd[i], sg[i], 2 * q + 1);
    }
    auto mma = [&](auto zero_c) {
#pragma unroll
      for (int kk = 0; kk < kStageK / 32; ++kk) {
        // byte cb of nibble dword q: blocks 8cb + 2q (low nibble) and
        // 8cb + 2q + 1 (high) = k 32cb + 8q .. +7 of the superblock, which is
        // chunk q of k-step kk of this stage
        const int cb = kk;
        bf16x8 a[kTN];
#pragma unroll
        for (int i = 0; i < kTN; ++i) {
          const uint2 wl = *reinterpret_cast<const uint2*>(dt + __builtin_amdgcn_ubfe(off_lo[i], 8 * cb, 8));
          const uint2 wh = *reinterpret_cast<const uint2*>(dt + __builtin_amdgcn_ubfe(off_hi[i], 8 * cb, 8));
          a[i] = __builtin_bit_cast(bf16x8, u32x4{wl.x, wl.y, wh.x, wh.y});
        }
        const int ch = kk * 4 + q;
        bf16x8 ad[AR ? kTN : 1];
        if constexpr (C::kWReg) {
#pragma unroll
          for (int i = 0; i < kTN; ++i) ad[i] = __builtin_bit_cast(bf16x8, wreg[decltype(J)::value][i][kk]);
        } else if constexpr (AR) {
#pragma unroll
          for (int i = 0; i < kTN; ++i)
            ad[i] = *reinterpret_cast<const bf16x8*>(WT(J) + swz(wave * kWN + i * 16 + r, ch));
        }
        bf16x8 bv[kTM];
#pragma unroll
        for (int jj = 0; jj < kTM; ++jj) bv[jj] = *reinterpret_cast<const bf16x8*>(xb + swz(jj * 16 + r, ch));
#pragma unroll
        for (int jj = 0; jj < kTM; ++jj) {
          const bf16x8 b = bv[jj];
#pragma unroll
          for (int i = 0; i < kTN; ++i) {
            if constexpr (C::kGroup) {
              const f32x4 c_in = (decltype(zero_c)::value && kk == 0) ? f32x4{0.f, 0.f, 0.f, 0.f} : accg[i][jj];
              accg[i][jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b, c_in, 0, 0, 0);
            } else {
              acc[i][jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b, acc[i][jj], 0, 0, 0);
            }
            if constexpr (MERGE) acc[i][jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ad[i], b, acc[i][jj], 0, 0, 0);
            else if constexpr (AR) accd[i][jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ad[i], b, accd[i][jj], 0, 0, 0);
          }
        }
      }
    };
    if (C::kGroup && gpos == 0) {
      mma(std::true_type{});
    } else {
      mma(std::false_type{});
    }

    if constexpr (C::kGroup) {
      {
        if (group_end) {
          // the group's scales came with this stage's copies and are still in
          // its slot (the copies in flight go to the other one): scales of
          // rows 4q .. 4q+3 of each row tile, read here rather than held in
          // registers through the stage (which made the 256-row tiles spill)
          const uint32_t rb = (uint32_t)(size_t)(__attribute__((address_space(3))) char*)(RC(J) + wave * kRecWave);
          f32x4 av[kTN];
#pragma unroll
          for (int pr = 0; pr < kTN / 2; ++pr) {
            f32x4 a0v, a1v;
            asm volatile(
                "ds_read_b128 %0, %2\n"
                "ds_read_b128 %1, %2 offset:64\n"
                "s_waitcnt lgkmcnt(0)"
                : "=&v"(a0v), "=&v"(a1v)
                : "v"(rb + kRecAlpha + pr * 128 + q * 16)
                : "memory");
            av[2 * pr] = a0v;
            av[2 * pr + 1] = a1v;
          }
#pragma unroll
          for (int i = 0; i < kTN; ++i) {
#pragma unroll
            for (int jj = 0; jj < kTM; ++jj) {
#pragma unroll
              for (int e = 0; e < 4; ++e) acc[i][jj][e] += (MERGE ? av[i][e] * rlam : av[i][e]) * accg[i][jj][e];
            }
          }
          gpos = 0;
        } else {
          ++gpos;
        }
      }
    }

    // this wave's copies of stage st+1 (issued at the start of this stage)
    // have landed; the barrier then publishes every wave's
    wait_vmcnt<0>();
    read_records(Slot<j2>{});
    lds_barrier();
  };

  // prologue: stage 0 landed
  issue(Slot<0>{}, 0);
  wait_vmcnt<0>();
  read_records(Slot<0>{});
  lds_barrier();  // decode table and stage 0 visible

  // (every early exit leaves the loop, so each path into a stage passes
  // through the stage before it)
  for (int st = 0;; st += 2) {
    stage(Slot<0>{}, st);
    if (st + 1 >= stages) break;
    stage(Slot<1>{}, st + 1);
    if (st + 2 >= stages) break;
  }
  wait_vmcnt<0>();  // the trailing repeat copies have landed before the wave ends

  // epilogue: lane holds Y[m0 + 16jj + r][n0 + 32 wave + 16i + 4q + e]
#pragma unroll
  for (int i = 0; i < kTN; ++i) {
    const int64_t gn0 = n0 + wave * kWN + i * 16 + 4 * q;
    const bool full4 = gn0 + 3 < n && (n & 3) == 0;
    // scale applied here: per_channel / per_tensor when writing Y, and always
    // for AR (its partials carry the finished value); per_group is scaled
    float sc[4] = {1.f, 1.f, 1.f, 1.f};
    if (partial == nullptr || AR) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if constexpr (GRAN == SHERRY_PER_CHANNEL) sc[e] = (gn0 + e < n) ? alpha[gn0 + e] : 0.f;
        if constexpr (GRAN == SHERRY_PER_TENSOR) sc[e] = alpha[0];
      }
    }
#pragma unroll
    for (int jj = 0; jj < kTM; ++jj) {
      const int64_t gm = m0 + jj * 16 + r;
      if (gm >= m) continue;
      f32x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if constexpr (MERGE) {
          v[e] = acc[i][jj][e] * lam;
        } else {
          v[e] = acc[i][jj][e] * sc[e];
          if constexpr (AR) v[e] += lam * accd[i][jj][e];
        }
      }
      if (partial != nullptr) {
        float* dst = partial + (int64_t)kz * m * n + gm * n + gn0;
        if (full4) {
          *reinterpret_cast<f32x4*>(dst) = v;
        } else {
          for (int e = 0; e < 4; ++e)
            if (gn0 + e < n) dst[e] = v[e];
        }
        continue;
      }
      uint16_t h[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) h[e] = f32_to_bf16_rne(v[e]);
      uint16_t* dst = y + gm * n + gn0;
      if (full4) {
        *reinterpret_cast<uint2*>(dst) = make_uint2(h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16));
      } else {
        for (int e = 0; e < 4; ++e)
          if (gn0 + e < n) dst[e] = h[e];
      }
    }
  }
}

// Y = bf16(scale(n) * sum over splits, in split order, of partial[z][m][n]).
template <int GRAN>
__global__ __launch_bounds__(256) void gemm_split_reduce(const float* __restrict__ partial,
                                                         const float* __restrict__ alpha,
                                                         uint16_t* __restrict__ y, int64_t mn, int64_t n,
                                                         int splits) {
  const int64_t i0 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (i0 >= mn) return;
  float s[4] = {0.f, 0.f, 0.f, 0.f};
  if ((mn & 3) == 0) {
    // every split's load first (splits <= 8), then the adds in split order
    f32x4 v[8];
#pragma unroll
    for (int z = 0; z < 8; ++z)
      if (z < splits) v[z] = *reinterpret_cast<const f32x4*>(partial + z * mn + i0);
#pragma unroll
    for (int z = 0; z < 8; ++z)
      if (z < splits)
#pragma unroll
        for (int e = 0; e < 4; ++e) s[e] += v[z][e];
  } else {
    for (int z = 0; z < splits; ++z)
      for (int e = 0; e < 4; ++e)
        if (i0 + e < mn) s[e] += partial[z * mn + i0 + e];
  }
  uint16_t h[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float sc = 1.f;
    if constexpr (GRAN == SHERRY_PER_CHANNEL) sc = (i0 + e < mn) ? alpha[(i0 + e) % n] : 0.f;
    if constexpr (GRAN == SHERRY_PER_TENSOR) sc = alpha[0];
    h[e] = f32_to_bf16_rne(s[e] * sc);
  }
  if ((mn & 3) == 0) {
    *reinterpret_cast<uint2*>(y + i0) = make_uint2(h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16));
  } else {
    for (int e = 0; e < 4; ++e)
      if (i0 + e < mn) y[i0 + e] = h[e];
  }
}

// Rows of X per launch: buffer offsets, including the tail tile's rows past
// the end, stay below 2^31 bytes.
int64_t gemm_chunk_rows(int64_t k) { return ((((int64_t)1 << 31) / (2 * k) - kMaxBM) / kMaxBM) * kMaxBM; }

template <int GRAN, int TM, bool AR, int TN, bool MERGE = false>
hipError_t launch_g(const GemmPlan& p, int64_t n, int64_t k, int group_sbs, const uint8_t* packed,
                    const float* alpha, const uint16_t* x, int64_t m, uint16_t* y, float* ws,
                    const uint16_t* wd, float lam, hipStream_t s) {
  constexpr int kBM = GemmCfg<GRAN, TM, AR, TN, MERGE>::kBM, kBN = GemmCfg<GRAN, TM, AR, TN, MERGE>::kBN;
  const int64_t chunk = gemm_chunk_rows(k);
  if (chunk < kMaxBM) return hipErrorInvalidValue;
  const int tiles_n = (int)((n + kBN - 1) / kBN);
  const int64_t nsb = k / kSuperblock;
  const int splits = p.splits;
  if (splits < 1 || splits > 8) return hipErrorInvalidValue;  // the reducer holds up to 8 partials
  const int sb_per_split = (int)(nsb / splits);
  for (int64_t r0 = 0; r0 < m; r0 += chunk) {
    const int64_t mc = m - r0 < chunk ? m - r0 : chunk;
    const int tiles_m = (int)((mc + kBM - 1) / kBM);
    hipLaunchKernelGGL((gemm_kernel<GRAN, TM, AR, TN, MERGE>), dim3((unsigned)(tiles_m * tiles_n), (unsigned)splits),
                       dim3(kThreads), 0, s, packed, alpha, x + r0 * k, y + r0 * n, splits > 1 ? ws : nullptr, n, k,
                       mc, group_sbs, tiles_m, tiles_n, sb_per_split, wd, lam);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (splits > 1) {
      const int64_t mn = mc * n;
      const int64_t threads = (mn + 3) / 4;
      // AR partials are already scaled: sum them with the scale-free reducer
      hipLaunchKernelGGL((gemm_split_reduce<AR ? SHERRY_PER_GROUP : GRAN>), dim3((unsigned)((threads + 255) / 256)),
                         dim3(256), 0, s, ws, alpha, y + r0 * n, mn, n, splits);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

}  // namespace

// Tile width and splits of K.  Launches with at least SHERRY_GEMM_WIDE_TILES
// tiles 256 weight rows wide (two per CU fill the GPU) use them: each
// activation fragment read from LDS then feeds twice the MFMAs.  Others use
// 128-row tiles and split K for launches with few tiles: the smallest power
// of two (at most 8) that brings the launch to 512 workgroups (two per CU),
// over whole groups and at least two superblocks per split.  Measured on the
// LLaMA-3.2-1B shapes at M = 512 and 2048, fuller launches gain nothing from
// splitting and deeper splits lose to their shorter K loops and partial
// traffic.  The Arenas forward (`wide` false) keeps 128-row tiles: its dense
// weight operands, held in registers a stage ahead, leave no room for twice
// as many weight rows per wave.
GemmPlan plan_gemm(int64_t n, int64_t k, int gran, int group_size, int64_t m, bool wide) {
  GemmPlan p{};
  p.tile_m = GemmCfg<SHERRY_PER_GROUP, kGemmTM, false, 2>::kBM;
  p.splits = 1;
  const int64_t nsb = k / kSuperblock;
  const int64_t group_sbs = gran == SHERRY_PER_GROUP ? group_size / kSuperblock : 1;
  const int64_t chunk = gemm_chunk_rows(k);
  const int64_t mc = chunk > 0 && m > chunk ? chunk : m;
  const int64_t tiles_m = (mc + p.tile_m - 1) / p.tile_m;
  if (wide && tiles_m * ((n + 255) / 256) >= SHERRY_GEMM_WIDE_TILES) {
    p.tile_n = 256;
    p.workspace_bytes = 0;
    return p;
  }
  p.tile_n = 128;
  const int64_t tiles = tiles_m * ((n + p.tile_n - 1) / p.tile_n);
  auto valid = [&](int64_t s) { return nsb % s == 0 && (nsb / s) % group_sbs == 0 && nsb / s >= 2; };
  while (tiles * p.splits < SHERRY_GEMM_SPLIT_TARGET && p.splits < 8 && valid(2 * p.splits)) p.splits *= 2;
  p.workspace_bytes = p.splits > 1 ? (size_t)p.splits * (size_t)mc * (size_t)n * sizeof(float) : 0;
  return p;
}

hipError_t launch_gemm(const GemmPlan& p, int64_t n, int64_t k, int gran, int group_size,
                       const uint8_t* packed, const float* alpha, const uint16_t* x, int64_t m,
                       uint16_t* y, float* ws, hipStream_t s) {
  const int group_sbs = gran == SHERRY_PER_GROUP ? group_size / kSuperblock : 1;
#define SHERRY_GEMM_LAUNCH(G, TN) \
  return launch_g<G, kGemmTM, false, TN>(p, n, k, group_sbs, packed, alpha, x, m, y, ws, nullptr, 0.f, s)
  if (p.tile_n == 256) {
    if (gran == SHERRY_PER_GROUP) SHERRY_GEMM_LAUNCH(SHERRY_PER_GROUP, 4);
    if (gran == SHERRY_PER_CHANNEL) SHERRY_GEMM_LAUNCH(SHERRY_PER_CHANNEL, 4);
    SHERRY_GEMM_LAUNCH(SHERRY_PER_TENSOR, 4);
  }
  if (gran == SHERRY_PER_GROUP) SHERRY_GEMM_LAUNCH(SHERRY_PER_GROUP, 2);
  if (gran == SHERRY_PER_CHANNEL) SHERRY_GEMM_LAUNCH(SHERRY_PER_CHANNEL, 2);
  SHERRY_GEMM_LAUNCH(SHERRY_PER_TENSOR, 2);
#undef SHERRY_GEMM_LAUNCH
}

hipError_t launch_arenas_gemm(const GemmPlan& p, int64_t n, int64_t k, int gran, int group_size,
                              const uint8_t* packed, const float* alpha, const uint16_t* wd, float lam,
                              const uint16_t* x, int64_t m, uint16_t* y, float* ws, hipStream_t s) {
  if (p.tile_n != 128) return hipErrorInvalidValue;
  const int group_sbs = gran == SHERRY_PER_GROUP ? group_size / kSuperblock : 1;
  if (gran == SHERRY_PER_GROUP) {
    // the merged-accumulator kernel scales each group by alpha / lambda: used
    // when 1 / lambda is comfortably finite (scales are means of |w|, far
    // below 2^60 / |1 / lambda| for any realistic weight)
    if (std::fabs(lam) >= 0x1p-60f && std::fabs(lam) <= 0x1p60f)
      return launch_g<SHERRY_PER_GROUP, kGemmTM, true, 2, true>(p, n, k, group_sbs, packed, alpha, x, m, y, ws, wd, lam,
                                                                s);
    return launch_g<SHERRY_PER_GROUP, kGemmTM, true, 2>(p, n, k, group_sbs, packed, alpha, x, m, y, ws, wd, lam, s);
  }
  if (gran == SHERRY_PER_CHANNEL)
    return launch_g<SHERRY_PER_CHANNEL, kGemmTM, true, 2>(p, n, k, group_sbs, packed, alpha, x, m, y, ws, wd, lam, s);
  return launch_g<SHERRY_PER_TENSOR, kGemmTM, true, 2>(p, n, k, group_sbs, packed, alpha, x, m, y, ws, wd, lam, s);
}

}  // namespace sherry
