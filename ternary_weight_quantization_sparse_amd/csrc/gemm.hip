// Prefill product Y[m, n] = sum_k X[m, k] * T[n, k] * alpha(n, k) on bf16 MFMA.
//
// Method: "Sherry, Tequila and Fairies in Python", section 1.1 (SherryLinear:
// F.linear with the dequantized ternary weight); activations stay bf16 (same
// section, and the agihunt digest's limits paragraph).
//
// Tiling: one workgroup of 4 waves (2 x 2) per BM (m) x BN (n) output tile;
// a wave owns (BM/2) x (BN/2) as 16 x 16 tiles of v_mfma_f32_16x16x32_bf16
// with the weight tile as the A operand (MFMA row = n) and the activations as
// B (MFMA column = m), so each lane's four accumulators are four consecutive n
// of one output row: one 8-byte bf16 store per tile.
//
// K loop: stages of 64 (half a 128-weight superblock), double-buffered in
// LDS.  While the MFMAs of stage s run, the threads fetch stage s+1 into
// registers: X with dwordx4 loads, and the packed weight record of their row.
// After the MFMAs they store X to LDS and decode the weights: a byte of a
// nibble dword holds two consecutive blocks (8 consecutive k), and with their
// two adjacent sign bits it forms a 10-bit index into a 16 KB LDS table of
// ready-made 16-byte bf16 chunks {-1, 0, +1}; one ds_read_b128 + one
// ds_write_b128 decode 8 weights.  LDS rows are 128 bytes (64 bf16); 16-byte
// chunks are XOR-swizzled by (row & 7) so MFMA operand loads are
// conflict-free.
//
// Scales: per_group keeps an fp32 accumulator per group (over its 2 or more
// stages) and adds alpha(n, group) * acc_g to the output accumulator in fp32
// when the group ends; per_channel / per_tensor accumulate directly and scale
// once in the epilogue.
#include <type_traits>

#include "sherry_internal.h"

namespace sherry {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kStageK = 64;                 // k per LDS stage
constexpr int kRowBytes = kStageK * 2;      // one LDS row: 64 bf16
constexpr int kChunks = kRowBytes / 16;     // 8 chunks of 8 k per row

#ifndef SHERRY_GEMM_WAVES
#define SHERRY_GEMM_WAVES 8  // waves per workgroup for 256-row tiles (8: 2 per SIMD, 64 x 64 each)
#endif
#ifndef SHERRY_GEMM_SWZ
#define SHERRY_GEMM_SWZ 1  // 0: chunk ^ (row & 7); 1: chunk ^ ((row >> 1) & 7)
#endif
__device__ inline int swz_key(int row) { return SHERRY_GEMM_SWZ ? ((row >> 1) & 7) : (row & 7); }
__device__ inline int swz(int row, int ch) { return row * kRowBytes + ((ch ^ swz_key(row)) << 4); }

// bf16 patterns of one block (4 weights) from its 5-bit code.
__device__ inline uint2 decode_bf16(uint32_t code) {
  const uint32_t z = (code >> 2) & 3;
  const uint32_t neg0 = (code >> 4) & 1;
  const uint32_t neg1 = neg0 ^ (code & 1);
  const uint32_t neg2 = neg0 ^ ((code >> 1) & 1);
  uint32_t h[4];
  uint32_t rank = 0;
#pragma unroll
  for (uint32_t pos = 0; pos < 4; ++pos) {
    const uint32_t neg = rank == 0 ? neg0 : (rank == 1 ? neg1 : neg2);
    h[pos] = (pos == z) ? 0u : (neg ? 0xBF80u : 0x3F80u);
    rank += (pos == z) ? 0u : 1u;
  }
  return make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
}

template <int GRAN, int BM, int BN, int WAVES>
struct GemmCfg {
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int WAVES_N = 2, WAVES_M = WAVES / 2;  // wave grid (m x n)
  static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;  // wave tile (m, n)
  static constexpr int TM = WM / 16, TN = WN / 16;  // MFMA tiles per wave
  static constexpr int XLOADS = BM / 8 / WAVES;     // 1 KB X copies per wave per stage (8 rows each)
  static constexpr int ROWS_PER_WAVE = BN / WAVES;  // weight rows each wave copies and decodes
  static constexpr int THREADS_PER_ROW = THREADS / BN;
  static constexpr int CHUNKS_PER_THREAD = 8 / THREADS_PER_ROW;  // of the stage's 8 chunks per row
  static constexpr bool kGroup = GRAN == SHERRY_PER_GROUP;
  // copies per wave per stage: X pieces, nibble and sign records, and for
  // per_group the scales of the stage's group
  static constexpr int VM_PER_STAGE = XLOADS + 2 + (kGroup ? 1 : 0);
};

// s_waitcnt with only a vmcnt limit (expcnt / lgkmcnt left at their maxima).
template <int VM>
__device__ inline void wait_vmcnt() {
  static_assert(VM >= 0 && VM < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((VM & 15) | (7 << 4) | (15 << 8) | ((VM >> 4) << 14));
}

// Direct global -> LDS copy: lane l of the wave writes lds_wave_base + size*l
// (the LDS base is wave-uniform; inactive lanes write nothing).
typedef __attribute__((address_space(3))) void lds_void;
// Word 3 of a raw buffer resource on gfx9-class parts: 32-bit data format
// (a zero format would make every access read zero), no swizzle, no stride.
constexpr int kBufferWord3 = 0x00020000;
__device__ inline void g2l_16(const void* g, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(const_cast<void*>(g), (lds_void*)lds_wave_base, 16, 0, 0);
}
__device__ inline void g2l_4(const void* g, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(const_cast<void*>(g), (lds_void*)lds_wave_base, 4, 0, 0);
}

// Workgroup barrier that orders LDS only: this wave's LDS reads and writes
// are complete (lgkmcnt 0) before it arrives.  Unlike __syncthreads it does
// not wait for vector-memory operations, so direct copies for later stages
// stay in flight; their completion is waited for explicitly (vmcnt) before
// the barrier that publishes them.  The memory clobber keeps the compiler
// from moving LDS accesses across it.
__device__ inline void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
  asm volatile("s_barrier" ::: "memory");
}

template <int J>
using Slot = std::integral_constant<int, J>;

template <int GRAN, int BM, int BN, int WAVES>
__global__ __launch_bounds__(64 * WAVES, 1) void gemm_kernel(const uint8_t* __restrict__ packed,
                                                      const float* __restrict__ alpha,
                                                      const uint16_t* __restrict__ x,
                                                      uint16_t* __restrict__ y, int64_t n, int64_t k,
                                                      int64_t m, int group_sbs, int tiles_m, int tiles_n) {
  using C = GemmCfg<GRAN, BM, BN, WAVES>;
  static_assert(BN == 128, "the record copies and the decode assume 128 weight rows");
  // record slot: nibble records + sign dwords of one superblock (+ per_group:
  // the scales of its group)
  constexpr int kAlphaOff = BN * 16 + BN * 4;
  constexpr int kRecBytes = kAlphaOff + (C::kGroup ? BN * 4 : 0);
  // Three-deep rings, one __shared__ object per slot: the compiler's wait
  // insertion then knows an LDS read of one slot never aliases the direct
  // copies in flight into another.
  __shared__ __attribute__((aligned(16))) char xs0[BM * kRowBytes], xs1[BM * kRowBytes], xs2[BM * kRowBytes];
  __shared__ __attribute__((aligned(16))) char ws0[BN * kRowBytes], ws1[BN * kRowBytes], ws2[BN * kRowBytes];
  __shared__ __attribute__((aligned(16))) char rc0[kRecBytes], rc1[kRecBytes], rc2[kRecBytes];
  __shared__ __attribute__((aligned(16))) uint2 dtab[32];

  auto XS = [&](auto J) -> char* {
    if constexpr (decltype(J)::value == 0) return xs0; else if constexpr (decltype(J)::value == 1) return xs1; else return xs2;
  };
  auto WS = [&](auto J) -> char* {
    if constexpr (decltype(J)::value == 0) return ws0; else if constexpr (decltype(J)::value == 1) return ws1; else return ws2;
  };
  auto RC = [&](auto J) -> char* {
    if constexpr (decltype(J)::value == 0) return rc0; else if constexpr (decltype(J)::value == 1) return rc1; else return rc2;
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave % C::WAVES_M, wn = wave / C::WAVES_M;
  const int r = lane & 15, q = lane >> 4;

  // XCD-aware tile order: consecutive workgroup ids land on different XCDs;
  // give each XCD a contiguous range of tiles (m-major) so its L2 shares X.
  const int tiles = tiles_m * tiles_n;
  int bid = blockIdx.x;
  if ((tiles & 7) == 0) bid = (bid & 7) * (tiles >> 3) + (bid >> 3);
  const int tm = bid / tiles_n, tn = bid % tiles_n;
  const int64_t m0 = (int64_t)tm * BM;
  const int64_t n0 = (int64_t)tn * BN;

  if (tid < 32) dtab[tid] = decode_bf16(tid);

  const int64_t nsb = k / kSuperblock;
  const int stages = (int)(nsb * 2);
  const uint8_t* __restrict__ nib_plane = packed;
  const uint8_t* __restrict__ sgn_plane = packed + nibble_plane_bytes(n, k);

  // this thread decodes weight row tid / THREADS_PER_ROW; wave w owns rows
  // ROWS_PER_WAVE*w .. +ROWS_PER_WAVE-1, which it also copies
  const int wrow = tid / C::THREADS_PER_ROW;
  const int wsub = tid % C::THREADS_PER_ROW;

  // Direct copies of stage st into ring slot J.  X: wave w copies rows
  // [w*BM/WAVES, (w+1)*BM/WAVES) in pieces of 8 rows; lane l -> physical chunk
  // l%8 of row l/8, which holds logical chunk (l%8) ^ swz_key(row).  Records:
  // each wave copies the rows it decodes (the other lanes idle).
  // X copies are buffer loads: the per-stage base is wave-uniform (a buffer
  // resource in SGPRs), the lane offset a 32-bit VGPR, and rows past m fall
  // outside the resource's range, so they read zeros (the host keeps
  // (m + BM) * k * 2 below 2^31).  The lane part of the offset only depends
  // on the parity of the 8-row piece (the swizzle key has period 16 rows).
  static_assert(C::XLOADS % 2 == 0, "pieces of one wave alternate parity");
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  uint32_t xlane[2];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int prow = p * 8 + (lane >> 3);
    xlane[p] = (uint32_t)((lane >> 3) * k * 2) + (uint32_t)((((lane & 7) ^ swz_key(prow))) * 16);
  }
  const uint32_t xbytes = (uint32_t)(m * k * 2);
  int64_t rrow = n0 + wave * C::ROWS_PER_WAVE + (lane % C::ROWS_PER_WAVE);
  rrow = rrow < n ? rrow : n - 1;
  const uint32_t nrow_off = (uint32_t)(rrow * 16), srow_off = (uint32_t)(rrow * 4);
  auto issue = [&](auto J, int st) {
    const uint32_t sbyte = (uint32_t)st * (kStageK * 2);
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(reinterpret_cast<const char*>(x)) + sbyte, (short)0, (int)(xbytes - sbyte), kBufferWord3);
    char* xb = XS(J);
#pragma unroll
    for (int i = 0; i < C::XLOADS; ++i) {
      const int piece = wave_u * C::XLOADS + i;
      const uint32_t voff = xlane[i & 1] + (uint32_t)((m0 + piece * 8) * k * 2);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_void*)(xb + piece * 1024), 16, voff, 0, 0, 0);
    }
    char* rb = RC(J);
    const int64_t g = st >> 1;
    if (lane < C::ROWS_PER_WAVE) {
      g2l_16(nib_plane + g * n * 16 + nrow_off, rb + wave * C::ROWS_PER_WAVE * 16);
      g2l_4(sgn_plane + g * n * 4 + srow_off, rb + BN * 16 + wave * C::ROWS_PER_WAVE * 4);
      if constexpr (C::kGroup)
        g2l_4(alpha + (g / group_sbs) * n + (srow_off >> 2), rb + kAlphaOff + wave * C::ROWS_PER_WAVE * 4);
    }
  };
  // Decode stage st from record slot J into the bf16 tile slot J.  Byte cb
  // of nibble dword d holds blocks 8cb + 2d and 8cb + 2d + 1 = the 8 weights
  // of chunk d + 4cb; stage st covers cb = 2*(st&1) + {0, 1}, i.e. 8 chunks
  // per row, CHUNKS_PER_THREAD of them per thread.
  auto decode = [&](auto J, int st) {
    const char* rb = RC(J);
    char* wb = WS(J);
    const uint4 nr = *reinterpret_cast<const uint4*>(rb + wrow * 16);
    const uint32_t sg = *reinterpret_cast<const uint32_t*>(rb + BN * 16 + wrow * 4);
    const uint32_t nd[4] = {nr.x, nr.y, nr.z, nr.w};
#pragma unroll
    for (int cc = 0; cc < C::CHUNKS_PER_THREAD; ++cc) {
      const int lc = wsub * C::CHUNKS_PER_THREAD + cc;  // 0..7: (cb & 1, d)
      const int d = lc & 3;
      const int cb = 2 * (st & 1) + (lc >> 2);
      const uint32_t byte = __builtin_amdgcn_ubfe(nd[d], 8 * cb, 8);
      const uint32_t s2 = __builtin_amdgcn_ubfe(sg, 2 * d + 8 * cb, 2);
      const uint2 lo = dtab[(byte & 15u) | ((s2 & 1u) << 4)];
      const uint2 hi = dtab[(byte >> 4) | ((s2 >> 1) << 4)];
      *reinterpret_cast<u32x4*>(wb + swz(wrow, lc)) = u32x4{lo.x, lo.y, hi.x, hi.y};
    }
  };

  f32x4 acc[C::TN][C::TM];
  f32x4 accg[C::kGroup ? C::TN : 1][C::kGroup ? C::TM : 1];
#pragma unroll
  for (int i = 0; i < C::TN; ++i)
#pragma unroll
    for (int j = 0; j < C::TM; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  int gpos = 0;  // superblocks done in the current group (its first stage zeroes accg)

  // One stage: stage st sits in slot J = st % 3.
  auto stage = [&](auto J, int st) {
    constexpr int j = decltype(J)::value;
    constexpr int j1 = (j + 1) % 3, j2 = (j + 2) % 3;
    const bool group_end = C::kGroup && (st & 1) == 1 && gpos + 1 == group_sbs;
    // copies two stages ahead (slot j2 was consumed in the previous stage)
    const bool ahead = st + 2 < stages;
    if (ahead) issue(Slot<j2>{}, st + 2);

    const char* xb = XS(J);
    const char* wb = WS(J);
    // per_group: the first k-step of a group starts its accumulators from 0
    auto mma = [&](auto zero_c) {
#pragma unroll
      for (int kk = 0; kk < kStageK / 32; ++kk) {
        const int ch = kk * 4 + q;
        bf16x8 a[C::TN], b[C::TM];
#pragma unroll
        for (int i = 0; i < C::TN; ++i)
          a[i] = *reinterpret_cast<const bf16x8*>(wb + swz(wn * C::WN + i * 16 + r, ch));
#pragma unroll
        for (int jj = 0; jj < C::TM; ++jj)
          b[jj] = *reinterpret_cast<const bf16x8*>(xb + swz(wm * C::WM + jj * 16 + r, ch));
#pragma unroll
        for (int i = 0; i < C::TN; ++i)
#pragma unroll
          for (int jj = 0; jj < C::TM; ++jj) {
            if constexpr (C::kGroup) {
              const f32x4 c_in = (decltype(zero_c)::value && kk == 0) ? f32x4{0.f, 0.f, 0.f, 0.f} : accg[i][jj];
              accg[i][jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[jj], c_in, 0, 0, 0);
            } else {
              acc[i][jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[jj], acc[i][jj], 0, 0, 0);
            }
          }
      }
    };
    if (C::kGroup && (st & 1) == 0 && gpos == 0) {
      mma(std::true_type{});
    } else {
      mma(std::false_type{});
    }

    if constexpr (C::kGroup) {
      if ((st & 1) == 1) {
        if (group_end) {
          // the group's scales came with this stage's record copy
          const char* rb = RC(J);
#pragma unroll
          for (int i = 0; i < C::TN; ++i) {
            const f32x4 av = *reinterpret_cast<const f32x4*>(rb + kAlphaOff + (wn * C::WN + i * 16 + 4 * q) * 4);
#pragma unroll
            for (int jj = 0; jj < C::TM; ++jj) {
#pragma unroll
              for (int e = 0; e < 4; ++e) acc[i][jj][e] += av[e] * accg[i][jj][e];
            }
          }
          gpos = 0;
        } else {
          ++gpos;
        }
      }
    }

    if (st + 1 < stages) {
      // this wave's copies of stage st+1 (issued one stage ago) have landed;
      // only this stage's copies may still be in flight
      if (ahead) wait_vmcnt<C::VM_PER_STAGE>(); else wait_vmcnt<0>();
      decode(Slot<j1>{}, st + 1);
    }
    lds_barrier();
  };

  // prologue: stages 0 and 1 copied, stage 0 decoded
  issue(Slot<0>{}, 0);
  if (stages > 1) issue(Slot<1>{}, 1);
  if (stages > 1) wait_vmcnt<C::VM_PER_STAGE>(); else wait_vmcnt<0>();
  lds_barrier();  // decode table written
  decode(Slot<0>{}, 0);
  lds_barrier();

  for (int st = 0; st < stages; st += 3) {
    stage(Slot<0>{}, st);
    if (st + 1 < stages) stage(Slot<1>{}, st + 1);
    if (st + 2 < stages) stage(Slot<2>{}, st + 2);
  }

  // epilogue: lane holds Y[m0 + wm*WM + 16j + r][n0 + wn*WN + 16i + 4q + e]
#pragma unroll
  for (int i = 0; i < C::TN; ++i) {
    const int64_t gn0 = n0 + wn * C::WN + i * 16 + 4 * q;
    float sc[4] = {1.f, 1.f, 1.f, 1.f};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if constexpr (GRAN == SHERRY_PER_CHANNEL) sc[e] = (gn0 + e < n) ? alpha[gn0 + e] : 0.f;
      if constexpr (GRAN == SHERRY_PER_TENSOR) sc[e] = alpha[0];
    }
#pragma unroll
    for (int jj = 0; jj < C::TM; ++jj) {
      const int64_t gm = m0 + wm * C::WM + jj * 16 + r;
      if (gm >= m) continue;
      uint16_t h[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) h[e] = f32_to_bf16_rne(acc[i][jj][e] * sc[e]);
      uint16_t* dst = y + gm * n + gn0;
      if (gn0 + 3 < n && (n & 3) == 0) {
        *reinterpret_cast<uint2*>(dst) = make_uint2(h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16));
      } else {
        for (int e = 0; e < 4; ++e)
          if (gn0 + e < n) dst[e] = h[e];
      }
    }
  }
}

template <int GRAN, int BM, int WAVES>
hipError_t launch_t(int64_t n, int64_t k, int group_sbs, const uint8_t* packed, const float* alpha,
                    const uint16_t* x, int64_t m, uint16_t* y, hipStream_t s) {
  constexpr int BN = 128;
  // one launch covers at most `chunk` rows of X so that its buffer offsets,
  // including the tail tile's rows past the end, stay below 2^31 bytes
  const int64_t chunk = ((((int64_t)1 << 31) / (2 * k) - BM) / BM) * BM;
  if (chunk < BM) return hipErrorInvalidValue;
  const int tiles_n = (int)((n + BN - 1) / BN);
  for (int64_t r0 = 0; r0 < m; r0 += chunk) {
    const int64_t mc = m - r0 < chunk ? m - r0 : chunk;
    const int tiles_m = (int)((mc + BM - 1) / BM);
    hipLaunchKernelGGL((gemm_kernel<GRAN, BM, BN, WAVES>), dim3((unsigned)(tiles_m * tiles_n)), dim3(64 * WAVES), 0,
                       s, packed, alpha, x + r0 * k, y + r0 * n, n, k, mc, group_sbs, tiles_m, tiles_n);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int GRAN>
hipError_t launch_g(const GemmPlan& p, int64_t n, int64_t k, int group_sbs, const uint8_t* packed,
                    const float* alpha, const uint16_t* x, int64_t m, uint16_t* y, hipStream_t s) {
  if (p.tile_m == 256) return launch_t<GRAN, 256, SHERRY_GEMM_WAVES>(n, k, group_sbs, packed, alpha, x, m, y, s);
  return launch_t<GRAN, 128, 4>(n, k, group_sbs, packed, alpha, x, m, y, s);
}

}  // namespace

GemmPlan plan_gemm(int64_t n, int64_t k, int gran, int group_size, int64_t m) {
  (void)k; (void)group_size;
  GemmPlan p{};
  p.tile_n = 128;
  // 256-row tiles (8 waves of 64 x 64) once they still give >= 2 tiles per CU
  const int64_t big = ((m + 255) / 256) * ((n + 127) / 128);
  p.tile_m = (big >= 512 && (gran != SHERRY_PER_GROUP || SHERRY_GEMM_WAVES == 8)) ? 256 : 128;
  p.workspace_bytes = 0;
  return p;
}

hipError_t launch_gemm(const GemmPlan& p, int64_t n, int64_t k, int gran, int group_size,
                       const uint8_t* packed, const float* alpha, const uint16_t* x, int64_t m,
                       uint16_t* y, hipStream_t s) {
  const int group_sbs = gran == SHERRY_PER_GROUP ? group_size / kSuperblock : 1;
  if (gran == SHERRY_PER_GROUP) return launch_g<SHERRY_PER_GROUP>(p, n, k, group_sbs, packed, alpha, x, m, y, s);
  if (gran == SHERRY_PER_CHANNEL) return launch_g<SHERRY_PER_CHANNEL>(p, n, k, group_sbs, packed, alpha, x, m, y, s);
  return launch_g<SHERRY_PER_TENSOR>(p, n, k, group_sbs, packed, alpha, x, m, y, s);
}

}  // namespace sherry
