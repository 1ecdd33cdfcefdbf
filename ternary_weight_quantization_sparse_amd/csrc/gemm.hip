// Prefill product Y[m, n] = sum_k X[m, k] * T[n, k] * alpha(n, k) on bf16 MFMA.
//
// Method: "Sherry, Tequila and Fairies in Python", section 1.1 (SherryLinear:
// F.linear with the dequantized ternary weight; activations stay bf16 per the
// same section and the agihunt digest's limits paragraph).
//
// Tiling: one workgroup (4 waves, 2 x 2) per 128 (n) x 128 (m) output tile;
// each wave owns 64 x 64 = 4 x 4 tiles of v_mfma_f32_16x16x32_bf16.  The K
// loop steps one superblock (128 = one scale group at G = 128) at a time:
//   1. X[m0:m0+128, k0:k0+128] (bf16) is copied to LDS with dwordx4 loads;
//   2. the packed weights of rows n0:n0+128 are decoded to bf16 {-1, 0, +1}
//      and written to LDS;
//   3. 4 k-steps of 32 run 16 MFMAs each per wave into a per-group fp32
//      accumulator, which is then scaled by alpha(n, group) and added to the
//      output accumulator in fp32 (per_group); per_channel / per_tensor
//      accumulate directly and scale once at the end.
// LDS rows are 256 bytes (128 bf16); 16-byte chunks are XOR-swizzled by the
// row index so the 16 rows read by one MFMA operand load hit distinct banks.
// The MFMA A operand is the weight tile (M index = n) and B the activations
// (N index = m), so each lane's four accumulators are four consecutive n of
// one output row m: one 8-byte bf16 store per tile.
#include "sherry_internal.h"

namespace sherry {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kTile = 128;
constexpr int kRowBytes = kTile * 2;  // one LDS row: 128 bf16

// Byte offset of 16-byte chunk `ch` (0..15) of LDS row `row`.
__device__ inline int swz(int row, int ch) { return row * kRowBytes + ((ch ^ (row & 15)) << 4); }

// bf16 patterns of one block (4 weights) from its 5-bit code: two dwords.
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

template <int GRAN>
__global__ __launch_bounds__(256) void gemm_kernel(const uint8_t* __restrict__ packed,
                                                   const float* __restrict__ alpha,
                                                   const uint16_t* __restrict__ x,
                                                   uint16_t* __restrict__ y, int64_t n, int64_t k,
                                                   int64_t m, int group_sbs) {
  __shared__ __attribute__((aligned(16))) char xs[kTile * kRowBytes];
  __shared__ __attribute__((aligned(16))) char ws[kTile * kRowBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wn = wave >> 1, wm = wave & 1;  // wave position in the 2 x 2 grid
  const int r = lane & 15, q = lane >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * kTile;
  const int64_t m0 = (int64_t)blockIdx.y * kTile;
  const int64_t nsb = k / kSuperblock;
  const uint32_t* __restrict__ nibw = reinterpret_cast<const uint32_t*>(packed);
  const uint32_t* __restrict__ sgn = reinterpret_cast<const uint32_t*>(packed + nibble_plane_bytes(n, k));

  f32x4 acc[4][4], accg[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
      accg[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

  int gpos = 0;
  for (int64_t g = 0; g < nsb; ++g) {
    __syncthreads();
    // 1. activations: 128 rows x 16 chunks of 16 B; thread -> 8 chunks
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int idx = it * 256 + tid;
      const int row = idx >> 4, ch = idx & 15;
      const int64_t gm = m0 + row;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (gm < m) v = *reinterpret_cast<const u32x4*>(x + gm * k + g * kSuperblock + ch * 8);
      *reinterpret_cast<u32x4*>(xs + swz(row, ch)) = v;
    }
    // 2. weights: thread -> (row tid/2, 16 blocks = 8 chunks)
    {
      const int row = tid >> 1, hb = tid & 1;
      const int64_t gn = n0 + row;
      uint32_t nd[4] = {0u, 0u, 0u, 0u};
      uint32_t sg = 0;
      if (gn < n) {
        const uint4 v = reinterpret_cast<const uint4*>(nibw)[g * n + gn];
        nd[0] = v.x; nd[1] = v.y; nd[2] = v.z; nd[3] = v.w;
        sg = sgn[g * n + gn];
      }
#pragma unroll
      for (int c2 = 0; c2 < 8; ++c2) {
        const int j0 = hb * 16 + 2 * c2;  // blocks j0, j0+1 -> chunk j0/2
        uint2 a = make_uint2(0u, 0u), b = make_uint2(0u, 0u);
        if (gn < n) {
          const uint32_t ja = j0, jb = j0 + 1;
          const uint32_t ca = (((nd[(ja & 7) >> 1] >> (4 * (ja & 1) + 8 * (ja >> 3))) & 15u)) | (((sg >> ja) & 1u) << 4);
          const uint32_t cb = (((nd[(jb & 7) >> 1] >> (4 * (jb & 1) + 8 * (jb >> 3))) & 15u)) | (((sg >> jb) & 1u) << 4);
          a = decode_bf16(ca);
          b = decode_bf16(cb);
        }
        const u32x4 v = {a.x, a.y, b.x, b.y};
        *reinterpret_cast<u32x4*>(ws + swz(row, j0 >> 1)) = v;
      }
    }
    __syncthreads();

    // 3. MFMA: 4 k-steps of 32
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int ch = kk * 4 + q;  // this lane's 8 k values
      bf16x8 a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        a[i] = *reinterpret_cast<const bf16x8*>(ws + swz(wn * 64 + i * 16 + r, ch));
#pragma unroll
      for (int j = 0; j < 4; ++j)
        b[j] = *reinterpret_cast<const bf16x8*>(xs + swz(wm * 64 + j * 16 + r, ch));
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if constexpr (GRAN == SHERRY_PER_GROUP) {
            accg[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], accg[i][j], 0, 0, 0);
          } else {
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
          }
        }
    }

    if constexpr (GRAN == SHERRY_PER_GROUP) {
      if (++gpos == group_sbs) {
        const int64_t gg = g / group_sbs;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          // accumulator element e of tile i is weight row n0 + wn*64 + 16i + 4q + e
          float av[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int64_t gn = n0 + wn * 64 + i * 16 + 4 * q + e;
            av[e] = gn < n ? alpha[gg * n + gn] : 0.f;
          }
#pragma unroll
          for (int j = 0; j < 4; ++j) {
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[i][j][e] += av[e] * accg[i][j][e];
            accg[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
          }
        }
        gpos = 0;
      }
    }
  }

  // epilogue: lane holds Y[m0 + wm*64 + 16j + r][n0 + wn*64 + 16i + 4q + e]
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t gn0 = n0 + wn * 64 + i * 16 + 4 * q;
    float sc[4] = {1.f, 1.f, 1.f, 1.f};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if constexpr (GRAN == SHERRY_PER_CHANNEL) sc[e] = (gn0 + e < n) ? alpha[gn0 + e] : 0.f;
      if constexpr (GRAN == SHERRY_PER_TENSOR) sc[e] = alpha[0];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t gm = m0 + wm * 64 + j * 16 + r;
      if (gm >= m) continue;
      uint16_t h[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) h[e] = f32_to_bf16_rne(acc[i][j][e] * sc[e]);
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

}  // namespace

GemmPlan plan_gemm(int64_t n, int64_t k, int gran, int group_size, int64_t m) {
  (void)n; (void)k; (void)gran; (void)group_size; (void)m;
  GemmPlan p{};
  p.tile_n = kTile;
  p.tile_m = kTile;
  p.workspace_bytes = 0;
  return p;
}

hipError_t launch_gemm(const GemmPlan& p, int64_t n, int64_t k, int gran, int group_size,
                       const uint8_t* packed, const float* alpha, const uint16_t* x, int64_t m,
                       uint16_t* y, hipStream_t s) {
  const dim3 grid((unsigned)((n + p.tile_n - 1) / p.tile_n), (unsigned)((m + p.tile_m - 1) / p.tile_m));
  const int group_sbs = gran == SHERRY_PER_GROUP ? group_size / kSuperblock : 1;
  if (gran == SHERRY_PER_GROUP) {
    hipLaunchKernelGGL(gemm_kernel<SHERRY_PER_GROUP>, grid, dim3(256), 0, s, packed, alpha, x, y, n, k, m, group_sbs);
  } else if (gran == SHERRY_PER_CHANNEL) {
    hipLaunchKernelGGL(gemm_kernel<SHERRY_PER_CHANNEL>, grid, dim3(256), 0, s, packed, alpha, x, y, n, k, m, group_sbs);
  } else {
    hipLaunchKernelGGL(gemm_kernel<SHERRY_PER_TENSOR>, grid, dim3(256), 0, s, packed, alpha, x, y, n, k, m, group_sbs);
  }
  return hipGetLastError();
}

}  // namespace sherry
