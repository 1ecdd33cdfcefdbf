// Sparse-AbsMean quantize + 5-bit pack, and the scale reduction.
//
// Method: "Sherry: Hardware-Efficient 1.25-Bit Ternary Quantization via
// Fine-grained Sparsification" (agihunt digest, format paragraph): in every
// block of 4 weights along K the smallest |w| becomes 0, the other three keep
// their sign, and the scale is the mean |w| of the kept weights.  Granules and
// the nominal kept count L/4*3: "Sherry, Tequila and Fairies in Python",
// section 1.1 (_reshape_by_granularity, SherryNMQuant.forward).
//
// Mapping: one workgroup (4 waves) per tile of 64 rows x one superblock of
// 128 weights.  Each half-wave owns one (row, superblock) pair and each of its
// 32 lanes one block of 4 weights, so a wave's loads are two contiguous row
// segments (coalesced dwordx4 for fp32, dwordx2 for bf16).  The sign plane is
// a ballot, the nibble dwords an OR-reduction over lanes 1/8/16 apart, and the
// kept-|w| sum of the superblock a butterfly over XOR offsets 1..16 -- which
// is exactly the index-order pairwise tree (each level adds lanes 2i and
// 2i+1, and fp32 addition is commutative).
#include "sherry_internal.h"

namespace sherry {
namespace {

constexpr int kRowsPerTile = 64;
// Grid: x = superblock, y = 64-row tile, so consecutive workgroups read
// adjacent 128-weight spans of the same rows.
constexpr int kIters = kRowsPerTile / 8;  // 4 waves x 2 halves = 8 rows per iteration

template <bool BF16>
struct Block4 { float v[4]; };

template <bool BF16>
__device__ inline Block4<BF16> load_block(const void* w, int64_t row, int64_t k, int64_t col) {
  Block4<BF16> b;
  if constexpr (BF16) {
    const uint2 u = *reinterpret_cast<const uint2*>(
        reinterpret_cast<const uint16_t*>(w) + row * k + col);
    b.v[0] = __uint_as_float(u.x << 16);
    b.v[1] = __uint_as_float(u.x & 0xFFFF0000u);
    b.v[2] = __uint_as_float(u.y << 16);
    b.v[3] = __uint_as_float(u.y & 0xFFFF0000u);
  } else {
    const float4 f = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(w) + row * k + col);
    b.v[0] = f.x; b.v[1] = f.y; b.v[2] = f.z; b.v[3] = f.w;
  }
  return b;
}

// Quantize one block: returns the 5-bit code, and the kept-|w| sum of the
// block as a two-level pairwise tree ((a0 + a1) + (a2 + a3)) with the zeroed
// weight contributing +0.
__device__ inline uint32_t quantize_block(const float v[4], float& kept_sum) {
  const float a0 = fabsf(v[0]), a1 = fabsf(v[1]), a2 = fabsf(v[2]), a3 = fabsf(v[3]);
  // zero position: first index of the minimum magnitude (strict compares)
  uint32_t z = 0;
  float m = a0;
  if (a1 < m) { z = 1; m = a1; }
  if (a2 < m) { z = 2; m = a2; }
  if (a3 < m) { z = 3; }
  // positive-sign mask, bit i = (v[i] > 0)
  const uint32_t pos = (v[0] > 0.f ? 1u : 0u) | (v[1] > 0.f ? 2u : 0u) |
                       (v[2] > 0.f ? 4u : 0u) | (v[3] > 0.f ? 8u : 0u);
  // kept positions k0 < k1 < k2
  const uint32_t k0 = (z == 0) ? 1u : 0u;
  const uint32_t k1 = (z <= 1) ? 2u : 1u;
  const uint32_t k2 = (z <= 2) ? 3u : 2u;
  const uint32_t g0 = (pos >> k0) & 1u, g1 = (pos >> k1) & 1u, g2 = (pos >> k2) & 1u;
  const uint32_t s = g0 ^ 1u;        // 1 when the first kept weight is negative
  const uint32_t p0 = g1 ^ g0;       // second kept sign differs from the first
  const uint32_t p1 = g2 ^ g0;       // third kept sign differs from the first
  kept_sum = ((z == 0 ? 0.f : a0) + (z == 1 ? 0.f : a1)) +
             ((z == 2 ? 0.f : a2) + (z == 3 ? 0.f : a3));
  return (s << 4) | (z << 2) | (p1 << 1) | p0;
}

// DENSE = 0: write the packed planes (and the scale or the superblock sum).
// DENSE = SHERRY_F32 + 1 / SHERRY_BF16 + 1 (per_group G = 128 only): the
// fused fake-quant forward -- write T * alpha densely in fp32 (exact) or bf16
// (round to nearest even) and the scales, no planes.
template <bool BF16, int DENSE = 0>
__global__ __launch_bounds__(256) void quantize_pack_kernel(
    const void* __restrict__ w, int64_t n, int64_t k, uint8_t* __restrict__ packed,
    float* __restrict__ alpha_direct, float* __restrict__ sb_sums, void* __restrict__ dense = nullptr) {
  const int64_t nsb = k / kSuperblock;
  const int64_t g = blockIdx.x;
  const int64_t row0 = (int64_t)blockIdx.y * kRowsPerTile;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int half = lane >> 5;
  const int j = lane & 31;  // block index inside the superblock
  const int64_t col = g * kSuperblock + 4 * j;

  // Issue every load of this thread first (8 rows), then compute.
  Block4<BF16> blk[kIters];
#pragma unroll
  for (int it = 0; it < kIters; ++it) {
    const int64_t row = row0 + wave * (2 * kIters) + 2 * it + half;
    if (row < n) {
      blk[it] = load_block<BF16>(w, row, k, col);
    } else {
      blk[it].v[0] = blk[it].v[1] = blk[it].v[2] = blk[it].v[3] = 0.f;
    }
  }

  uint32_t* nib_plane = reinterpret_cast<uint32_t*>(packed);
  uint32_t* sign_plane = reinterpret_cast<uint32_t*>(packed + nibble_plane_bytes(n, k));

#pragma unroll
  for (int it = 0; it < kIters; ++it) {
    const int64_t row = row0 + wave * (2 * kIters) + 2 * it + half;
    float sum;
    const uint32_t code = quantize_block(blk[it].v, sum);

    // sign plane: bit j of the dword = sign bit of block j
    const unsigned long long ballot = __ballot((code >> 4) & 1u);
    const uint32_t sign_word = (uint32_t)(ballot >> (32 * half));

    // nibble dword (j & 7) >> 1: block 2d + h + 8b sits at bit 4h + 8b
    uint32_t nib = (code & 15u) << (4 * (j & 1) + 8 * (j >> 3));
    nib |= __shfl_xor(nib, 1);
    nib |= __shfl_xor(nib, 8);
    nib |= __shfl_xor(nib, 16);

    // pairwise tree over the 32 blocks of the superblock
    sum += __shfl_xor(sum, 1);
    sum += __shfl_xor(sum, 2);
    sum += __shfl_xor(sum, 4);
    sum += __shfl_xor(sum, 8);
    sum += __shfl_xor(sum, 16);

    if constexpr (DENSE != 0) {
      // every lane holds the superblock's sum after the butterfly
      const float a = (float)((double)sum / 96.0);
      if (row < n) {
        if (j == 3) alpha_direct[g * n + row] = a;
        const uint32_t z = (code >> 2) & 3u;
        float f[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) f[i] = (uint32_t)i == z ? 0.f : (blk[it].v[i] > 0.f ? a : -a);
        if constexpr (DENSE == SHERRY_F32 + 1) {
          *reinterpret_cast<float4*>(reinterpret_cast<float*>(dense) + row * k + col) =
              make_float4(f[0], f[1], f[2], f[3]);
        } else {
          uint2 v;
          v.x = (uint32_t)f32_to_bf16_rne(f[0]) | ((uint32_t)f32_to_bf16_rne(f[1]) << 16);
          v.y = (uint32_t)f32_to_bf16_rne(f[2]) | ((uint32_t)f32_to_bf16_rne(f[3]) << 16);
          *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(dense) + row * k + col) = v;
        }
      }
      continue;
    }
    if (row < n) {
      const int64_t rec = g * n + row;  // (superblock, row) record index
      if (j < 8 && (j & 1) == 0) nib_plane[rec * 4 + (j >> 1)] = nib;
      if (j == 1) sign_plane[rec] = sign_word;
      if (j == 3) {
        if (alpha_direct) {
          alpha_direct[g * n + row] = (float)((double)sum / 96.0);
        } else {
          sb_sums[row * nsb + g] = sum;
        }
      }
    }
  }
}

// Pairwise tree over `width` (a power of two) consecutive values starting at
// x, of which only the first `real` are read; the rest count as +0.  The
// sequential form keeps one partial per tree level: after element i, the
// partials of completed subtrees are merged (left + right), so the adds are
// exactly those of the level-by-level tree.
__device__ inline float tree_sum(const float* __restrict__ x, int64_t real, int64_t width) {
  float stack[40];
  int top_level = 0;
  for (int64_t i = 0; i < width; ++i) {
    float v = (i < real) ? x[i] : 0.f;
    int lvl = 0;
    int64_t t = i;
    while (t & 1) {
      v = stack[lvl] + v;
      t >>= 1;
      ++lvl;
    }
    stack[lvl] = v;
    top_level = lvl;
  }
  return stack[top_level];
}

__host__ __device__ inline int64_t next_pow2(int64_t v) {
  int64_t p = 1;
  while (p < v) p <<= 1;
  return p;
}

// per_group with G = 128*r (r > 1): tree over r superblock sums per group.
__global__ void alpha_group_kernel(const float* __restrict__ sb, int64_t n, int64_t nsb, int r,
                                   float* __restrict__ alpha) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t groups = nsb / r;
  if (idx >= n * groups) return;
  const int64_t gg = idx / n, row = idx % n;
  const float s = tree_sum(sb + row * nsb + gg * r, r, next_pow2(r));
  const double d = (double)r * kSuperblock / 4.0 * 3.0;
  alpha[gg * n + row] = (float)((double)s / d);
}

// per_channel: tree over the nsb superblock sums of a row (K flat order).
__global__ void alpha_channel_kernel(const float* __restrict__ sb, int64_t n, int64_t nsb, int64_t k,
                                     float* __restrict__ alpha) {
  const int64_t row = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (row >= n) return;
  const float s = tree_sum(sb + row * nsb, nsb, next_pow2(nsb));
  alpha[row] = (float)((double)s / ((double)k / 4.0 * 3.0));
}

// per_channel, one wave per row: lane l holds superblock sums E*l .. E*l+E-1
// of the row (+0 past nsb), reduces them pairwise in registers, and the XOR
// butterfly over 1..32 continues the tree: the index-order tree over 64*E
// values, which equals the tree over the row padded to a power of two.
template <int E>
__global__ __launch_bounds__(256) void alpha_channel_wave_kernel(const float* __restrict__ sb, int64_t n,
                                                                 int64_t nsb, int64_t k,
                                                                 float* __restrict__ alpha) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= n) return;
  float v[E];
#pragma unroll
  for (int i = 0; i < E; ++i) {
    const int64_t idx = (int64_t)lane * E + i;
    v[i] = idx < nsb ? sb[row * nsb + idx] : 0.f;
  }
#pragma unroll
  for (int w = E; w > 1; w >>= 1)
#pragma unroll
    for (int i = 0; i < w / 2; ++i) v[i] = v[2 * i] + v[2 * i + 1];
  float sum = v[0];
  sum += __shfl_xor(sum, 1);
  sum += __shfl_xor(sum, 2);
  sum += __shfl_xor(sum, 4);
  sum += __shfl_xor(sum, 8);
  sum += __shfl_xor(sum, 16);
  sum += __shfl_xor(sum, 32);
  if (lane == 0) alpha[row] = (float)((double)sum / ((double)k / 4.0 * 3.0));
}

// per_tensor: one level of the pairwise tree over the row-major sequence of
// superblock sums (the flat weight order cut at 128).  Each workgroup reduces
// one aligned chunk of 4096 values: lane l of wave w holds values
// 16*(64w + l) .. +15 and reduces them level by level in registers, the XOR
// butterfly over offsets 1..32 continues the same tree across lanes, and the
// four wave sums are added as (w0 + w1) + (w2 + w3).  Values past `real` are
// +0, which leaves every sum unchanged, so chunks of 4096 reproduce the tree
// over the padded power-of-two width exactly.  With `denom` > 0 the single
// chunk's sum is turned into the scale.
constexpr int kTreeChunk = 4096;
__global__ __launch_bounds__(256) void tree_level_kernel(const float* __restrict__ in, int64_t real,
                                                         float* __restrict__ out, double denom) {
  __shared__ float wsum[4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t base = (int64_t)blockIdx.x * kTreeChunk + (int64_t)(wave * 64 + lane) * 16;
  float v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] = (base + i < real) ? in[base + i] : 0.f;
#pragma unroll
  for (int w = 16; w > 1; w >>= 1)
#pragma unroll
    for (int i = 0; i < w / 2; ++i) v[i] = v[2 * i] + v[2 * i + 1];
  float sum = v[0];
  sum += __shfl_xor(sum, 1);
  sum += __shfl_xor(sum, 2);
  sum += __shfl_xor(sum, 4);
  sum += __shfl_xor(sum, 8);
  sum += __shfl_xor(sum, 16);
  sum += __shfl_xor(sum, 32);
  if (lane == 0) wsum[wave] = sum;
  __syncthreads();
  if (threadIdx.x == 0) {
    const float total = (wsum[0] + wsum[1]) + (wsum[2] + wsum[3]);
    if (denom > 0.0) {
      out[0] = (float)((double)total / denom);
    } else {
      out[blockIdx.x] = total;
    }
  }
}

}  // namespace

QuantizePlan plan_quantize(int64_t n, int64_t k, int gran, int group_size) {
  QuantizePlan p{};
  const int64_t nsb = k / kSuperblock;
  p.direct_alpha = (gran == SHERRY_PER_GROUP && group_size == kSuperblock);
  if (p.direct_alpha) return p;
  p.sb_sums = n * nsb;
  if (gran == SHERRY_PER_TENSOR) {
    p.chunk = kTreeChunk;
    p.chunks = 2 * ((p.sb_sums + kTreeChunk - 1) / kTreeChunk);  // two level buffers
  }
  p.workspace_bytes = (size_t)(p.sb_sums + p.chunks) * sizeof(float);
  return p;
}

hipError_t launch_quantize_pack(const QuantizePlan& p, int64_t n, int64_t k, int gran,
                                int group_size, const void* w, bool w_bf16, uint8_t* packed,
                                float* alpha, float* ws, hipStream_t s) {
  const int64_t nsb = k / kSuperblock;
  dim3 grid((unsigned)nsb, (unsigned)((n + kRowsPerTile - 1) / kRowsPerTile));
  float* direct = p.direct_alpha ? alpha : nullptr;
  if (w_bf16) {
    hipLaunchKernelGGL(quantize_pack_kernel<true>, grid, dim3(256), 0, s, w, n, k, packed, direct, ws);
  } else {
    hipLaunchKernelGGL(quantize_pack_kernel<false>, grid, dim3(256), 0, s, w, n, k, packed, direct, ws);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.direct_alpha) return e;

  if (gran == SHERRY_PER_GROUP) {
    const int r = group_size / kSuperblock;
    const int64_t items = n * (nsb / r);
    hipLaunchKernelGGL(alpha_group_kernel, dim3((unsigned)((items + 255) / 256)), dim3(256), 0, s,
                       ws, n, nsb, r, alpha);
  } else if (gran == SHERRY_PER_CHANNEL) {
    const dim3 g4((unsigned)((n + 3) / 4)), b256(256);
    if (nsb <= 64) hipLaunchKernelGGL(alpha_channel_wave_kernel<1>, g4, b256, 0, s, ws, n, nsb, k, alpha);
    else if (nsb <= 128) hipLaunchKernelGGL(alpha_channel_wave_kernel<2>, g4, b256, 0, s, ws, n, nsb, k, alpha);
    else if (nsb <= 256) hipLaunchKernelGGL(alpha_channel_wave_kernel<4>, g4, b256, 0, s, ws, n, nsb, k, alpha);
    else if (nsb <= 512) hipLaunchKernelGGL(alpha_channel_wave_kernel<8>, g4, b256, 0, s, ws, n, nsb, k, alpha);
    else if (nsb <= 1024) hipLaunchKernelGGL(alpha_channel_wave_kernel<16>, g4, b256, 0, s, ws, n, nsb, k, alpha);
    else hipLaunchKernelGGL(alpha_channel_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                            ws, n, nsb, k, alpha);
  } else {
    const double denom = (double)n * (double)k / 4.0 * 3.0;
    const float* in = ws;
    float* bufs[2] = {ws + p.sb_sums, ws + p.sb_sums + p.chunks / 2};
    int64_t real = p.sb_sums;
    for (int level = 0;; ++level) {
      const int64_t chunks = (real + kTreeChunk - 1) / kTreeChunk;
      if (chunks == 1) {
        hipLaunchKernelGGL(tree_level_kernel, dim3(1), dim3(256), 0, s, in, real, alpha, denom);
        break;
      }
      float* out = bufs[level & 1];
      hipLaunchKernelGGL(tree_level_kernel, dim3((unsigned)chunks), dim3(256), 0, s, in, real, out, 0.0);
      in = out;
      real = chunks;
    }
  }
  return hipGetLastError();
}

FakeQuantPlan plan_fake_quant(int64_t n, int64_t k, int gran, int group_size) {
  FakeQuantPlan p{};
  p.fused = gran == SHERRY_PER_GROUP && group_size == kSuperblock;
  if (p.fused) return p;
  p.packed_offset = 0;
  p.quant_ws_offset = ((size_t)(n * k / 32 * 5) + 255) / 256 * 256;
  p.workspace_bytes = p.quant_ws_offset + plan_quantize(n, k, gran, group_size).workspace_bytes;
  return p;
}

hipError_t launch_fake_quant(const FakeQuantPlan& p, int64_t n, int64_t k, int gran, int group_size,
                             const void* w, bool w_bf16, void* out, int out_dtype, float* alpha,
                             uint8_t* ws, hipStream_t s) {
  if (p.fused) {
    const int64_t nsb = k / kSuperblock;
    dim3 grid((unsigned)nsb, (unsigned)((n + kRowsPerTile - 1) / kRowsPerTile));
#define SHERRY_FQ(B, D) \
  hipLaunchKernelGGL((quantize_pack_kernel<B, D>), grid, dim3(256), 0, s, w, n, k, nullptr, alpha, nullptr, out)
    if (w_bf16) {
      if (out_dtype == SHERRY_F32) SHERRY_FQ(true, SHERRY_F32 + 1); else SHERRY_FQ(true, SHERRY_BF16 + 1);
    } else {
      if (out_dtype == SHERRY_F32) SHERRY_FQ(false, SHERRY_F32 + 1); else SHERRY_FQ(false, SHERRY_BF16 + 1);
    }
#undef SHERRY_FQ
    return hipGetLastError();
  }
  // other granularities: the scale needs sums beyond one superblock, so
  // quantize + pack into the workspace, then decode densely
  uint8_t* packed = ws + p.packed_offset;
  const QuantizePlan qp = plan_quantize(n, k, gran, group_size);
  hipError_t e = launch_quantize_pack(qp, n, k, gran, group_size, w, w_bf16, packed, alpha,
                                      reinterpret_cast<float*>(ws + p.quant_ws_offset), s);
  if (e != hipSuccess) return e;
  return launch_unpack(n, k, gran, group_size, packed, alpha, out, out_dtype, s);
}

}  // namespace sherry
