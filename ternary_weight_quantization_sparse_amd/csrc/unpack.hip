// Decode packed planes to the ternary matrix T or the dequantized weight
// T*alpha ("Sherry, Tequila and Fairies in Python", section 1.1: the quantizer
// returns sign times scale; the 5-bit code is a sign bit plus 4 lookup bits
// per the agihunt digest, format paragraph).
//
// HBM-bound: each output element is written once, the planes are read once.
// Every lane writes 16 output bytes (4 blocks of int8, 2 of bf16, 1 of fp32),
// so the lanes that share one superblock record (8, 16 or 32 of them) write
// that record's 128 weights of one row as one contiguous segment, and the
// records of consecutive rows, which sit next to each other in the planes,
// are read by consecutive lane groups.  A 32-entry LDS table maps a code to
// the 16-byte output pattern of its block: int8 values for T, and for the
// scaled outputs a mask that is all ones where the weight is -1, ones except
// the sign bit where it is +1 and zero where it is 0, so that
// mask & (sign bit | bits of alpha) is the output (alpha >= 0; a -1 weight
// with alpha = 0 gives -0, as -1 * 0.0 does).  The output is written with
// non-temporal stores: it is not read back by this kernel, and streaming it
// past the caches measured 1.3-1.4x faster than plain stores on 8192 x 8192.
#include "sherry_internal.h"

namespace sherry {
namespace {

constexpr int kThreads = 256;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int kSbPerLane = 4;  // superblock columns handled by one lane

template <int OUT> struct UnpackTraits;
template <> struct UnpackTraits<SHERRY_I8> {
  static constexpr int kBlocksPerLane = 4;
  typedef uint32_t Entry;    // one block: 4 int8 values
  typedef uint4 Out;         // 16 bytes = 4 blocks
};
template <> struct UnpackTraits<SHERRY_BF16> {
  static constexpr int kBlocksPerLane = 2;
  typedef uint2 Entry;       // one block: 4 bf16 masks
  typedef uint4 Out;
};
template <> struct UnpackTraits<SHERRY_F32> {
  static constexpr int kBlocksPerLane = 1;
  typedef uint4 Entry;       // one block: 4 fp32 masks
  typedef uint4 Out;
};

template <int OUT>
__device__ inline typename UnpackTraits<OUT>::Entry table_entry(uint32_t code) {
  int t[4];
  decode_block(code, t);
  if constexpr (OUT == SHERRY_I8) {
    uint32_t v = 0;
#pragma unroll
    for (int p = 0; p < 4; ++p) v |= (uint32_t)(uint8_t)(int8_t)t[p] << (8 * p);
    return v;
  } else if constexpr (OUT == SHERRY_BF16) {
    uint32_t m[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) m[p] = t[p] == 0 ? 0u : (t[p] > 0 ? 0x7FFFu : 0xFFFFu);
    return make_uint2(m[0] | (m[1] << 16), m[2] | (m[3] << 16));
  } else {
    uint32_t m[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) m[p] = t[p] == 0 ? 0u : (t[p] > 0 ? 0x7FFFFFFFu : 0xFFFFFFFFu);
    return make_uint4(m[0], m[1], m[2], m[3]);
  }
}

// grid.x: groups of kThreads / lanes_per_record rows; grid.y: groups of
// kSbPerLane superblock columns.
template <int OUT>
__global__ __launch_bounds__(kThreads) void unpack_kernel(const uint8_t* __restrict__ packed,
                                                          const float* __restrict__ alpha,
                                                          uint8_t* __restrict__ out, int64_t n, int64_t k,
                                                          int gran, int group_size) {
  using Tr = UnpackTraits<OUT>;
  using Entry = typename Tr::Entry;
  constexpr int kBpl = Tr::kBlocksPerLane;
  constexpr int kLanesPerRec = kBlocksPerSb / kBpl;
  constexpr int kRowsPerWg = kThreads / kLanesPerRec;
  constexpr int kOutBytes = OUT == SHERRY_I8 ? 1 : (OUT == SHERRY_BF16 ? 2 : 4);

  __shared__ Entry table[32];
  if (threadIdx.x < 32) table[threadIdx.x] = table_entry<OUT>(threadIdx.x);
  __syncthreads();

  const int sub = threadIdx.x % kLanesPerRec;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerWg + threadIdx.x / kLanesPerRec;
  if (row >= n) return;
  const int64_t nsb = k / kSuperblock;
  const uint32_t sb_per_group = gran == SHERRY_PER_GROUP ? (uint32_t)(group_size / kSuperblock) : 1u;
  const int j0 = sub * kBpl;  // first block of this lane in the superblock
  // nibble dword of block j: (j & 7) >> 1, byte j >> 3, nibble j & 1
  const int dw0 = (j0 & 7) >> 1;
  const int byte_sh = 8 * (j0 >> 3);
  const uint32_t* nib_plane = reinterpret_cast<const uint32_t*>(packed);
  const uint32_t* sgn_plane = reinterpret_cast<const uint32_t*>(packed + nibble_plane_bytes(n, k));

  uint32_t nib[kSbPerLane][2], sgn[kSbPerLane];
  float a[kSbPerLane];
  int64_t gs[kSbPerLane];
#pragma unroll
  for (int s = 0; s < kSbPerLane; ++s) {
    // columns past the end repeat the last one (loaded, never stored)
    const int64_t g = min((int64_t)blockIdx.y * kSbPerLane + s, nsb - 1);
    gs[s] = g;
    const int64_t rec = g * n + row;
    if constexpr (kBpl == 4) {
      const uint2 d = *reinterpret_cast<const uint2*>(nib_plane + rec * 4 + dw0);
      nib[s][0] = d.x;
      nib[s][1] = d.y;
    } else {
      nib[s][0] = nib_plane[rec * 4 + dw0];
      nib[s][1] = 0;
    }
    sgn[s] = sgn_plane[rec];
    if constexpr (OUT != SHERRY_I8) {
      if (gran == SHERRY_PER_TENSOR) a[s] = alpha[0];
      else if (gran == SHERRY_PER_CHANNEL) a[s] = alpha[row];
      else a[s] = alpha[(int64_t)((uint32_t)g / sb_per_group) * n + row];
    } else {
      a[s] = 0.f;
    }
  }
#pragma unroll
  for (int s = 0; s < kSbPerLane; ++s) {
    if ((int64_t)blockIdx.y * kSbPerLane + s >= nsb) break;
    Entry e[kBpl];
#pragma unroll
    for (int i = 0; i < kBpl; ++i) {
      // block j0 + i: dword dw0 + (i >> 1) (kBpl == 4) or dw0, nibble (j0 + i) & 1
      const uint32_t d = nib[s][kBpl == 4 ? (i >> 1) : 0];
      const uint32_t code = ((d >> (byte_sh + 4 * ((j0 + i) & 1))) & 15u) | (((sgn[s] >> (j0 + i)) & 1u) << 4);
      e[i] = table[code];
    }
    uint4 v;
    if constexpr (OUT == SHERRY_I8) {
      v = make_uint4(e[0], e[1], e[2], e[3]);
    } else if constexpr (OUT == SHERRY_BF16) {
      const uint32_t h = (uint32_t)f32_to_bf16_rne(a[s]) | 0x8000u;
      const uint32_t hh = h | (h << 16);
      v = make_uint4(e[0].x & hh, e[0].y & hh, e[1].x & hh, e[1].y & hh);
    } else {
      const uint32_t f = __float_as_uint(a[s]) | 0x80000000u;
      v = make_uint4(e[0].x & f, e[0].y & f, e[0].z & f, e[0].w & f);
    }
    const int64_t col = gs[s] * kSuperblock + j0 * kBlock;
    const u32x4 vv = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(vv, reinterpret_cast<u32x4*>(out + (row * k + col) * kOutBytes));
  }
}

}  // namespace

hipError_t launch_unpack(int64_t n, int64_t k, int gran, int group_size, const uint8_t* packed,
                         const float* alpha, void* out, int out_dtype, hipStream_t s) {
  const int64_t nsb = k / kSuperblock;
  const unsigned gy = (unsigned)((nsb + kSbPerLane - 1) / kSbPerLane);
  uint8_t* o = static_cast<uint8_t*>(out);
  if (out_dtype == SHERRY_I8) {
    const dim3 grid((unsigned)((n + 31) / 32), gy);
    hipLaunchKernelGGL(unpack_kernel<SHERRY_I8>, grid, dim3(kThreads), 0, s, packed, alpha, o, n, k, gran,
                       group_size);
  } else if (out_dtype == SHERRY_F32) {
    const dim3 grid((unsigned)((n + 7) / 8), gy);
    hipLaunchKernelGGL(unpack_kernel<SHERRY_F32>, grid, dim3(kThreads), 0, s, packed, alpha, o, n, k, gran,
                       group_size);
  } else {
    const dim3 grid((unsigned)((n + 15) / 16), gy);
    hipLaunchKernelGGL(unpack_kernel<SHERRY_BF16>, grid, dim3(kThreads), 0, s, packed, alpha, o, n, k, gran,
                       group_size);
  }
  return hipGetLastError();
}

}  // namespace sherry
