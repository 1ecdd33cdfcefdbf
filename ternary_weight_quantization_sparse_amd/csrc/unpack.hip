// Decode packed planes to the ternary matrix T or the dequantized weight
// T*alpha ("Sherry, Tequila and Fairies in Python", section 1.1: the quantizer
// returns sign times scale; the 5-bit code is a sign bit plus 4 lookup bits
// per the agihunt digest, format paragraph).
//
// One thread per block of 4 output weights; consecutive threads walk K inside
// a row so the output stores are contiguous.
#include "sherry_internal.h"

namespace sherry {
namespace {

__device__ inline float scale_of(const float* __restrict__ alpha, int gran, int group_size,
                                 int64_t n, int64_t row, int64_t col) {
  if (gran == SHERRY_PER_TENSOR) return alpha[0];
  if (gran == SHERRY_PER_CHANNEL) return alpha[row];
  return alpha[(col / group_size) * n + row];
}

template <int OUT>
__global__ __launch_bounds__(256) void unpack_kernel(const uint8_t* __restrict__ packed,
                                                     const float* __restrict__ alpha, void* out,
                                                     int64_t n, int64_t k, int gran, int group_size) {
  const int64_t blocks_per_row = k / 4;
  const int64_t total = n * blocks_per_row;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = idx / blocks_per_row;
    const int64_t blk = idx % blocks_per_row;
    int t[4];
    decode_block(load_code(packed, n, k, row, blk), t);
    const int64_t off = row * k + blk * 4;
    if constexpr (OUT == SHERRY_I8) {
      const uint32_t v = (uint32_t)(uint8_t)(int8_t)t[0] | ((uint32_t)(uint8_t)(int8_t)t[1] << 8) |
                         ((uint32_t)(uint8_t)(int8_t)t[2] << 16) | ((uint32_t)(uint8_t)(int8_t)t[3] << 24);
      *reinterpret_cast<uint32_t*>(reinterpret_cast<int8_t*>(out) + off) = v;
    } else {
      const float a = scale_of(alpha, gran, group_size, n, row, blk * 4);
      float f[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) f[i] = t[i] == 0 ? 0.f : (t[i] > 0 ? a : -a);
      if constexpr (OUT == SHERRY_F32) {
        *reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + off) = make_float4(f[0], f[1], f[2], f[3]);
      } else {
        uint2 v;
        v.x = (uint32_t)f32_to_bf16_rne(f[0]) | ((uint32_t)f32_to_bf16_rne(f[1]) << 16);
        v.y = (uint32_t)f32_to_bf16_rne(f[2]) | ((uint32_t)f32_to_bf16_rne(f[3]) << 16);
        *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(out) + off) = v;
      }
    }
  }
}

}  // namespace

hipError_t launch_unpack(int64_t n, int64_t k, int gran, int group_size, const uint8_t* packed,
                         const float* alpha, void* out, int out_dtype, hipStream_t s) {
  const int64_t total = n * (k / 4);
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  const dim3 grid((unsigned)blocks), block(256);
  if (out_dtype == SHERRY_I8) {
    hipLaunchKernelGGL(unpack_kernel<SHERRY_I8>, grid, block, 0, s, packed, alpha, out, n, k, gran, group_size);
  } else if (out_dtype == SHERRY_F32) {
    hipLaunchKernelGGL(unpack_kernel<SHERRY_F32>, grid, block, 0, s, packed, alpha, out, n, k, gran, group_size);
  } else {
    hipLaunchKernelGGL(unpack_kernel<SHERRY_BF16>, grid, block, 0, s, packed, alpha, out, n, k, gran, group_size);
  }
  return hipGetLastError();
}

}  // namespace sherry
