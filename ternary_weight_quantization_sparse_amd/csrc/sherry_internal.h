// Internal declarations shared by the libsherry translation units (HIP kernels
// and the C-ABI host code).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/sherry.h"

namespace sherry {

constexpr int kBlock = 4;            // weights per block
constexpr int kSuperblock = 128;     // weights per superblock (32 blocks)
constexpr int kBlocksPerSb = 32;

// Offsets into the packed buffer.
inline __host__ __device__ int64_t nibble_plane_bytes(int64_t n, int64_t k) { return n * k / 8; }

// ---------------------------------------------------------------- quantize
struct QuantizePlan {
  bool rows;               // row-group kernel (K up to 512 superblocks)
  int rows_mode;           // its scale stage
  int64_t wg_rows;         // rows per workgroup of that kernel
  bool direct_alpha;       // superblock-tile kernel, per_group with G == 128: alpha written by the pack kernel
  int64_t sb_sums;         // number of fp32 superblock sums in the workspace
  int64_t chunk;           // per_tensor first-stage chunk (power of two)
  int64_t chunks;          // per_tensor first-stage partials
  size_t workspace_bytes;
};
QuantizePlan plan_quantize(int64_t n, int64_t k, int gran, int group_size);
hipError_t launch_quantize_pack(const QuantizePlan& p, int64_t n, int64_t k, int gran,
                                int group_size, const void* w, bool w_bf16, uint8_t* packed,
                                float* alpha, float* ws, hipStream_t s);
// Static quantize workspace on the current device (the allocation-free entry
// point's): its device address, looked up on the first call per device.
constexpr size_t kQuantizeScratchBytes = SHERRY_QUANTIZE_SCRATCH_BYTES;
hipError_t quantize_scratch(float** ptr);

// ---------------------------------------------------------------- fake quant
struct FakeQuantPlan {
  bool fused;              // per_group G = 128: one kernel writes T*alpha and the scales
  bool fused_rows;         // per_channel / per_group G > 128, K <= 16384: the row-group kernel writes them
  size_t packed_offset;    // otherwise: packed planes, then the quantize workspace
  size_t quant_ws_offset;
  size_t workspace_bytes;
};
FakeQuantPlan plan_fake_quant(int64_t n, int64_t k, int gran, int group_size);
hipError_t launch_fake_quant(const FakeQuantPlan& p, int64_t n, int64_t k, int gran, int group_size,
                             const void* w, bool w_bf16, void* out, int out_dtype, float* alpha,
                             uint8_t* ws, hipStream_t s);

// ---------------------------------------------------------------- comparison packings
int64_t compare_k_padded(int fmt, int64_t k);
size_t compare_bytes(int fmt, int64_t n, int64_t k);
hipError_t launch_compare_repack(int fmt, int64_t n, int64_t k, const uint8_t* packed, uint8_t* out,
                                 hipStream_t s);
hipError_t launch_compare_gemv(int fmt, int64_t n, int64_t k, const uint8_t* planes, const float* alpha,
                               const uint16_t* x, uint16_t* y, int count, int64_t planes_stride,
                               int64_t alpha_stride, int64_t y_stride, hipStream_t s);

// ---------------------------------------------------------------- unpack
hipError_t launch_unpack(int64_t n, int64_t k, int gran, int group_size, const uint8_t* packed,
                         const float* alpha, void* out, int out_dtype, hipStream_t s);

// ---------------------------------------------------------------- gemv
struct GemvPlan {
  int kind;               // 0 = table-lookup kernel (batch 1), 1 = MFMA kernel (batch 2..16)
  int rows_per_thread;    // kind 0
  int window_sbs;         // kind 0: superblocks per LDS table window
  int ksplit;             // kind 1: split of K across workgroups (1 = none)
  int rw, kw;             // kind 0: row waves x K-slices per workgroup
  int64_t panels;         // workgroups along N
  size_t workspace_bytes; // ksplit > 1: fp32 partials [count][ksplit][batch][N]
};
GemvPlan plan_gemv(int64_t n, int64_t k, int gran, int group_size, int batch, int count);
hipError_t launch_gemv(const GemvPlan& p, int64_t n, int64_t k, int gran, int group_size,
                       const uint8_t* packed, const float* alpha, const uint16_t* x, int batch,
                       void* y, bool y_bf16, int count, int64_t packed_stride,
                       int64_t alpha_stride, int64_t y_stride, float* ws, hipStream_t s);

// ---------------------------------------------------------------- gemm
struct GemmPlan {
  int tile_n, tile_m;
  int splits;              // K ranges per output tile (1 = none)
  size_t workspace_bytes;  // splits > 1: fp32 partials [splits][M][N]
};
// wide: 256-row weight tiles allowed (the plain GEMM; the Arenas forward
// passes false).
GemmPlan plan_gemm(int64_t n, int64_t k, int gran, int group_size, int64_t m, bool wide);
hipError_t launch_gemm(const GemmPlan& p, int64_t n, int64_t k, int gran, int group_size,
                       const uint8_t* packed, const float* alpha, const uint16_t* x, int64_t m,
                       uint16_t* y, float* ws, hipStream_t s);
// Arenas training forward: Y = X (T alpha)^T + lam X W^T, W the dense bf16
// latent weight [N, K]; same plan and workspace as the GEMM.
hipError_t launch_arenas_gemm(const GemmPlan& p, int64_t n, int64_t k, int gran, int group_size,
                              const uint8_t* packed, const float* alpha, const uint16_t* wd, float lam,
                              const uint16_t* x, int64_t m, uint16_t* y, float* ws, hipStream_t s);

// ---------------------------------------------------------------- device helpers
// Ternary values of a block from its code.  The sign bit gives the sign of
// the first kept weight; p0 / p1 say whether the second / third kept weight
// has the opposite sign.  Position z is the zero.
__device__ inline void decode_block(uint32_t code, int t[4]) {
  const int z = (code >> 2) & 3;
  const int neg0 = (code >> 4) & 1;
  const int neg1 = neg0 ^ (code & 1);
  const int neg2 = neg0 ^ ((code >> 1) & 1);
#pragma unroll
  for (int pos = 0; pos < 4; ++pos) {
    const int rank = pos - (pos > z ? 1 : 0);  // index among kept positions
    const int neg = rank == 0 ? neg0 : (rank == 1 ? neg1 : neg2);
    t[pos] = (pos == z) ? 0 : (neg ? -1 : 1);
  }
}

__device__ inline uint32_t load_code(const uint8_t* __restrict__ packed, int64_t n, int64_t k,
                                     int64_t row, int64_t blk) {
  const int64_t g = blk >> 5;
  const int j = (int)(blk & 31);
  const int64_t rec = g * n + row;
  const uint32_t* nib_plane = reinterpret_cast<const uint32_t*>(packed);
  const uint32_t* sign_plane = reinterpret_cast<const uint32_t*>(packed + nibble_plane_bytes(n, k));
  const uint32_t d = nib_plane[rec * 4 + ((j & 7) >> 1)];
  const uint32_t nib = (d >> (4 * (j & 1) + 8 * (j >> 3))) & 15u;
  const uint32_t sgn = (sign_plane[rec] >> j) & 1u;
  return (sgn << 4) | nib;
}

// bf16 patterns of one block (4 weights, +-1 or 0) from its code, as the two
// dwords of an MFMA operand: positions 0,1 in the first, 2,3 in the second.
__device__ inline uint2 decode_bf16(uint32_t code) {
  int t[4];
  decode_block(code, t);
  uint32_t h[4];
#pragma unroll
  for (int pos = 0; pos < 4; ++pos) h[pos] = t[pos] == 0 ? 0u : (t[pos] < 0 ? 0xBF80u : 0x3F80u);
  return make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
}

// Byte offsets (code * 8, into a table of 8-byte entries) of the blocks of
// quad q = 2d + h of a superblock record (blocks q + 8b, b = 0..3, in byte
// b): nibble dword d, half h, sign bits q + 8b moved to bit 7 of byte b.
__device__ inline uint32_t quad_offsets8(uint32_t nib_dword, uint32_t sign_word, int q) {
  const uint32_t nq = (q & 1) ? (nib_dword >> 1) : (nib_dword << 3);
  const uint32_t sq = (sign_word << (7 - q)) & 0x80808080u;
  return __builtin_amdgcn_bitop3_b32(nq, sq, 0x78787878u, 0xEC);  // (nq & mask) | sq
}

// s_waitcnt with only a vmcnt limit (expcnt / lgkmcnt left at their maxima).
template <int VM>
__device__ inline void wait_vmcnt() {
  static_assert(VM >= 0 && VM < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((VM & 15) | (7 << 4) | (15 << 8) | ((VM >> 4) << 14));
}

// LDS pointer type of the copy builtins that write LDS directly.
typedef __attribute__((address_space(3))) void lds_void;

// Word 3 of a raw buffer resource on gfx9-class parts: 32-bit data format
// (a zero format would make every access read zero), no swizzle, no stride.
constexpr int kBufferWord3 = 0x00020000;

// Workgroup barrier that orders LDS only: this wave's LDS reads and writes
// are complete (lgkmcnt 0) before it arrives.  Unlike __syncthreads it does
// not wait for vector-memory operations, so copies for later stages stay in
// flight; their completion is waited for explicitly (vmcnt) before the
// barrier that publishes them.  The memory clobber keeps the compiler from
// moving LDS accesses across it.
__device__ inline void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
  asm volatile("s_barrier" ::: "memory");
}

// Round an fp32 value to bf16, nearest-even (inputs are finite).
__device__ inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ inline float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

}  // namespace sherry
