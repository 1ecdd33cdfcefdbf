// C-ABI entry points of libsherry: argument checks, launch plans, launches.
//
// Every check runs on the host before anything is enqueued, in this order:
// shape/granularity/group (the conditions of _reshape_by_granularity and
// SherryNMQuant.forward in "Sherry, Tequila and Fairies in Python", section
// 1.1, plus this build's K % 128 / G % 128 restriction), dtype, NULL pointers,
// 16-byte alignment, batch/count/strides, workspace.  Launch errors reported by
// the HIP runtime map to SHERRY_ERR_HIP.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "sherry_internal.h"

using namespace sherry;

namespace {

constexpr int64_t kMaxElems = (int64_t)1 << 46;
// GEMM: 32-bit buffer offsets into X need 512 rows of K bf16 below 2^31 bytes
constexpr int64_t kGemmMaxK = (int64_t)1 << 21;

int check_shape(int64_t n, int64_t k, int32_t gran, int32_t group_size) {
  if (n <= 0 || k <= 0 || k % kBlock != 0) return SHERRY_ERR_SHAPE;
  if (n > kMaxElems / k) return SHERRY_ERR_SHAPE;
  if (gran != SHERRY_PER_TENSOR && gran != SHERRY_PER_CHANNEL && gran != SHERRY_PER_GROUP)
    return SHERRY_ERR_GRANULARITY;
  if (gran == SHERRY_PER_GROUP && (group_size <= 0 || k % group_size != 0 || group_size % kBlock != 0))
    return SHERRY_ERR_GROUP;
  if (k % kSuperblock != 0) return SHERRY_ERR_UNSUPPORTED;
  if (gran == SHERRY_PER_GROUP && group_size % kSuperblock != 0) return SHERRY_ERR_UNSUPPORTED;
  if (k / kSuperblock > 65535) return SHERRY_ERR_UNSUPPORTED;  // grid dimension limits:
  if ((n + 63) / 64 > 65535) return SHERRY_ERR_UNSUPPORTED;      // superblocks and 64-row tiles
  return SHERRY_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int64_t num_scales(int64_t n, int64_t k, int32_t gran, int32_t group_size) {
  if (gran == SHERRY_PER_TENSOR) return 1;
  if (gran == SHERRY_PER_CHANNEL) return n;
  return n * (k / group_size);
}

int hip_status(hipError_t e) { return e == hipSuccess ? SHERRY_OK : SHERRY_ERR_HIP; }

}  // namespace

extern "C" {

int32_t sherry_abi_version(void) { return SHERRY_ABI_VERSION; }

const char* sherry_status_string(int32_t status) {
  switch (status) {
    case SHERRY_OK: return "SHERRY_OK";
    case SHERRY_ERR_NULL: return "SHERRY_ERR_NULL: a required pointer is NULL";
    case SHERRY_ERR_SHAPE: return "SHERRY_ERR_SHAPE: N and K must be positive and K divisible by 4";
    case SHERRY_ERR_GROUP: return "SHERRY_ERR_GROUP: per_group needs 0 < G, K % G == 0 and G % 4 == 0";
    case SHERRY_ERR_GRANULARITY: return "SHERRY_ERR_GRANULARITY: unsupported granularity";
    case SHERRY_ERR_DTYPE: return "SHERRY_ERR_DTYPE: dtype not allowed for this operand";
    case SHERRY_ERR_UNSUPPORTED: return "SHERRY_ERR_UNSUPPORTED: this build needs K % 128 == 0 and G % 128 == 0";
    case SHERRY_ERR_ALIGN: return "SHERRY_ERR_ALIGN: device pointers and strides must be 16-byte aligned";
    case SHERRY_ERR_WORKSPACE: return "SHERRY_ERR_WORKSPACE: workspace missing or too small";
    case SHERRY_ERR_BATCH: return "SHERRY_ERR_BATCH: batch must be 1..16, m and count >= 1, strides large enough";
    case SHERRY_ERR_HIP: return "SHERRY_ERR_HIP: the HIP runtime reported an error";
    default: return "unknown sherry status";
  }
}

size_t sherry_packed_bytes(int64_t n, int64_t k) {
  if (n <= 0 || k <= 0 || k % kSuperblock != 0 || n > kMaxElems / k) return 0;
  return (size_t)(n * k / 32 * 5);
}

int64_t sherry_num_scales(int64_t n, int64_t k, int32_t granularity, int32_t group_size) {
  const int st = check_shape(n, k, granularity, group_size);
  if (st != SHERRY_OK && st != SHERRY_ERR_UNSUPPORTED) return -1;
  return num_scales(n, k, granularity, group_size);
}

size_t sherry_workspace_bytes(int32_t op, int64_t n, int64_t k, int32_t granularity,
                              int32_t group_size, int64_t batch_or_m, int32_t count) {
  if (check_shape(n, k, granularity, group_size) != SHERRY_OK) return (size_t)-1;
  switch (op) {
    case SHERRY_OP_QUANTIZE_PACK:
      return plan_quantize(n, k, granularity, group_size).workspace_bytes;
    case SHERRY_OP_UNPACK:
      return 0;
    case SHERRY_OP_GEMV:
      if (batch_or_m < 1 || batch_or_m > 16 || count < 1) return (size_t)-1;
      return plan_gemv(n, k, granularity, group_size, (int)batch_or_m, count).workspace_bytes;
    case SHERRY_OP_GEMM:
      if (batch_or_m < 1) return (size_t)-1;
      return plan_gemm(n, k, granularity, group_size, batch_or_m, true).workspace_bytes;
    case SHERRY_OP_FAKE_QUANT:
      return plan_fake_quant(n, k, granularity, group_size).workspace_bytes;
    case SHERRY_OP_ARENAS_GEMM:
      if (batch_or_m < 1) return (size_t)-1;
      return plan_gemm(n, k, granularity, group_size, batch_or_m, false).workspace_bytes;
    default:
      return (size_t)-1;
  }
}

int32_t sherry_quantize_pack(int64_t n, int64_t k, int32_t granularity, int32_t group_size,
                             const void* w, int32_t w_dtype, void* packed, float* alpha,
                             void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_shape(n, k, granularity, group_size);
  if (st != SHERRY_OK) return st;
  if (w_dtype != SHERRY_F32 && w_dtype != SHERRY_BF16) return SHERRY_ERR_DTYPE;
  if (!w || !packed || !alpha) return SHERRY_ERR_NULL;
  if (!aligned16(w) || !aligned16(packed) || !aligned16(alpha)) return SHERRY_ERR_ALIGN;
  const QuantizePlan plan = plan_quantize(n, k, granularity, group_size);
  if (plan.workspace_bytes > 0 && (!workspace || workspace_bytes < plan.workspace_bytes))
    return SHERRY_ERR_WORKSPACE;
  if (plan.workspace_bytes > 0 && !aligned16(workspace)) return SHERRY_ERR_ALIGN;
  return hip_status(launch_quantize_pack(plan, n, k, granularity, group_size, w, w_dtype == SHERRY_BF16,
                                         static_cast<uint8_t*>(packed), alpha,
                                         static_cast<float*>(workspace),
                                         static_cast<hipStream_t>(stream)));
}

int32_t sherry_quantize_pack_noalloc(int64_t n, int64_t k, int32_t granularity, int32_t group_size,
                                     const void* w, int32_t w_dtype, void* packed, float* alpha,
                                     void* stream) {
  int st = check_shape(n, k, granularity, group_size);
  if (st != SHERRY_OK) return st;
  if (w_dtype != SHERRY_F32 && w_dtype != SHERRY_BF16) return SHERRY_ERR_DTYPE;
  if (!w || !packed || !alpha) return SHERRY_ERR_NULL;
  if (!aligned16(w) || !aligned16(packed) || !aligned16(alpha)) return SHERRY_ERR_ALIGN;
  const QuantizePlan plan = plan_quantize(n, k, granularity, group_size);
  if (plan.workspace_bytes > kQuantizeScratchBytes) return SHERRY_ERR_WORKSPACE;
  float* ws = nullptr;
  if (plan.workspace_bytes > 0 && quantize_scratch(&ws) != hipSuccess) return SHERRY_ERR_HIP;
  return hip_status(launch_quantize_pack(plan, n, k, granularity, group_size, w, w_dtype == SHERRY_BF16,
                                         static_cast<uint8_t*>(packed), alpha, ws,
                                         static_cast<hipStream_t>(stream)));
}

int32_t sherry_unpack(int64_t n, int64_t k, int32_t granularity, int32_t group_size,
                      const void* packed, const float* alpha, void* out, int32_t out_dtype,
                      void* stream) {
  int st = check_shape(n, k, granularity, group_size);
  if (st != SHERRY_OK) return st;
  if (out_dtype != SHERRY_I8 && out_dtype != SHERRY_F32 && out_dtype != SHERRY_BF16) return SHERRY_ERR_DTYPE;
  if (!packed || !out || (out_dtype != SHERRY_I8 && !alpha)) return SHERRY_ERR_NULL;
  if (!aligned16(packed) || !aligned16(out) || (alpha && !aligned16(alpha))) return SHERRY_ERR_ALIGN;
  return hip_status(launch_unpack(n, k, granularity, group_size, static_cast<const uint8_t*>(packed), alpha,
                                  out, out_dtype, static_cast<hipStream_t>(stream)));
}

int32_t sherry_gemv(int64_t n, int64_t k, int32_t granularity, int32_t group_size,
                    const void* packed, const float* alpha, const void* x, int32_t batch,
                    void* y, int32_t y_dtype, int32_t count, int64_t packed_stride,
                    int64_t alpha_stride, int64_t y_stride, void* workspace,
                    size_t workspace_bytes, void* stream) {
  int st = check_shape(n, k, granularity, group_size);
  if (st != SHERRY_OK) return st;
  if (y_dtype != SHERRY_BF16 && y_dtype != SHERRY_F32) return SHERRY_ERR_DTYPE;
  if (!packed || !alpha || !x || !y) return SHERRY_ERR_NULL;
  if (!aligned16(packed) || !aligned16(alpha) || !aligned16(x) || !aligned16(y)) return SHERRY_ERR_ALIGN;
  if (batch < 1 || batch > 16 || count < 1) return SHERRY_ERR_BATCH;
  if (count > 65535) return SHERRY_ERR_BATCH;
  if (count == 1) {
    packed_stride = alpha_stride = y_stride = 0;
  } else {
    if (packed_stride < (int64_t)sherry_packed_bytes(n, k) ||
        alpha_stride < num_scales(n, k, granularity, group_size) || y_stride < (int64_t)batch * n)
      return SHERRY_ERR_BATCH;
    if (packed_stride % 16 != 0 || alpha_stride % 4 != 0 || y_stride % 8 != 0) return SHERRY_ERR_ALIGN;
  }
  const GemvPlan plan = plan_gemv(n, k, granularity, group_size, batch, count);
  if (plan.workspace_bytes > 0 && (!workspace || workspace_bytes < plan.workspace_bytes))
    return SHERRY_ERR_WORKSPACE;
  if (plan.workspace_bytes > 0 && !aligned16(workspace)) return SHERRY_ERR_ALIGN;
  return hip_status(launch_gemv(plan, n, k, granularity, group_size, static_cast<const uint8_t*>(packed), alpha,
                                static_cast<const uint16_t*>(x), batch, y, y_dtype == SHERRY_BF16, count,
                                packed_stride, alpha_stride, y_stride, static_cast<float*>(workspace),
                                static_cast<hipStream_t>(stream)));
}

int32_t sherry_gemm(int64_t n, int64_t k, int32_t granularity, int32_t group_size,
                    const void* packed, const float* alpha, const void* x, int64_t m,
                    void* y, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_shape(n, k, granularity, group_size);
  if (st != SHERRY_OK) return st;
  if (k > kGemmMaxK) return SHERRY_ERR_UNSUPPORTED;
  if (!packed || !alpha || !x || !y) return SHERRY_ERR_NULL;
  if (!aligned16(packed) || !aligned16(alpha) || !aligned16(x) || !aligned16(y)) return SHERRY_ERR_ALIGN;
  if (m < 1 || m > kMaxElems / k || (m + 127) / 128 > 65535) return SHERRY_ERR_BATCH;
  const GemmPlan plan = plan_gemm(n, k, granularity, group_size, m, true);
  if (plan.workspace_bytes > 0 && (!workspace || workspace_bytes < plan.workspace_bytes))
    return SHERRY_ERR_WORKSPACE;
  if (plan.workspace_bytes > 0 && !aligned16(workspace)) return SHERRY_ERR_ALIGN;
  return hip_status(launch_gemm(plan, n, k, granularity, group_size, static_cast<const uint8_t*>(packed), alpha,
                                static_cast<const uint16_t*>(x), m, static_cast<uint16_t*>(y),
                                static_cast<float*>(workspace), static_cast<hipStream_t>(stream)));
}

int32_t sherry_fake_quant(int64_t n, int64_t k, int32_t granularity, int32_t group_size,
                          const void* w, int32_t w_dtype, void* out, int32_t out_dtype, float* alpha,
                          void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_shape(n, k, granularity, group_size);
  if (st != SHERRY_OK) return st;
  if (w_dtype != SHERRY_F32 && w_dtype != SHERRY_BF16) return SHERRY_ERR_DTYPE;
  if (out_dtype != SHERRY_F32 && out_dtype != SHERRY_BF16) return SHERRY_ERR_DTYPE;
  if (!w || !out || !alpha) return SHERRY_ERR_NULL;
  if (!aligned16(w) || !aligned16(out) || !aligned16(alpha)) return SHERRY_ERR_ALIGN;
  const FakeQuantPlan plan = plan_fake_quant(n, k, granularity, group_size);
  if (plan.workspace_bytes > 0 && (!workspace || workspace_bytes < plan.workspace_bytes))
    return SHERRY_ERR_WORKSPACE;
  if (plan.workspace_bytes > 0 && !aligned16(workspace)) return SHERRY_ERR_ALIGN;
  return hip_status(launch_fake_quant(plan, n, k, granularity, group_size, w, w_dtype == SHERRY_BF16, out,
                                      out_dtype, alpha, static_cast<uint8_t*>(workspace),
                                      static_cast<hipStream_t>(stream)));
}

int32_t sherry_arenas_gemm(int64_t n, int64_t k, int32_t granularity, int32_t group_size,
                           const void* packed, const float* alpha, const void* w, float lambda,
                           const void* x, int64_t m, void* y, void* workspace, size_t workspace_bytes,
                           void* stream) {
  int st = check_shape(n, k, granularity, group_size);
  if (st != SHERRY_OK) return st;
  if (k > kGemmMaxK || (n + 128) > ((int64_t)1 << 31) / (2 * k)) return SHERRY_ERR_UNSUPPORTED;
  if (!packed || !alpha || !w || !x || !y) return SHERRY_ERR_NULL;
  if (!aligned16(packed) || !aligned16(alpha) || !aligned16(w) || !aligned16(x) || !aligned16(y))
    return SHERRY_ERR_ALIGN;
  if (m < 1 || m > kMaxElems / k || (m + 127) / 128 > 65535) return SHERRY_ERR_BATCH;
  const GemmPlan plan = plan_gemm(n, k, granularity, group_size, m, false);
  if (plan.workspace_bytes > 0 && (!workspace || workspace_bytes < plan.workspace_bytes))
    return SHERRY_ERR_WORKSPACE;
  if (plan.workspace_bytes > 0 && !aligned16(workspace)) return SHERRY_ERR_ALIGN;
  return hip_status(launch_arenas_gemm(plan, n, k, granularity, group_size, static_cast<const uint8_t*>(packed),
                                       alpha, static_cast<const uint16_t*>(w), lambda,
                                       static_cast<const uint16_t*>(x), m, static_cast<uint16_t*>(y),
                                       static_cast<float*>(workspace), static_cast<hipStream_t>(stream)));
}

double sherry_arenas_lambda(int64_t step, int64_t total_steps, double lambda0) {
  if (total_steps <= 0 || step >= total_steps) return 0.0;
  const double pi = 3.141592653589793;
  return lambda0 * 0.5 * (1.0 + std::cos(pi * (double)step / (double)total_steps));
}

size_t sherry_compare_bytes(int32_t format, int64_t n, int64_t k) {
  if ((format != SHERRY_CMP_2BIT && format != SHERRY_CMP_TL2) || n <= 0 || k <= 0 || k % kSuperblock != 0 ||
      n > kMaxElems / k)
    return 0;
  return compare_bytes(format, n, k);
}

int32_t sherry_compare_repack(int32_t format, int64_t n, int64_t k, const void* packed, void* out,
                              void* stream) {
  if (format != SHERRY_CMP_2BIT && format != SHERRY_CMP_TL2) return SHERRY_ERR_DTYPE;
  const int st = check_shape(n, k, SHERRY_PER_CHANNEL, 0);
  if (st != SHERRY_OK) return st;
  if (!packed || !out) return SHERRY_ERR_NULL;
  if (!aligned16(packed) || !aligned16(out)) return SHERRY_ERR_ALIGN;
  return hip_status(launch_compare_repack(format, n, k, static_cast<const uint8_t*>(packed),
                                          static_cast<uint8_t*>(out), static_cast<hipStream_t>(stream)));
}

int32_t sherry_compare_gemv(int32_t format, int64_t n, int64_t k, const void* planes, const float* alpha,
                            const void* x, void* y, int32_t count, int64_t planes_stride,
                            int64_t alpha_stride, int64_t y_stride, void* stream) {
  if (format != SHERRY_CMP_2BIT && format != SHERRY_CMP_TL2) return SHERRY_ERR_DTYPE;
  const int st = check_shape(n, k, SHERRY_PER_CHANNEL, 0);
  if (st != SHERRY_OK) return st;
  if (!planes || !alpha || !x || !y) return SHERRY_ERR_NULL;
  if (!aligned16(planes) || !aligned16(alpha) || !aligned16(x) || !aligned16(y)) return SHERRY_ERR_ALIGN;
  if (count < 1 || count > 65535) return SHERRY_ERR_BATCH;
  if (count == 1) {
    planes_stride = alpha_stride = y_stride = 0;
  } else {
    if (planes_stride < (int64_t)compare_bytes(format, n, k) || alpha_stride < n || y_stride < n)
      return SHERRY_ERR_BATCH;
    if (planes_stride % 16 != 0 || alpha_stride % 4 != 0 || y_stride % 8 != 0) return SHERRY_ERR_ALIGN;
  }
  return hip_status(launch_compare_gemv(format, n, k, static_cast<const uint8_t*>(planes), alpha,
                                        static_cast<const uint16_t*>(x), static_cast<uint16_t*>(y), count,
                                        planes_stride, alpha_stride, y_stride, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
