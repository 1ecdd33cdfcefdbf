/*
 * sherry.h -- C ABI of libsherry, the Sherry 1.25-bit ternary linear layer for
 * AMD Instinct MI355X (gfx950).
 *
 * The method.  Every block of 4 consecutive weights along K keeps three +-1
 * values and one 0, stored in 5 bits: 4 zero positions x 8 sign patterns = 32
 * states, split into a sign bit and 4 lookup bits ("Sherry: Hardware-Efficient
 * 1.25-Bit Ternary Quantization via Fine-grained Sparsification", agihunt
 * digest, format paragraph; ACL 2026 abstract).  A scale alpha per tensor,
 * output channel or group of G weights multiplies the ternary matrix T, and
 * the layer computes y = x * (T*alpha)^T with bf16 activations ("Sherry,
 * Tequila and Fairies in Python", section 1.1, SherryNMQuant and
 * SherryLinear; digest, inference paragraph).
 *
 * Conventions for every entry point:
 *  - Shapes follow nn.Linear: W is [N, K] row-major (N = out_features,
 *    K = in_features).  Blocks and groups run along K.
 *  - Pointers are DEVICE pointers (hipMalloc'd or torch CUDA tensors) unless
 *    stated otherwise; the caller owns all memory.  The library never
 *    allocates, frees or synchronizes, and is thread-safe.  Its only state is
 *    the static device workspace of sherry_quantize_pack_noalloc (one per
 *    device, with its address cached on first use).
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  All
 *    work is enqueued asynchronously on it.
 *  - Argument checks run on the host before any launch.  A bad argument
 *    returns its status code and nothing is launched.  A launch failure
 *    reported by the HIP runtime returns SHERRY_ERR_HIP.  On any error the
 *    outputs are undefined.  No C++ exception crosses this boundary.
 *  - Device pointers must be 16-byte aligned.
 *
 * Byte layout of `packed` (fixed by this library; the pages give none):
 *   K is cut into superblocks of 128 weights (32 blocks); nsb = K/128.
 *   Block code: code = s<<4 | z<<2 | p1<<1 | p0, with z the zero position,
 *   k0<k1<k2 the kept positions, s = [sign(k0) = -1], p0 = [sign(k1) !=
 *   sign(k0)], p1 = [sign(k2) != sign(k0)].  Flipping s negates the block.
 *   nibble plane (N*K/8 bytes): 16 bytes per (superblock g, row n), g-major;
 *     4 little-endian dwords d; byte b of dword d holds block 2d+8b (low
 *     nibble) and block 2d+1+8b (high nibble); nibble = code & 15.
 *   sign plane (N*K/32 bytes, right after): one dword per (g, n), g-major;
 *     bit j = code >> 4 of block j.
 *   Total N*K*5/32 bytes = 1.25 bits per weight.
 * Scale layout (fp32): per_group [K/G][N] (group-major), per_channel [N],
 *   per_tensor [1].
 */
#ifndef SHERRY_H
#define SHERRY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SHERRY_ABI_VERSION 2

/* Status codes. */
typedef enum {
  SHERRY_OK = 0,
  SHERRY_ERR_NULL = 1,        /* a required pointer is NULL */
  SHERRY_ERR_SHAPE = 2,       /* N <= 0, K <= 0 or K % 4 != 0 (the block size) */
  SHERRY_ERR_GROUP = 3,       /* per_group with G <= 0, K % G != 0 or G % 4 != 0 */
  SHERRY_ERR_GRANULARITY = 4, /* granularity is not one of sherry_granularity */
  SHERRY_ERR_DTYPE = 5,       /* a dtype argument not allowed for that operand */
  SHERRY_ERR_UNSUPPORTED = 6, /* legal for the method but not built here:
                                 K % 128 != 0, per_group with G % 128 != 0,
                                 K/128 or N/64 above 65535, or a GEMM with
                                 K > 2^21 */
  SHERRY_ERR_ALIGN = 7,       /* a device pointer or stride is not 16-byte aligned */
  SHERRY_ERR_WORKSPACE = 8,   /* workspace NULL or smaller than sherry_workspace_bytes */
  SHERRY_ERR_BATCH = 9,       /* batch outside 1..16, m < 1, count < 1, or a
                                 stride too small for its operand */
  SHERRY_ERR_HIP = 10         /* the HIP runtime reported an error at launch */
} sherry_status;

/* Scale granules ("Sherry, Tequila and Fairies in Python", section 1.1,
 * _reshape_by_granularity): the whole matrix, one output row, or G
 * consecutive weights of a row. */
typedef enum {
  SHERRY_PER_TENSOR = 0,
  SHERRY_PER_CHANNEL = 1,
  SHERRY_PER_GROUP = 2
} sherry_granularity;

typedef enum {
  SHERRY_F32 = 0,
  SHERRY_BF16 = 1,
  SHERRY_I8 = 2
} sherry_dtype;

/* Operation ids for sherry_workspace_bytes. */
typedef enum {
  SHERRY_OP_QUANTIZE_PACK = 0,
  SHERRY_OP_UNPACK = 1,
  SHERRY_OP_GEMV = 2,
  SHERRY_OP_GEMM = 3,
  SHERRY_OP_FAKE_QUANT = 4,
  SHERRY_OP_ARENAS_GEMM = 5
} sherry_op;

/* Library ABI version (SHERRY_ABI_VERSION of the build). */
int32_t sherry_abi_version(void);

/* Human-readable name of a status code; never NULL. */
const char* sherry_status_string(int32_t status);

/* Bytes of the packed planes: N*K*5/32 (5 bits per 4 weights; digest, format
 * paragraph).  Returns 0 if N or K is not positive or K % 128 != 0. */
size_t sherry_packed_bytes(int64_t n, int64_t k);

/* Number of fp32 scales: 1 (per_tensor), N (per_channel), N*K/G (per_group).
 * Returns -1 on invalid arguments. */
int64_t sherry_num_scales(int64_t n, int64_t k, int32_t granularity, int32_t group_size);

/* Workspace bytes an operation needs for these arguments (0 if none).
 * `batch_or_m` is the GEMV batch or the GEMM row count; `count` the GEMV
 * count (1 otherwise).  Returns (size_t)-1 on invalid arguments. */
size_t sherry_workspace_bytes(int32_t op, int64_t n, int64_t k, int32_t granularity,
                              int32_t group_size, int64_t batch_or_m, int32_t count);

/*
 * sherry_quantize_pack -- Sparse-AbsMean quantization and 5-bit packing of a
 * latent weight (digest, format paragraph: zero the smallest |w| of each
 * block of 4, keep the signs of the other three, scale = mean |w| of the kept
 * weights; "Sherry, Tequila and Fairies in Python", section 1.1,
 * SherryNMQuant.forward: granules and the nominal kept count L/4*3 as the
 * denominator; digest, inference paragraph: packing happens offline).
 *
 *   w        [N, K] latent weight, row-major, dtype SHERRY_F32 or SHERRY_BF16.
 *            Values must be finite (not checked).
 *   packed   out, sherry_packed_bytes(n, k) bytes, layout above.
 *   alpha    out, sherry_num_scales(...) fp32, layout above.
 *   Ties for the smallest |w| go to the lowest index; -0 equals +0; a kept
 *   weight's sign is +1 iff w > 0.  Scale: S = pairwise tree of fp32 adds of
 *   the kept |w| of the granule in flat index order (padded with +0 to a power
 *   of two), alpha = fp32(fp64(S) / fp64(L/4*3)).  Codes, bytes and scales
 *   are deterministic.
 *   workspace: sherry_workspace_bytes(SHERRY_OP_QUANTIZE_PACK, ...) bytes.
 *   For K up to 65536 (512 superblocks) per_group and per_channel need none
 *   and per_tensor needs ceil(N/8) fp32 partials when K/128 is a power of two
 *   (else N*K/128); longer rows need N*K/128 fp32 superblock sums except
 *   per_group with G == 128.  Per_tensor adds two level buffers of
 *   ceil(partials / 4096) values.
 */
int32_t sherry_quantize_pack(int64_t n, int64_t k, int32_t granularity, int32_t group_size,
                             const void* w, int32_t w_dtype, void* packed, float* alpha,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * sherry_quantize_pack_noalloc -- for callers that cannot allocate memory:
 * code under HIP graph capture, tight serving or training loops that
 * re-quantize every step, harnesses that forbid hipMalloc.  The same
 * operation, results and argument rules as sherry_quantize_pack, with the
 * workspace taken from a static device buffer of the library
 * (SHERRY_QUANTIZE_SCRATCH_BYTES, 8 MiB, on each device the library runs on,
 * held until the process ends) instead of a caller's buffer.  Nothing is
 * allocated.
 *
 *   Limit: sherry_workspace_bytes(SHERRY_OP_QUANTIZE_PACK, ...) must not
 *   exceed SHERRY_QUANTIZE_SCRATCH_BYTES, else SHERRY_ERR_WORKSPACE and
 *   nothing is launched.  Weights that need no workspace (per_group and
 *   per_channel with K up to 65536, per_group G == 128 at any K) have no
 *   limit; per_tensor with K/128 a power of two allows about 16 M rows;
 *   the other cases keep N*K/128 fp32 sums: about 2^28 weights.
 *   The buffer belongs to the current device: `stream` must be a stream of
 *   the current device.  Every call on a device shares that device's buffer
 *   and leaves its contents behind (every value is written before it is read,
 *   so nothing needs clearing): calls that overlap on one device (two
 *   streams, two threads) race and must be serialized by the caller.
 */
#define SHERRY_QUANTIZE_SCRATCH_BYTES ((size_t)8 << 20)
int32_t sherry_quantize_pack_noalloc(int64_t n, int64_t k, int32_t granularity, int32_t group_size,
                                     const void* w, int32_t w_dtype, void* packed, float* alpha,
                                     void* stream);

/*
 * sherry_unpack -- decode packed planes back to the ternary matrix or the
 * dequantized weight T*alpha ("Sherry, Tequila and Fairies in Python",
 * section 1.1: the quantizer returns sign times scale).
 *
 *   out_dtype SHERRY_I8:   out [N, K] int8 T in {-1, 0, 1}; alpha may be NULL.
 *   out_dtype SHERRY_F32:  out [N, K] fp32 T*alpha (exact).
 *   out_dtype SHERRY_BF16: out [N, K] bf16 round-to-nearest-even(T*alpha).
 */
int32_t sherry_unpack(int64_t n, int64_t k, int32_t granularity, int32_t group_size,
                      const void* packed, const float* alpha, void* out, int32_t out_dtype,
                      void* stream);

/*
 * sherry_gemv -- decode-time product y[b, n] = sum_k x[b, k] * T[n, k] * alpha(n, k)
 * ("Sherry, Tequila and Fairies in Python", section 1.1: SherryLinear applies
 * F.linear with the quantized weight, no bias here; digest, inference
 * paragraph: accumulate, then apply the scale; activations stay bf16).
 * Accumulation is fp32 with one scale multiply per group.
 *
 *   x        [batch, K] bf16 row-major, shared by all `count` matrices.
 *   batch    1..16.
 *   y        [batch, N] per matrix, dtype SHERRY_BF16 (round to nearest
 *            even) or SHERRY_F32.
 *   count    number of same-shape matrices in one launch (>= 1).  Matrix c
 *            uses packed + c*packed_stride bytes, alpha + c*alpha_stride
 *            floats, y + c*y_stride elements.  Strides are ignored when
 *            count == 1; otherwise packed_stride >= packed bytes (multiple of
 *            16), alpha_stride >= number of scales (multiple of 4), y_stride >=
 *            batch*N (multiple of 8).
 *   workspace: sherry_workspace_bytes(SHERRY_OP_GEMV, ...) bytes (split-K
 *            partial sums for launches too small to fill the GPU; may be 0).
 * Result within 1e-3 * sum_k |x[b,k] * alpha(n,k)| of the exact product.
 */
int32_t sherry_gemv(int64_t n, int64_t k, int32_t granularity, int32_t group_size,
                    const void* packed, const float* alpha, const void* x, int32_t batch,
                    void* y, int32_t y_dtype, int32_t count, int64_t packed_stride,
                    int64_t alpha_stride, int64_t y_stride, void* workspace,
                    size_t workspace_bytes, void* stream);

/*
 * sherry_gemm -- prefill product Y[m, n] = sum_k X[m, k] * T[n, k] * alpha(n, k)
 * (same definition as sherry_gemv with M rows of activations).  Each wave
 * decodes its ternary blocks into bf16 MFMA operands (+-1 / 0) in registers
 * through a 32-entry LDS table; bf16 MFMA with fp32 accumulation per group,
 * then scaled.
 *
 *   x   [M, K] bf16 row-major;  y [M, N] bf16 row-major (round to nearest even).
 *   m   >= 1.
 *   K   at most 2^21 (SHERRY_ERR_UNSUPPORTED above).
 *   workspace: sherry_workspace_bytes(SHERRY_OP_GEMM, ...) bytes (may be 0).
 * Result within 1e-3 * sum_k |X[m,k] * alpha(n,k)| of the exact product.
 */
int32_t sherry_gemm(int64_t n, int64_t k, int32_t granularity, int32_t group_size,
                    const void* packed, const float* alpha, const void* x, int64_t m,
                    void* y, void* workspace, size_t workspace_bytes, void* stream);

/*
 * sherry_fake_quant -- the quantize -> dequantize forward used in
 * quantization-aware training: out = T * alpha, dense, from the latent weight
 * ("Sherry, Tequila and Fairies in Python", section 1.1: SherryNMQuant.forward
 * returns the ternary signs times the scale, and its backward passes the
 * gradient through unchanged, the straight-through estimator; the identity
 * backward needs no kernel and lives in the Python binding).
 *
 *   w        [N, K] latent weight, row-major, SHERRY_F32 or SHERRY_BF16.
 *   out      [N, K] row-major, out_dtype SHERRY_F32 (exact T*alpha) or
 *            SHERRY_BF16 (T*alpha rounded to nearest even).  May not alias w.
 *   alpha    out, sherry_num_scales(...) fp32, the same scales (and layout)
 *            sherry_quantize_pack writes.
 *   Codes and scales are those of sherry_quantize_pack, bit for bit.
 *   workspace: sherry_workspace_bytes(SHERRY_OP_FAKE_QUANT, ...) bytes: 0 for
 *            per_group with G == 128 and, for K up to 16384, per_channel and
 *            per_group G > 128 (one kernel each); otherwise (per_tensor,
 *            longer rows) room for the packed planes plus the quantize
 *            workspace (quantize + pack, then a dense decode).
 */
int32_t sherry_fake_quant(int64_t n, int64_t k, int32_t granularity, int32_t group_size,
                          const void* w, int32_t w_dtype, void* out, int32_t out_dtype, float* alpha,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * sherry_arenas_gemm -- the Arenas training forward Y = X (T*alpha)^T +
 * lambda * X W^T: the Sherry product plus an annealed full-precision residual
 * over the latent weight W ("Sherry: Hardware-Efficient 1.25-Bit Ternary
 * Quantization via Fine-grained Sparsification", agihunt digest, the
 * weight-trapping paragraph: the residual weight lambda_t decays to 0 on a
 * cosine schedule and is gone at inference).  One kernel runs both products
 * in the same K loop on bf16 MFMA with fp32 accumulation; the residual weight
 * of a step comes from sherry_arenas_lambda (below) or from the caller.
 *
 *   packed, alpha   the quantized weight, as for sherry_gemm.
 *   w       [N, K] bf16 row-major: the latent weight (round an fp32 master
 *           weight to bf16 first); (N + 128) * K * 2 must stay below 2^31
 *           (SHERRY_ERR_UNSUPPORTED otherwise).
 *   lambda  the residual weight for this step, any finite value (not
 *           checked: a NaN or infinite lambda gives NaN or infinite outputs,
 *           as the formula does).
 *   x, m, y, workspace: as for sherry_gemm
 *           (sherry_workspace_bytes(SHERRY_OP_ARENAS_GEMM, ...)).
 * Result within 1e-3 * sum_k |X[m,k]| * (alpha(n,k) + |lambda * W[n,k]|) of
 * the exact value (plus half a bf16 ulp of the output).
 */
int32_t sherry_arenas_gemm(int64_t n, int64_t k, int32_t granularity, int32_t group_size,
                           const void* packed, const float* alpha, const void* w, float lambda,
                           const void* x, int64_t m, void* y, void* workspace, size_t workspace_bytes,
                           void* stream);

/*
 * sherry_arenas_lambda -- the residual weight of the Arenas forward at a
 * training step: the weight decays from lambda0 to 0 along half a cosine wave
 * over the annealing steps and is gone afterwards, so inference runs the
 * plain Sherry product ("Sherry: Hardware-Efficient 1.25-Bit Ternary
 * Quantization via Fine-grained Sparsification", agihunt digest, the
 * weight-trapping paragraph).
 *
 *   returns lambda0 * (1 + cos(pi * step / total_steps)) / 2 in fp64 for
 *   step < total_steps, and 0 when step >= total_steps or total_steps <= 0.
 *   Host arithmetic only: no device, no stream, no error status.  Pass the
 *   result (rounded to fp32) as sherry_arenas_gemm's lambda.
 */
double sherry_arenas_lambda(int64_t step, int64_t total_steps, double lambda0);

/*
 * Comparison packings of the same ternary matrix -- the two ways of storing
 * ternary weights the pages set Sherry's 1.25 bits against ("Sherry:
 * Hardware-Efficient 1.25-Bit Ternary Quantization via Fine-grained
 * Sparsification", agihunt digest, problem paragraph: pad every weight to 2
 * bits, or pack three weights in 5 bits, the 1.67-bit width of the "TL2"
 * kernels in its results table).  They exist to measure that claim on this
 * GPU: same T, same per-channel scales, same product.
 *
 * Layouts (this library's):
 *   SHERRY_CMP_2BIT  value 0 / +1 / -1 -> code 0 / 1 / 2, 2 bits per weight.
 *                    K in superblocks of 128; the 32-byte record of
 *                    (superblock g, row n) at byte (g*N + n)*32; byte j holds
 *                    block j's 4 weights, weight i in bits 2i.  N*K/4 bytes.
 *   SHERRY_CMP_TL2   digits d = v + 1; triple code d0 + 3 d1 + 9 d2 in 5 bits.
 *                    K in superblocks of 192 (64 triples), zero-padded to a
 *                    multiple of 192; the 40-byte record of (superblock g,
 *                    row n) at byte (g*N + n)*40 holds code t in bits
 *                    [5t, 5t+5).  N*ceil(K/192)*40 bytes.
 */
typedef enum { SHERRY_CMP_2BIT = 0, SHERRY_CMP_TL2 = 1 } sherry_compare_format;

/* Bytes of a comparison packing; 0 on invalid arguments (format, N <= 0,
 * K <= 0 or K % 128 != 0). */
size_t sherry_compare_bytes(int32_t format, int64_t n, int64_t k);

/* Re-encode Sherry planes (sherry_quantize_pack output, [N, K]) into a
 * comparison packing: out receives sherry_compare_bytes(format, n, k) bytes. */
int32_t sherry_compare_repack(int32_t format, int64_t n, int64_t k, const void* packed, void* out,
                              void* stream);

/* Batch-1 GEMV over a comparison packing with per-channel scales:
 * y[n] = alpha[n] * sum_k x[k] T[n, k], bf16 out (round to nearest even).
 *   alpha   [N] fp32 (the per_channel scales of the same T).
 *   x       [K] bf16.   y  [N] bf16 per matrix.
 *   count / strides as for sherry_gemv (count matrices, shared x; strides
 *   ignored when count == 1; planes_stride >= sherry_compare_bytes, a multiple
 *   of 16; alpha_stride >= N; y_stride >= N).
 * No split of K: launches with few rows are slow (this is a measuring tool).
 * Result within 1e-3 * sum_k |x[k] * alpha[n]| of the exact product. */
int32_t sherry_compare_gemv(int32_t format, int64_t n, int64_t k, const void* planes, const float* alpha,
                            const void* x, void* y, int32_t count, int64_t planes_stride,
                            int64_t alpha_stride, int64_t y_stride, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SHERRY_H */
