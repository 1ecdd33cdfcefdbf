// Sparse-AbsMean quantize + 5-bit pack, and the scale reduction.
//
// Method: "Sherry: Hardware-Efficient 1.25-Bit Ternary Quantization via
// Fine-grained Sparsification" (agihunt digest, format paragraph): in every
// block of 4 weights along K the smallest |w| becomes 0, the other three keep
// their sign, and the scale is the mean |w| of the kept weights.  Granules and
// the nominal kept count L/4*3: "Sherry, Tequila and Fairies in Python",
// section 1.1 (_reshape_by_granularity, SherryNMQuant.forward).
//
// Mapping (details at the kernel): each lane quantizes a few adjacent blocks
// of one row, a wave covers a contiguous row span of several superblocks, and
// the per-superblock reductions (kept-|w| sum, sign dword, nibble dwords) are
// cross-lane DPP moves inside rows of 16 lanes that reproduce the pairwise
// tree's additions exactly.
#include <mutex>

#include "sherry_internal.h"

namespace sherry {
namespace {

// Static workspace of the allocation-free quantize entry point: superblock
// sums and tree partials live here instead of in a caller-provided buffer.
// Host code never names this array (in host code the name is a stand-in, not
// a device address); quantize_scratch() looks up its address on each device.
static __device__ __align__(256) float scratch[kQuantizeScratchBytes / sizeof(float)];

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_ptr[kMaxScratchDevices] = {};

#ifndef SHERRY_Q_BPL
#define SHERRY_Q_BPL 2  // blocks per lane
#endif

// Zero position and kept-|w| sum of one block.  The zero is the first index
// of the minimum |w|, found as a tournament: the smaller of each pair (ties
// keep the lower index), then the smaller of the two winners (ties keep the
// left pair).  The kept-|w| sum is the two-level pairwise tree ((a0 + a1) +
// (a2 + a3)) with the zeroed weight contributing +0; the pair holding the
// zero sums to its other member, the larger one (x + 0 = x exactly), so each
// half of the tree is an add or a pick.
__device__ inline uint32_t block_zero(const float v[4], float& kept_sum) {
  const float a0 = fabsf(v[0]), a1 = fabsf(v[1]), a2 = fabsf(v[2]), a3 = fabsf(v[3]);
  const bool c01 = a1 < a0;  // zero candidate of the left pair is 1 (and a0 is its larger)
  const bool c23 = a3 < a2;  // ... of the right pair is 3 (and a2 is its larger)
  const float m01 = c01 ? a1 : a0, m23 = c23 ? a3 : a2;
  const bool c = m23 < m01;  // the zero is in the right pair
  const float left = c ? a0 + a1 : (c01 ? a0 : a1);
  const float right = c ? (c23 ? a2 : a3) : a2 + a3;
  kept_sum = left + right;
  return c ? (c23 ? 3u : 2u) : (c01 ? 1u : 0u);
}

// The code of a block from its zero position z and positive mask (bit i =
// weight i > 0): the kept positions k0 < k1 < k2 are all but z; s = the first
// kept weight is not positive, p0 / p1 = the second / third kept weight's
// sign differs from the first.  code = s<<4 | z<<2 | p1<<1 | p0.
__device__ inline uint32_t block_code(uint32_t z, uint32_t pos) {
  uint32_t k[3], r = 0;
  for (uint32_t i = 0; i < 4; ++i)
    if (i != z) k[r++] = i;
  const uint32_t q0 = (pos >> k[0]) & 1u, q1 = (pos >> k[1]) & 1u, q2 = (pos >> k[2]) & 1u;
  return ((q0 ^ 1u) << 4) | (z << 2) | ((q2 ^ q0) << 1) | (q1 ^ q0);
}

// Lookup index of a block: z << 4 | pos', where pos' holds the positive flags
// of weights 0, 2, 1, 3 in bits 0..3 (the order the bf16 path produces them).
__device__ inline uint32_t code_index(uint32_t z, uint32_t pos_perm) { return (z << 4) | pos_perm; }
__device__ inline uint32_t unpermute_pos(uint32_t pp) {
  return (pp & 1u) | ((pp >> 1) & 1u) << 2 | ((pp >> 2) & 1u) << 1 | ((pp >> 3) & 1u) << 3;
}

// pos' of a block of 4 bf16 weights held as dwords d0 = w0 | w1 << 16 and
// d1 = w2 | w3 << 16: clamp each 16-bit weight (as a signed integer) to [0, 1]
// -- 1 exactly for the positive ones (sign clear, not zero) -- then fold the
// four flags into one nibble.  The clamps are written as packed 16-bit
// instructions (register operands only): the compiler would otherwise split
// them into per-half compares and selects.
__device__ inline uint32_t pos_perm_bf16(uint32_t d0, uint32_t d1) {
  uint32_t t01, t23;
  asm("v_pk_min_i16 %0, %2, %4\n"
      "v_pk_min_i16 %1, %3, %4\n"
      "v_pk_max_i16 %0, %0, 0\n"
      "v_pk_max_i16 %1, %1, 0"
      : "=&v"(t01), "=&v"(t23)
      : "v"(d0), "v"(d1), "v"(0x00010001u));
  const uint32_t sum = t01 + (t23 << 1);  // pos0 + 2 pos2 | (pos1 + 2 pos3) << 16
  return (sum & 3u) | (sum >> 14);        // pos0 | pos2 << 1 | pos1 << 2 | pos3 << 3
}
__device__ inline uint32_t pos_perm_f32(const float v[4]) {
  return (v[0] > 0.f ? 1u : 0u) | (v[2] > 0.f ? 2u : 0u) | (v[1] > 0.f ? 4u : 0u) | (v[3] > 0.f ? 8u : 0u);
}

// Cross-lane moves inside a row of 16 lanes (DPP): row_shr:n gives lane i
// the value of lane i - n, row_ror:n that of lane (i - n) mod 16.
template <int CTRL>
__device__ inline uint32_t dpp(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ inline float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int kShr1 = 0x111, kShr2 = 0x112, kShr4 = 0x114, kShr8 = 0x118, kRor4 = 0x124, kRor8 = 0x128;
// row_shl:n (n = 1..15) / row_shr:n (n = 1..7): lane i gets lane i + n /
// i - n of its row
template <typename T>
__device__ inline T dpp_shl(T v, int n) {
  switch (n) {
    case 1: return dpp<0x101>(v);
    case 2: return dpp<0x102>(v);
    case 3: return dpp<0x103>(v);
    case 4: return dpp<0x104>(v);
    case 5: return dpp<0x105>(v);
    case 6: return dpp<0x106>(v);
    case 7: return dpp<0x107>(v);
    case 8: return dpp<0x108>(v);
    case 9: return dpp<0x109>(v);
    case 10: return dpp<0x10A>(v);
    case 11: return dpp<0x10B>(v);
    case 12: return dpp<0x10C>(v);
    case 13: return dpp<0x10D>(v);
    case 14: return dpp<0x10E>(v);
    default: return dpp<0x10F>(v);
  }
}
template <typename T>
__device__ inline T dpp_shr(T v, int n) {
  switch (n) {
    case 1: return dpp<0x111>(v);
    case 2: return dpp<0x112>(v);
    case 3: return dpp<0x113>(v);
    case 4: return dpp<0x114>(v);
    case 5: return dpp<0x115>(v);
    case 6: return dpp<0x116>(v);
    default: return dpp<0x117>(v);
  }
}
constexpr int kQuadXor2 = 0x4E;  // quad_perm [2, 3, 0, 1]
// ds_swizzle patterns (bit mode, groups of 32 lanes): lane ^ 4, and the last
// lane of each group of 16 / 8
constexpr int kSwzXor4 = (4 << 10) | 0x1F, kSwzLast16 = (0x0F << 5) | 0x10, kSwzLast8 = (0x07 << 5) | 0x18;

// DENSE = 0: write the packed planes (and the scale or the superblock sum).
// DENSE = SHERRY_F32 + 1 / SHERRY_BF16 + 1 (per_group G = 128 only): the
// fused fake-quant forward -- write T * alpha densely in fp32 (exact) or bf16
// (round to nearest even) and the scales, no planes.
//
// Mapping: a wave quantizes one row at a time over 2*BPL consecutive
// superblocks; lane (s, i) -- s = lane / L, L = 32 / BPL lanes per
// superblock -- owns the BPL adjacent blocks BPL*i .. of superblock s, one
// contiguous 8*BPL-byte (bf16) or 16*BPL-byte (fp32) load.  The kept-|w| sum
// of the superblock is the index-order pairwise tree over its 32 block sums:
// the first log2(BPL) levels inside the lane, the rest across lanes with
// row_shr by 1, 2, 4 (, 8), which leaves the tree's root in the group's last
// lane (every add pairs the same two subtrees as the tree; fp32 addition is
// commutative).  The sign dword is an OR over the same shifts; a nibble dword
// collects its four bytes from the lanes that hold them (an OR over row_ror or
// XOR partners).  Workgroup = 4 waves x kRowsPerWave rows.
constexpr int kRowsPerWave = 8;
constexpr int kRowsPerWg = 4 * kRowsPerWave;

// Raw bytes of one lane's BPL blocks (8 per block for bf16, 16 for fp32),
// read with non-temporal loads: every weight is read once, and streaming it
// past the caches measured up to 16% faster (fake-quant, 8192 x 8192 bf16).
template <bool BF16, int BPL>
struct LaneRaw { uint4 q[BF16 ? BPL / 2 : BPL]; };

template <bool BF16, int BPL>
__device__ inline LaneRaw<BF16, BPL> load_lane(const char* p) {
  LaneRaw<BF16, BPL> r;
#pragma unroll
  for (int h = 0; h < (BF16 ? BPL / 2 : BPL); ++h) {
    typedef unsigned int v4u __attribute__((ext_vector_type(4)));
    const v4u t = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p) + h);
    r.q[h] = make_uint4(t.x, t.y, t.z, t.w);
  }
  return r;
}

// The 4 weights of block j of a lane as fp32.
template <bool BF16, int BPL>
__device__ inline void block_values(const LaneRaw<BF16, BPL>& r, int j, float v[4]) {
  if constexpr (BF16) {
    const uint4 u = r.q[j >> 1];
    const uint32_t d0 = (j & 1) ? u.z : u.x, d1 = (j & 1) ? u.w : u.y;
    v[0] = __uint_as_float(d0 << 16);
    v[1] = __uint_as_float(d0 & 0xFFFF0000u);
    v[2] = __uint_as_float(d1 << 16);
    v[3] = __uint_as_float(d1 & 0xFFFF0000u);
  } else {
    const uint4 u = r.q[j];
    v[0] = __uint_as_float(u.x); v[1] = __uint_as_float(u.y);
    v[2] = __uint_as_float(u.z); v[3] = __uint_as_float(u.w);
  }
}

template <bool BF16, int DENSE, int BPL>
__global__ __launch_bounds__(256) void quantize_pack_kernel(
    const void* __restrict__ w, int64_t n, int64_t k, uint8_t* __restrict__ packed,
    float* __restrict__ alpha_direct, float* __restrict__ sb_sums, void* __restrict__ dense = nullptr) {
  static_assert(BPL == 2 || BPL == 4, "blocks per lane");
  constexpr int L = 32 / BPL;         // lanes per superblock
  constexpr int SPW = 64 / L;         // superblocks per wave row
  const int64_t nsb = k / kSuperblock;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int s = lane / L, i = lane % L;
  const int64_t g = (int64_t)blockIdx.x * SPW + s;  // this lane's superblock
  const bool gv = g < nsb;
  const int64_t col = g * kSuperblock + i * (4 * BPL);
  const int64_t row0 = (int64_t)blockIdx.y * kRowsPerWg + wave * kRowsPerWave;

  // code of every (zero position, positive flags) pair
  __shared__ uint8_t code_tab[64];
  if (DENSE == 0 && threadIdx.x < 64)
    code_tab[threadIdx.x] = (uint8_t)block_code(threadIdx.x >> 4, unpermute_pos(threadIdx.x & 15));

  // every load of this lane first (kRowsPerWave rows), unconditionally from
  // clamped in-bounds addresses (rows past n and superblocks past K repeat the
  // last valid ones and are never stored), so all of them are in flight at once
  constexpr int64_t kElem = BF16 ? 2 : 4;
  const int64_t ccol = (gv ? g : nsb - 1) * kSuperblock + i * (4 * BPL);
  LaneRaw<BF16, BPL> lw[kRowsPerWave];
#pragma unroll
  for (int it = 0; it < kRowsPerWave; ++it) {
    const int64_t row = row0 + it < n ? row0 + it : n - 1;
    lw[it] = load_lane<BF16, BPL>(reinterpret_cast<const char*>(w) + (row * k + ccol) * kElem);
  }

  // this lane's records of row row0 (+ it below): (superblock, row) record
  // g * n + row; the scale or superblock sum likewise
  const int64_t rec0 = g * n + row0;
  if constexpr (DENSE == 0) __syncthreads();  // the code table is written
  uint32_t* nib_rec = reinterpret_cast<uint32_t*>(packed) + rec0 * 4;
  uint32_t* sgn_rec = reinterpret_cast<uint32_t*>(packed + (DENSE ? 0 : nibble_plane_bytes(n, k))) + rec0;
  float* al_rec = alpha_direct + rec0;
  float* sum_rec = sb_sums + row0 * nsb + g;

  float sums[kRowsPerWave];
  uint32_t sgns[kRowsPerWave];
  uint32_t zs[DENSE != 0 ? kRowsPerWave : 1];  // dense: the blocks' zero positions, 2 bits each
#pragma unroll
  for (int it = 0; it < kRowsPerWave; ++it) {
    const int64_t row = row0 + it;
    const bool valid = gv && row < n;
    uint32_t code[BPL];
    float bs[BPL];
    float wv[BPL][4];
#pragma unroll
    for (int j = 0; j < BPL; ++j) {
      block_values<BF16, BPL>(lw[it], j, wv[j]);
      const uint32_t z = block_zero(wv[j], bs[j]);
      if constexpr (DENSE != 0) {
        code[j] = z << 2;  // only the zero position is used
      } else {
        uint32_t pp;
        if constexpr (BF16) {
          const uint4 u = lw[it].q[j >> 1];
          pp = pos_perm_bf16((j & 1) ? u.z : u.x, (j & 1) ? u.w : u.y);
        } else {
          pp = pos_perm_f32(wv[j]);
        }
        code[j] = code_tab[code_index(z, pp)];
      }
    }

    // superblock sum: tree levels inside the lane, then across the L lanes
    float sum;
    if constexpr (BPL == 2) sum = bs[0] + bs[1];
    else sum = (bs[0] + bs[1]) + (bs[BPL - 2] + bs[BPL - 1]);
    sum += dpp<kShr1>(sum);
    sum += dpp<kShr2>(sum);
    sum += dpp<kShr4>(sum);
    if constexpr (L == 16) sum += dpp<kShr8>(sum);

    if constexpr (DENSE != 0) {
      sums[it] = sum;
      uint32_t zz = 0;  // zero position of block j in bits 2j, 2j+1
#pragma unroll
      for (int j = 0; j < BPL; ++j) zz |= (code[j] >> 2) << (2 * j);
      zs[it] = zz;
      continue;
    }

    // sign dword: bit b of superblock = sign bit of block b
    uint32_t sgn = 0;
#pragma unroll
    for (int j = 0; j < BPL; ++j) sgn |= ((code[j] >> 4) & 1u) << j;
    sgn <<= BPL * i;
    sgn |= dpp<kShr1>(sgn);
    sgn |= dpp<kShr2>(sgn);
    sgn |= dpp<kShr4>(sgn);
    if constexpr (L == 16) sgn |= dpp<kShr8>(sgn);

    // nibble dword d holds blocks 2d + 8b (low nibble of byte b) and 2d + 1 + 8b
    if constexpr (BPL == 2) {
      // lane i holds byte i >> 2 of dword i & 3
      uint32_t d = ((code[0] & 15u) | ((code[1] & 15u) << 4)) << (8 * (i >> 2));
      d |= dpp<kRor4>(d);
      d |= dpp<kRor8>(d);
      if (valid && i < 4) nib_rec[it * 4 + i] = d;
    } else {
      // lane i holds byte i >> 1 of dwords 2 (i & 1) and 2 (i & 1) + 1
      uint32_t d0 = ((code[0] & 15u) | ((code[1] & 15u) << 4)) << (8 * (i >> 1));
      uint32_t d1 = ((code[BPL - 2] & 15u) | ((code[BPL - 1] & 15u) << 4)) << (8 * (i >> 1));
      d0 |= dpp<kQuadXor2>(d0);
      d1 |= dpp<kQuadXor2>(d1);
      d0 |= (uint32_t)__builtin_amdgcn_ds_swizzle((int)d0, kSwzXor4);
      d1 |= (uint32_t)__builtin_amdgcn_ds_swizzle((int)d1, kSwzXor4);
      if (valid && i < 2) *reinterpret_cast<uint2*>(nib_rec + it * 4 + 2 * i) = make_uint2(d0, d1);
    }
    sums[it] = sum;
    sgns[it] = sgn;
  }
  if constexpr (DENSE != 0) {
    // Lane L-1-it of each group collects row it's sum; one division gives
    // every row's scale, which row_shr and a broadcast hand back to the group.
    float sv = sums[0];
#pragma unroll
    for (int it = 1; it < kRowsPerWave; ++it) {
      const float sh = dpp_shl(sums[it], it);
      if (i == L - 1 - it) sv = sh;
    }
    const float av = (float)((double)sv / 96.0);
    const int rit = L - 1 - i;
    if (gv && rit < kRowsPerWave && row0 + rit < n) al_rec[rit] = av;
#pragma unroll
    for (int it = 0; it < kRowsPerWave; ++it) {
      const float at = it == 0 ? av : dpp_shr(av, it);  // row it's scale in lane L-1
      const float a = __int_as_float(
          __builtin_amdgcn_ds_swizzle(__float_as_int(at), L == 16 ? kSwzLast16 : kSwzLast8));
      const int64_t row = row0 + it;
      if (!(gv && row < n)) continue;
#pragma unroll
      for (int j = 0; j < BPL; ++j) {
        float wv[4];
        block_values<BF16, BPL>(lw[it], j, wv);
        const uint32_t z = (zs[it] >> (2 * j)) & 3u;
        float f[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) f[e] = (uint32_t)e == z ? 0.f : (wv[e] > 0.f ? a : -a);
        const int64_t off = row * k + col + 4 * j;
        if constexpr (DENSE == SHERRY_F32 + 1) {
          *reinterpret_cast<float4*>(reinterpret_cast<float*>(dense) + off) = make_float4(f[0], f[1], f[2], f[3]);
        } else {
          uint2 v;
          v.x = (uint32_t)f32_to_bf16_rne(f[0]) | ((uint32_t)f32_to_bf16_rne(f[1]) << 16);
          v.y = (uint32_t)f32_to_bf16_rne(f[2]) | ((uint32_t)f32_to_bf16_rne(f[3]) << 16);
          *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(dense) + off) = v;
        }
      }
    }
  }
  if constexpr (DENSE == 0) {
    // Lane L-1-it of each group collects row it's superblock sum and sign
    // dword (both sit in lane L-1), so one division and one store of each
    // serve all the rows.
    static_assert(kRowsPerWave <= L && kRowsPerWave <= 8, "rows gathered by row_shl");
    float sv = sums[0];
    uint32_t sg = sgns[0];
#pragma unroll
    for (int it = 1; it < kRowsPerWave; ++it) {
      const float sh = dpp_shl(sums[it], it);
      const uint32_t gh = dpp_shl(sgns[it], it);
      if (i == L - 1 - it) { sv = sh; sg = gh; }
    }
    const int rit = L - 1 - i;  // the row this lane now holds
    if (gv && rit < kRowsPerWave && row0 + rit < n) {
      sgn_rec[rit] = sg;
      if (alpha_direct) {
        al_rec[rit] = (float)((double)sv / 96.0);
      } else {
        sum_rec[rit * nsb] = sv;
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

// ---------------------------------------------------------------------------
// Row-group quantize + pack (K up to kRowsMaxSb superblocks): the codes as
// above with fewer instructions per block, and the scales of every
// granularity finished in the same launch (per_tensor: down to one partial
// per row group).
//
// Work unit: one chunk (four superblocks) of a group of 8 rows, one wave: lane
// (s, i) reads blocks 2i, 2i + 1 of superblock 4c + s of each of the 8 rows,
// all 8 loads first.  Per block, block_zero gives the zero position and the
// kept-|w| sum, a dot product of the positive-flag bytes gives the table
// index 4 * pos + z, and one LDS table read returns the block's nibble and
// sign bit already placed for the lane's byte.  The 16 lanes of a superblock
// combine with row_ror DPP moves: the four nibble dwords, the sign dword (in
// every lane), and the superblock's kept-|w| sum, which lane 15 ends with as
// the index-order pairwise tree over the 32 blocks (every add pairs the same
// two subtrees as the tree; fp32 addition is commutative).  Each row's sign
// dword and sum are then gathered into lane 15 - row of the group, so one
// store covers the 8 rows.
//
// per_group G = 128 (kRowsDirect): workgroup (x, y) = chunk x of rows 32 y ..
// (four waves, 8 rows each) -- consecutive workgroups read adjacent spans of
// the same rows -- and each superblock sum over 96 is stored at once.  Every
// other scale needs a row's sums from all chunks, so there a workgroup of
// min(8, chunks) waves owns one row group and walks its chunks, the sums wait
// in LDS, and after a barrier:
//   kRowsGroup    per_group G = 128 r: the pairwise tree over each group's r
//                 sums, over 96 r;
//   kRowsChannel  per_channel: the tree over the row's nsb sums (E per lane,
//                 then an XOR butterfly: the index-order tree over 64 E values,
//                 i.e. over the row padded to a power of two), over 96 nsb;
//   kRowsTensor   per_tensor with nsb a power of two: a row is then an aligned
//                 subtree of the tree over the flat weight order, and so is
//                 the row group; the workgroup writes that subtree's root for
//                 the tree levels that follow;
//   kRowsSums     per_tensor otherwise: the superblock sums, row-major, for
//                 the tree levels.
// Measured on the 8192 x 8192 bf16 weight, 100 calls back to back:
// per_group 128 29.4 us, per_channel 30.2 us, per_tensor 33.6 us (with the
// tree launch).  Against the superblock-tile kernel and its second-stage
// launches the row-group kernel needs 18% fewer VALU instructions per weight
// (integer-domain selection) at about the same time: the memory pipeline, not
// the ALU, sets it.
constexpr int kRowsGroup = 0, kRowsChannel = 1, kRowsTensor = 2, kRowsSums = 3, kRowsDirect = 4;
constexpr int64_t kRowsMaxSb = 512;  // 8 rows x 512 superblock sums in LDS = 16 KB
constexpr int kRgRows = kRowsPerWave;  // rows per wave and per row group
// the fused fake quant: 4 rows per wave (its codes wait in LDS until the row
// scales are known, so fewer rows per row group mean more, shorter-lived
// workgroups; 3.6% faster than 8 for per_channel, slower for quantize)
constexpr int kRgRowsDense = 4;
constexpr int kRgWaves = 4;            // waves per workgroup, per_group 128 (one chunk per wave)
// waves per workgroup (at most) of the modes that walk a row group's chunks:
// 8 waves per SIMD in one round for 8192-wide rows; 1-2.5% faster than 4 for
// per_channel / per_tensor and 10% for the fused fake quant, 16 slower
constexpr int kRgWavesWalk = 8;
constexpr int64_t kDenseMaxSb = 128;   // fused fake quant: 8 rows x 128 superblocks of codes in LDS = 32 KB
constexpr int kRor1 = 0x121, kRor2 = 0x122;

// row_ror moves: every lane of the row has a source, so no bound control
template <int CTRL>
__device__ inline uint32_t dpp_ror(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, true);
}
template <int CTRL>
__device__ inline float dpp_ror(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}

// bytes 0..3 = 0xFF where bf16 weights w0..w3 are > 0 (d0 = w0 | w1 << 16,
// d1 = w2 | w3 << 16): the sign bit of each saturated 16-bit 0 - w (set
// exactly for w in 1 .. 0x7FFF; -0, 0x8000, saturates to 0x7FFF), gathered
// by v_perm's sign-replicating selectors 8..11 (bits 15 / 31 of each source).
__device__ inline uint32_t positive_bytes_bf16(uint32_t d0, uint32_t d1) {
  uint32_t t0, t1;
  asm("v_pk_sub_i16 %0, 0, %2 clamp\n"
      "v_pk_sub_i16 %1, 0, %3 clamp"
      : "=&v"(t0), "=&v"(t1)
      : "v"(d0), "v"(d1));
  return __builtin_amdgcn_perm(t1, t0, 0x0B0A0908u);
}

// Table index h of block j (0, 1) of a lane, returned as the byte offset 2h
// of its 16-bit entry; kept = the block's kept-|w| sum, the tree
// ((k0 + k1) + (k2 + k3)) with the zero position's term +0.
//
// bf16: h = 8 * pos + (c01 | c23 << 1 | c << 2), pos = the positive flags of
// weights 0..3 in bits 0..3, c01 = |w1| < |w0|, c23 = |w3| < |w2|, c = the
// smaller of the right pair is below the smaller of the left pair (so the
// zero is 2 + c23 if c, else c01: the smallest |w|, lowest index on ties).
// The magnitudes are compared as 15-bit integers, which order like the
// values they encode; the pairs (w0, w2) and (w1, w3) share a packed 16-bit
// operation.  A pair's kept sum is its larger magnitude plus its smaller one
// where the zero is in the other pair, +0 where it is not: the same fp32
// additions the tree makes, operands commuted.
// fp32: h = 4 * pos + z.
typedef short i16x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
__device__ inline i16x2 as_i16x2(uint32_t v) { return __builtin_bit_cast(i16x2, v); }
__device__ inline u16x2 as_u16x2(uint32_t v) { return __builtin_bit_cast(u16x2, v); }

template <bool BF16>
__device__ inline uint32_t lane_block(const LaneRaw<BF16, 2>& r, int j, float& kept) {
  if constexpr (BF16) {
    const uint32_t d0 = j ? r.q[0].z : r.q[0].x, d1 = j ? r.q[0].w : r.q[0].y;
    const uint32_t a = __builtin_amdgcn_perm(d1, d0, 0x05040100u) & 0x7FFF7FFFu;  // |w0|, |w2|
    const uint32_t b = __builtin_amdgcn_perm(d1, d0, 0x07060302u) & 0x7FFF7FFFu;  // |w1|, |w3|
    const uint32_t t1 = __builtin_bit_cast(uint32_t, as_i16x2(b) - as_i16x2(a));  // signs: c01, c23
    const uint32_t mn = __builtin_bit_cast(uint32_t, __builtin_elementwise_min(as_u16x2(a), as_u16x2(b)));
    const uint32_t mx = __builtin_bit_cast(uint32_t, __builtin_elementwise_max(as_u16x2(a), as_u16x2(b)));
    const uint32_t sw = __builtin_amdgcn_alignbit(mn, mn, 16);                    // halves swapped
    const uint32_t t2 = __builtin_bit_cast(uint32_t, as_i16x2(sw) - as_i16x2(mn)); // sign of the low half: c
    // kept smaller magnitudes: the left pair's if c, else the right pair's
    const uint32_t all_c = __builtin_amdgcn_perm(t2, t2, 0x08080808u);            // c ? ~0 : 0
    const uint32_t ms = __builtin_amdgcn_bitop3_b32(mn, all_c, 0xFFFF0000u, 0x60); // mn & (all_c ^ K)
    const float left = __uint_as_float(mx << 16) + __uint_as_float(ms << 16);
    const float right = __uint_as_float(mx & 0xFFFF0000u) + __uint_as_float(ms & 0xFFFF0000u);
    kept = left + right;
    // bytes of -1 where set: positive flags times -16 .. -128, c01 / c23 / c times -2, -4, -8
    const uint32_t cbytes = __builtin_amdgcn_perm(t2, t1, 0x0C0A0908u);
    const int ip = __builtin_amdgcn_sdot4((int)positive_bytes_bf16(d0, d1), (int)0x80C0E0F0u, 0, false);
    return (uint32_t)__builtin_amdgcn_sdot4((int)cbytes, (int)0x00F8FCFEu, ip, false);
  } else {
    float v[4];
    const uint4 u = r.q[j];
    v[0] = __uint_as_float(u.x); v[1] = __uint_as_float(u.y);
    v[2] = __uint_as_float(u.z); v[3] = __uint_as_float(u.w);
    const uint32_t z = block_zero(v, kept);
    return 2u * z | (v[0] > 0.f ? 8u : 0u) | (v[1] > 0.f ? 16u : 0u) | (v[2] > 0.f ? 32u : 0u) |
           (v[3] > 0.f ? 64u : 0u);
  }
}
// The block code of a table index h of lane_block.
template <bool BF16>
__device__ inline uint32_t lane_index_code(uint32_t idx) {
  if constexpr (BF16) {
    const uint32_t z = (idx & 4u) ? 2u + ((idx >> 1) & 1u) : (idx & 1u);
    return block_code(z, idx >> 3);
  } else {
    return block_code(idx & 3u, idx >> 2);
  }
}
template <bool BF16>
constexpr int kLaneIndices = BF16 ? 128 : 64;

// p, known to be the same in every lane, as a scalar global-memory address.
typedef __attribute__((address_space(1))) const char gchar;
__device__ inline gchar* uniform_ptr(const char* p) {
  const uint64_t u = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return reinterpret_cast<gchar*>(((uint64_t)hi << 32) | lo);
}
// The two blocks of a bf16 lane at row address p (scalar) + off.
__device__ inline LaneRaw<true, 2> load_lane_at(gchar* p, uint32_t off) {
  typedef unsigned int v4u __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(1))) const v4u gv4u;
  const v4u t = __builtin_nontemporal_load(reinterpret_cast<gv4u*>(p + off));
  LaneRaw<true, 2> r;
  r.q[0] = make_uint4(t.x, t.y, t.z, t.w);
  return r;
}
__device__ inline LaneRaw<false, 2> load_lane_at_f32(gchar* p, uint32_t off) {
  typedef unsigned int v4u __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(1))) const v4u gv4u;
  LaneRaw<false, 2> r;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const v4u t = __builtin_nontemporal_load(reinterpret_cast<gv4u*>(p + off) + h);
    r.q[h] = make_uint4(t.x, t.y, t.z, t.w);
  }
  return r;
}

// In-place pairwise tree over x[0 .. r) padded with +0 to a power of two
// (adds that would take a padded +0 leave the value as it is).
__device__ inline float tree_inplace(float* x, int64_t r) {
  int64_t width = 1;
  while (width < r) width <<= 1;
  for (int64_t h = 1; h < width; h <<= 1)
    for (int64_t j = 0; j + h < r; j += 2 * h) x[j] = x[j] + x[j + h];
  return x[0];
}

// DENSE (per_channel and per_group G > 128, rows of up to kDenseMaxSb
// superblocks): the fused fake-quant forward -- no planes; the codes stay in
// LDS and a last phase writes T * alpha densely (fp32, or bf16 rounded to
// nearest even) once the scales are known.  bf16: eight waves per SIMD, a
// register budget of 64; fp32 (twice the load registers): four, so nothing
// spills (1.8x faster than spilling at eight).
template <bool BF16, int MODE, int E, int DENSE = 0, int WM = kRgWaves, int RWT = kRgRows>
__global__ __launch_bounds__(64 * WM) __attribute__((amdgpu_waves_per_eu(BF16 ? 8 : 4)))
void quantize_rowgroup_kernel(
    const void* __restrict__ w, int64_t n, int64_t k, int group_r, uint8_t* __restrict__ packed,
    float* __restrict__ alpha, float* __restrict__ ws, void* __restrict__ dense = nullptr) {
  static_assert(DENSE == 0 || MODE == kRowsGroup || MODE == kRowsChannel, "dense output needs row-local scales");
  constexpr int RW = RWT;
  // [RW][4 C] superblock kept-|w| sums (unless per_group 128); with DENSE
  // then [RW][4 C][16] 16-bit block-pair entries (the codes) and the scales
  extern __shared__ float sb_lds[];
  __shared__ uint16_t tab[2 * 128];  // [slot][h]: block 2i's entry, then block 2i + 1's
  __shared__ float roots[RW];
  const int64_t nsb = k / kSuperblock;
  const int64_t C = (nsb + 3) / 4;  // chunks of four superblocks
  const int lane = threadIdx.x & 63, W = blockDim.x >> 6;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));  // uniform: scalar row addresses
  const int s = lane >> 4, i = lane & 15;
  constexpr bool direct = MODE == kRowsDirect;
  const int64_t grp = blockIdx.x;  // row group (modes other than direct)
  const int64_t row0 = direct ? ((int64_t)blockIdx.y * W + wave) * RW : grp * RW;

  // entry = the block's nibble and sign bit where the lane's byte wants them:
  // block 2i: nibble bits 0..3, sign bit 8; block 2i + 1: bits 4..7, bit 9
  for (int t = threadIdx.x; t < kLaneIndices<BF16>; t += blockDim.x) {
    const uint32_t code = lane_index_code<BF16>((uint32_t)t);
    tab[t] = (uint16_t)((code & 15u) | ((code >> 4) << 8));
    tab[128 + t] = (uint16_t)(((code & 15u) << 4) | ((code >> 4) << 9));
  }
  constexpr int64_t kElem = BF16 ? 2 : 4;
  // v_perm selector putting the low byte of its second source at byte i / 4
  const uint32_t sel_nib = 0x0C0C0C0Cu & ~(0xFFu << (8 * (i >> 2)));
  uint32_t* nib_plane = reinterpret_cast<uint32_t*>(packed);
  uint32_t* sgn_plane = reinterpret_cast<uint32_t*>(packed + (DENSE ? 0 : nibble_plane_bytes(n, k)));
  uint16_t* codes_lds = reinterpret_cast<uint16_t*>(sb_lds + RW * 4 * C);     // DENSE only
  float* scale_lds = reinterpret_cast<float*>(codes_lds + RW * 4 * C * 16);  // DENSE only: [RW][groups]

  // rows past row0 + last repeat it (last < RW; negative for a wave wholly past n)
  const int last = n - 1 - row0 < RW ? (int)(n - 1 - row0) : RW;
  // one chunk of the 8 rows, from registers already loaded
  auto process = [&](const LaneRaw<BF16, 2>(&lw)[RW], int64_t c) {
    const int64_t g = 4 * c + s;  // this lane's superblock
    const bool gv = g < nsb;
    const int64_t rec0 = g * n + row0;  // record of (g, row0); rows follow
    uint32_t* nib_rec = DENSE ? nullptr : nib_plane + rec0 * 4 + i;
    float sv = 0.f;
    uint32_t sgv = 0;
#pragma unroll
    for (int it = 0; it < RW; ++it) {
      float k0, k1;
      const uint32_t i0 = lane_block<BF16>(lw[it], 0, k0);
      const uint32_t i1 = lane_block<BF16>(lw[it], 1, k1);
      const char* tb = reinterpret_cast<const char*>(tab);
      const uint32_t comb = (uint32_t)*reinterpret_cast<const uint16_t*>(tb + i0) +
                            (uint32_t)*reinterpret_cast<const uint16_t*>(tb + 256 + i1);
      // nibble dwords: lane i's byte is byte i / 4 of dword i % 4
      uint32_t nib = __builtin_amdgcn_perm(0u, comb, sel_nib);
      nib |= dpp_ror<kRor4>(nib);
      nib |= dpp_ror<kRor8>(nib);
      if constexpr (DENSE != 0) {
        codes_lds[(it * 4 * C + g) * 16 + i] = (uint16_t)comb;  // (g < 4 C always)
      } else {
        if (gv && it <= last && i < 4) nib_rec[it * 4] = nib;
      }
      // sign dword (every lane of the group): bit b = sign bit of block b
      uint32_t sg = ((comb >> 8) & 3u) << (2 * i);
      sg |= dpp_ror<kRor1>(sg);
      sg |= dpp_ror<kRor2>(sg);
      sg |= dpp_ror<kRor4>(sg);
      sg |= dpp_ror<kRor8>(sg);
      // superblock sum: lane 15 pairs (14, 15), then (13, 15), (11, 15), (7, 15)
      float sum = k0 + k1;
      sum += dpp_ror<kRor1>(sum);
      sum += dpp_ror<kRor2>(sum);
      sum += dpp_ror<kRor4>(sum);
      sum += dpp_ror<kRor8>(sum);
      // lane 15 - it of each group keeps row it's sum (from lane 15) and sign
      // dword (its own), so one store of each serves the 8 rows
      if (it == 0) {
        sv = sum;
        sgv = sg;
      } else {
        const float sh = dpp_shl(sum, it);
        if (i == 15 - it) { sv = sh; sgv = sg; }
      }
    }
    const int rit = 15 - i;  // the row this lane now holds
    if (gv && rit < RW && rit <= last) {
      if constexpr (DENSE == 0) sgn_plane[rec0 + rit] = sgv;
      if (direct) alpha[rec0 + rit] = (float)((double)sv / 96.0);
      else sb_lds[rit * 4 * C + g] = sv;
    }
  };
  // every load of a chunk at once, from clamped in-bounds addresses (rows
  // past n and superblocks past K repeat the last valid ones, never stored)
  auto load = [&](LaneRaw<BF16, 2>(&lw)[RW], int64_t c) {
    // row addresses in scalar registers; the lane adds a 32-bit offset inside the chunk
    const int64_t g = 4 * c + s < nsb ? 4 * c + s : nsb - 1;
    const uint32_t off = (uint32_t)(((g - 4 * c) * kSuperblock + 8 * i) * kElem);
    const char* p = reinterpret_cast<const char*>(w) + (row0 * k + 4 * c * kSuperblock) * kElem;
#pragma unroll
    for (int it = 0; it < RW; ++it) {
      gchar* rp = uniform_ptr(p + (int64_t)(it < last ? it : last) * k * kElem);
      if constexpr (BF16) lw[it] = load_lane_at(rp, off);
      else lw[it] = load_lane_at_f32(rp, off);
    }
  };

  // direct: this wave's one chunk; otherwise the row group's chunks in turn
  const int64_t stride = direct ? (int64_t)gridDim.x : W;
  int64_t c = direct ? (int64_t)blockIdx.x : wave;
  __syncthreads();  // the table is written
  for (; c < C; c += stride) {
    LaneRaw<BF16, 2> lw[RW];
    load(lw, c);
    process(lw, c);
  }
  if constexpr (!direct) {
    __syncthreads();  // every superblock sum of the row group is in LDS
    if constexpr (MODE == kRowsGroup) {
      const int64_t groups = nsb / group_r;
      const double denom = (double)group_r * kSuperblock / 4.0 * 3.0;
      for (int64_t t = threadIdx.x; t < RW * groups; t += blockDim.x) {
        const int64_t rit = t / groups, gg = t % groups;
        const float a = (float)((double)tree_inplace(sb_lds + rit * 4 * C + gg * group_r, group_r) / denom);
        if (row0 + rit < n) alpha[gg * n + row0 + rit] = a;
        if constexpr (DENSE != 0) scale_lds[rit * groups + gg] = a;
      }
    } else if constexpr (MODE == kRowsSums) {
      for (int64_t t = threadIdx.x; t < RW * nsb; t += blockDim.x) {
        const int64_t rit = t / nsb, g = t % nsb;
        if (row0 + rit < n) ws[(row0 + rit) * nsb + g] = sb_lds[rit * 4 * C + g];
      }
    } else {
      for (int rit = wave; rit < RW; rit += W) {
        const float* rs = sb_lds + rit * 4 * C;
        float v[E];
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const int64_t idx = (int64_t)lane * E + e;
          v[e] = (row0 + rit < n && idx < nsb) ? rs[idx] : 0.f;
        }
#pragma unroll
        for (int h = E; h > 1; h >>= 1)
#pragma unroll
          for (int e = 0; e < h / 2; ++e) v[e] = v[2 * e] + v[2 * e + 1];
        float sum = v[0];
        sum += __shfl_xor(sum, 1);
        sum += __shfl_xor(sum, 2);
        sum += __shfl_xor(sum, 4);
        sum += __shfl_xor(sum, 8);
        sum += __shfl_xor(sum, 16);
        sum += __shfl_xor(sum, 32);
        if constexpr (MODE == kRowsChannel) {
          const float a = (float)((double)sum / ((double)k / 4.0 * 3.0));
          if (lane == 0 && row0 + rit < n) alpha[row0 + rit] = a;
          if constexpr (DENSE != 0)
            if (lane == 0) scale_lds[rit] = a;
        } else {
          if (lane == 0) roots[rit] = sum;  // rows past n: +0
        }
      }
      if constexpr (MODE == kRowsTensor) {
        __syncthreads();
        if (threadIdx.x == 0) ws[grp] = tree_inplace(roots, RW);
      }
    }
  }
  if constexpr (DENSE != 0) {
    // Dense T * alpha (the fake-quant forward): per (row, chunk) a wave writes
    // 4 superblocks, lane (s, i) the 8 weights of blocks 2i, 2i + 1 of
    // superblock 4c + s from that pair's entry: each block's nibble (z << 2 |
    // p1 << 1 | p0) and sign bit (its code is sign << 4 | nibble).
    __syncthreads();  // every scale of the row group is in LDS
    const int64_t groups = MODE == kRowsChannel ? 1 : nsb / group_r;
    for (int64_t task = wave; task < RW * C; task += W) {
      const int rit = (int)(task / C);
      const int64_t c = task % C, g = 4 * c + s, row = row0 + rit;
      if (row >= n || g >= nsb) continue;
      const float a = scale_lds[rit * groups + (MODE == kRowsChannel ? 0 : g / group_r)];
      const uint32_t comb = codes_lds[(rit * 4 * C + g) * 16 + i];
      float f[8];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint32_t code = (((comb >> (8 + j)) & 1u) << 4) | ((comb >> (4 * j)) & 15u);
        int t[4];
        decode_block(code, t);
#pragma unroll
        for (int e = 0; e < 4; ++e) f[4 * j + e] = t[e] == 0 ? 0.f : (t[e] > 0 ? a : -a);
      }
      const int64_t off = row * k + g * kSuperblock + 8 * i;
      if constexpr (DENSE == SHERRY_F32 + 1) {
        float4* d = reinterpret_cast<float4*>(reinterpret_cast<float*>(dense) + off);
        d[0] = make_float4(f[0], f[1], f[2], f[3]);
        d[1] = make_float4(f[4], f[5], f[6], f[7]);
      } else {
        uint32_t hv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          hv[e] = (uint32_t)f32_to_bf16_rne(f[2 * e]) | ((uint32_t)f32_to_bf16_rne(f[2 * e + 1]) << 16);
        *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(dense) + off) = make_uint4(hv[0], hv[1], hv[2], hv[3]);
      }
    }
  }
}

// Grid: x = groups of 2*BPL superblocks, y = tiles of kRowsPerWg rows, so
// consecutive workgroups read adjacent spans of the same rows.
inline dim3 quantize_grid(int64_t n, int64_t nsb) {
  constexpr int spw = 2 * SHERRY_Q_BPL;
  return dim3((unsigned)((nsb + spw - 1) / spw), (unsigned)((n + kRowsPerWg - 1) / kRowsPerWg));
}

}  // namespace

QuantizePlan plan_quantize(int64_t n, int64_t k, int gran, int group_size) {
  QuantizePlan p{};
  const int64_t nsb = k / kSuperblock;
  if (nsb <= kRowsMaxSb) {
    p.rows = true;
    p.wg_rows = kRgRows;
    const int64_t wgs = (n + p.wg_rows - 1) / p.wg_rows;
    if (gran == SHERRY_PER_GROUP) {
      p.rows_mode = kRowsGroup;
    } else if (gran == SHERRY_PER_CHANNEL) {
      p.rows_mode = kRowsChannel;
    } else {
      const bool pow2 = (nsb & (nsb - 1)) == 0;
      p.rows_mode = pow2 ? kRowsTensor : kRowsSums;
      p.sb_sums = pow2 ? wgs : n * nsb;  // workgroup subtree roots, or superblock sums
      p.chunk = kTreeChunk;
      p.chunks = 2 * ((p.sb_sums + kTreeChunk - 1) / kTreeChunk);
    }
    p.workspace_bytes = (size_t)(p.sb_sums + p.chunks) * sizeof(float);
    return p;
  }
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

namespace {

// per_tensor: tree levels over `real` partials at ws (each level one launch
// of aligned 4096-value chunks) down to the one scale.
void launch_tree_levels(const QuantizePlan& p, const float* in, int64_t real, double denom, float* alpha,
                        float* ws, hipStream_t s) {
  float* bufs[2] = {ws + p.sb_sums, ws + p.sb_sums + p.chunks / 2};
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

template <bool BF16, int MODE, int E>
void launch_rows(const QuantizePlan& p, int64_t n, int64_t k, int group_r, const void* w, uint8_t* packed,
                 float* alpha, float* ws, hipStream_t s) {
  const int64_t nsb = k / kSuperblock;
  const int64_t chunks = (nsb + 3) / 4;
  constexpr bool direct = MODE == kRowsDirect;
  constexpr int WM = direct ? kRgWaves : kRgWavesWalk;
  const int waves = direct ? kRgWaves : (int)(chunks < WM ? chunks : WM);
  const size_t lds = direct ? 0 : (size_t)kRgRows * 4 * chunks * sizeof(float);
  const int64_t groups = (n + kRgRows - 1) / kRgRows;
  const dim3 grid = direct ? dim3((unsigned)chunks, (unsigned)((groups + waves - 1) / waves)) : dim3((unsigned)groups);
  hipLaunchKernelGGL((quantize_rowgroup_kernel<BF16, MODE, E, 0, WM>), grid, dim3(64 * waves), lds, s, w, n, k, group_r,
                     packed, alpha, ws);
}

template <bool BF16>
void launch_rows_mode(const QuantizePlan& p, int64_t n, int64_t k, int group_r, const void* w, uint8_t* packed,
                      float* alpha, float* ws, hipStream_t s) {
  const int64_t nsb = k / kSuperblock;
  const int64_t e = (nsb + 63) / 64;
  switch (p.rows_mode) {
    case kRowsGroup:
      if (group_r == 1) launch_rows<BF16, kRowsDirect, 1>(p, n, k, group_r, w, packed, alpha, ws, s);
      else launch_rows<BF16, kRowsGroup, 1>(p, n, k, group_r, w, packed, alpha, ws, s);
      break;
    case kRowsSums: launch_rows<BF16, kRowsSums, 1>(p, n, k, group_r, w, packed, alpha, ws, s); break;
#define SHERRY_ROWS_E(M)                                                                        \
  if (e <= 1) launch_rows<BF16, M, 1>(p, n, k, group_r, w, packed, alpha, ws, s);               \
  else if (e <= 2) launch_rows<BF16, M, 2>(p, n, k, group_r, w, packed, alpha, ws, s);          \
  else if (e <= 4) launch_rows<BF16, M, 4>(p, n, k, group_r, w, packed, alpha, ws, s);          \
  else launch_rows<BF16, M, 8>(p, n, k, group_r, w, packed, alpha, ws, s);
    case kRowsChannel: SHERRY_ROWS_E(kRowsChannel) break;
    default: SHERRY_ROWS_E(kRowsTensor) break;
#undef SHERRY_ROWS_E
  }
}

}  // namespace

hipError_t launch_quantize_pack(const QuantizePlan& p, int64_t n, int64_t k, int gran,
                                int group_size, const void* w, bool w_bf16, uint8_t* packed,
                                float* alpha, float* ws, hipStream_t s) {
  const int64_t nsb = k / kSuperblock;
  if (p.rows) {
    static_assert(kRowsMaxSb <= 64 * 8, "row trees hold at most 8 sums per lane");
    const int group_r = gran == SHERRY_PER_GROUP ? group_size / kSuperblock : 1;
    if (w_bf16) launch_rows_mode<true>(p, n, k, group_r, w, packed, alpha, ws, s);
    else launch_rows_mode<false>(p, n, k, group_r, w, packed, alpha, ws, s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || gran != SHERRY_PER_TENSOR) return e;
    launch_tree_levels(p, ws, p.sb_sums, (double)n * (double)k / 4.0 * 3.0, alpha, ws, s);
    return hipGetLastError();
  }
  const dim3 grid = quantize_grid(n, nsb);
  float* direct = p.direct_alpha ? alpha : nullptr;
  if (w_bf16) {
    hipLaunchKernelGGL((quantize_pack_kernel<true, 0, SHERRY_Q_BPL>), grid, dim3(256), 0, s, w, n, k, packed,
                       direct, ws, nullptr);
  } else {
    hipLaunchKernelGGL((quantize_pack_kernel<false, 0, SHERRY_Q_BPL>), grid, dim3(256), 0, s, w, n, k, packed,
                       direct, ws, nullptr);
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
    launch_tree_levels(p, ws, p.sb_sums, (double)n * (double)k / 4.0 * 3.0, alpha, ws, s);
  }
  return hipGetLastError();
}

FakeQuantPlan plan_fake_quant(int64_t n, int64_t k, int gran, int group_size) {
  FakeQuantPlan p{};
  p.fused = gran == SHERRY_PER_GROUP && group_size == kSuperblock;
  if (p.fused) return p;
  // row-local scales over rows of up to kDenseMaxSb superblocks: the
  // row-group kernel writes T * alpha itself once its rows' scales are known
  p.fused_rows = gran != SHERRY_PER_TENSOR && k / kSuperblock <= kDenseMaxSb;
  if (p.fused_rows) return p;
  p.packed_offset = 0;
  p.quant_ws_offset = ((size_t)(n * k / 32 * 5) + 255) / 256 * 256;
  p.workspace_bytes = p.quant_ws_offset + plan_quantize(n, k, gran, group_size).workspace_bytes;
  return p;
}

namespace {

template <bool BF16, int MODE, int E, int DENSE>
void launch_rows_dense(int64_t n, int64_t k, int group_r, const void* w, float* alpha, void* out, hipStream_t s) {
  const int64_t nsb = k / kSuperblock;
  const int64_t chunks = (nsb + 3) / 4;
  constexpr int WM = kRgWavesWalk;
  const int waves = (int)(chunks < WM ? chunks : WM);
  const int64_t groups = MODE == kRowsChannel ? 1 : nsb / group_r;
  constexpr int RW = kRgRowsDense;
  const size_t lds = (size_t)RW * 4 * chunks * (sizeof(float) + 16 * sizeof(uint16_t)) +
                     (size_t)RW * groups * sizeof(float);
  const dim3 grid((unsigned)((n + RW - 1) / RW));
  hipLaunchKernelGGL((quantize_rowgroup_kernel<BF16, MODE, E, DENSE, WM, RW>), grid, dim3(64 * waves), lds, s, w, n,
                     k, group_r, nullptr, alpha, nullptr, out);
}

template <bool BF16, int DENSE>
void launch_rows_dense_mode(int64_t n, int64_t k, int gran, int group_size, const void* w, float* alpha, void* out,
                            hipStream_t s) {
  if (gran == SHERRY_PER_GROUP) {
    launch_rows_dense<BF16, kRowsGroup, 1, DENSE>(n, k, group_size / kSuperblock, w, alpha, out, s);
    return;
  }
  const int64_t e = (k / kSuperblock + 63) / 64;  // sums per lane in the row tree
  if (e <= 1) launch_rows_dense<BF16, kRowsChannel, 1, DENSE>(n, k, 1, w, alpha, out, s);
  else launch_rows_dense<BF16, kRowsChannel, 2, DENSE>(n, k, 1, w, alpha, out, s);
}

}  // namespace

hipError_t launch_fake_quant(const FakeQuantPlan& p, int64_t n, int64_t k, int gran, int group_size,
                             const void* w, bool w_bf16, void* out, int out_dtype, float* alpha,
                             uint8_t* ws, hipStream_t s) {
  if (p.fused_rows) {
    static_assert(kDenseMaxSb <= 128, "row trees of at most 2 sums per lane");
    if (w_bf16) {
      if (out_dtype == SHERRY_F32) launch_rows_dense_mode<true, SHERRY_F32 + 1>(n, k, gran, group_size, w, alpha, out, s);
      else launch_rows_dense_mode<true, SHERRY_BF16 + 1>(n, k, gran, group_size, w, alpha, out, s);
    } else {
      if (out_dtype == SHERRY_F32) launch_rows_dense_mode<false, SHERRY_F32 + 1>(n, k, gran, group_size, w, alpha, out, s);
      else launch_rows_dense_mode<false, SHERRY_BF16 + 1>(n, k, gran, group_size, w, alpha, out, s);
    }
    return hipGetLastError();
  }
  if (p.fused) {
    const int64_t nsb = k / kSuperblock;
    const dim3 grid = quantize_grid(n, nsb);
#define SHERRY_FQ(B, D)                                                                                  \
  hipLaunchKernelGGL((quantize_pack_kernel<B, D, SHERRY_Q_BPL>), grid, dim3(256), 0, s, w, n, k, nullptr, \
                     alpha, nullptr, out)
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

// Device address of `scratch` on the current device, looked up once per
// device (each device holds its own copy of the array) and cached.
hipError_t quantize_scratch(float** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = static_cast<float*>(p);
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace sherry
