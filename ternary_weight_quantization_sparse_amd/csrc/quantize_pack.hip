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
#include "sherry_internal.h"

namespace sherry {
namespace {

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
// row_shl:n / row_shr:n (lane i gets lane i + n / i - n of its row), n = 1..7
template <typename T>
__device__ inline T dpp_shl(T v, int n) {
  switch (n) {
    case 1: return dpp<0x101>(v);
    case 2: return dpp<0x102>(v);
    case 3: return dpp<0x103>(v);
    case 4: return dpp<0x104>(v);
    case 5: return dpp<0x105>(v);
    case 6: return dpp<0x106>(v);
    default: return dpp<0x107>(v);
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

}  // namespace sherry
