"""Plain, slow CPU oracle for the Sherry 1.25-bit ternary linear layer.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  It shares
no code with the HIP path (no kernels, headers, tables or helpers) and imports
nothing from it.  NumPy is its only dependency.

Sources (the pages that define the method):

* [P1] "Sherry, Tequila and Fairies in Python" (reeddaily.com), section 1.1
  "Sherry Quantization": the ``_reshape_by_granularity`` helper, the
  ``SherryNMQuant.forward`` listing and the ``SherryLinear`` layer.
* [P2] "Sherry: Hardware-Efficient 1.25-Bit Ternary Quantization via
  Fine-grained Sparsification", English digest (agihunt.info/en): the format
  paragraph (3:4 blocks, 32 states in 5 bits, sign bit plus 4 lookup bits,
  greedy Sparse-AbsMean) and the inference paragraph (pack offline, build
  lookup tables from activations, accumulate, apply the scale).
* [P3] the Chinese version of the same digest (agihunt.info), same paragraphs.
* [P4] the ACL 2026 abstract page (paperdot): four weights per five bits.

What the method computes, and where the pages leave a step open, the reading
taken here:

1. Blocks are 4 consecutive weights along K (the last dim of the ``[out, in]``
   weight) [P1 1.1, the reshape to ``(rows, K/m, m)``; P2 format].
2. Sparse-AbsMean zeroes the smallest |w| of each block [P2 format].  The
   listing uses ``topk``, which leaves ties open; reading: the lowest index
   wins a tie, and -0 compares equal to +0.
3. A kept weight's sign is +1 if w > 0 else -1.  The listing's ``sign`` would
   give 0 for an exact zero, which has no place among 32 states [P2 format];
   reading: -1.
4. The scale of a granule is the sum of kept |w| over the nominal kept count
   ``max(L/4*3, 1)`` [P1 1.1, ``denom`` and ``scale``].  Granules follow
   ``_reshape_by_granularity`` [P1 1.1]: per_tensor (whole matrix), per_channel
   (one output row), per_group (G consecutive weights of a row).  The order of
   the sum and its precision are not fixed by the pages; reading: a pairwise
   tree of fp32 adds over the granule in flat index order, padded with +0 to a
   power of two, then ``fp32(fp64(S) / fp64(D))``.
5. The 5-bit code is a sign bit plus 4 lookup bits [P2 format].  The bit
   assignment is fixed by this implementation: with kept positions
   k0 < k1 < k2 and zero position z,
   ``s = [sigma_k0 == -1]``, ``p0 = [sigma_k1 != sigma_k0]``,
   ``p1 = [sigma_k2 != sigma_k0]``, ``code = s<<4 | z<<2 | p1<<1 | p0``.
   Flipping ``s`` negates the decoded block (the mirror that lets a 16-entry
   table serve all 32 states, as in the pages' CPU kernel).
6. The byte layout is fixed by this implementation (the pages give none):
   see :func:`pack`.
7. The layer output is ``y = x @ (T*alpha)^T`` (``F.linear`` without bias)
   [P1 1.1, ``SherryLinear.forward``]; activations stay bf16 [P1 1.1 note on
   activations; P2 limits paragraph].

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
against brute force, closed forms or library routines; none is "parity
unpinned".  The pages print no worked numeric example, so no pin compares
against values printed on the pages.
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "BLOCK", "KEEP", "SUPERBLOCK", "GRANULARITIES",
    "validate", "select_zero", "kept_signs", "ternary",
    "encode_block", "decode_code", "encode", "decode_codes",
    "pack", "unpack", "packed_bytes",
    "pairwise_sum_f32", "alpha", "alpha_per_weight", "dequant",
    "quantize_pack", "fake_quant", "arenas_lambda", "arenas_forward", "gemv", "gemm", "tolerance_bound", "bf16_half_ulp", "round_to_bf16_bits",
    "bf16_bits_to_f32",
]

BLOCK = 4          # m: weights per block [P2 format]
KEEP = 3           # n: nonzeros kept per block [P2 format]
SUPERBLOCK = 128   # layout unit along K chosen by this implementation
GRANULARITIES = ("per_tensor", "per_channel", "per_group")


# --------------------------------------------------------------------------
# validation  [P1 1.1: _reshape_by_granularity and SherryNMQuant.forward]
# --------------------------------------------------------------------------
def validate(shape, granularity: str, group_size: int = 128) -> None:
    """Raise ValueError on the conditions the listings reject.

    Non-2-D weight, K not divisible by the block size, an unknown granularity,
    and for per_group a group size that is not positive or does not divide K
    [P1 1.1].  Added reading: per_group also needs G % 4 == 0 so that the
    nominal kept count G/4*3 is whole, and N, K must be positive.
    """
    if len(shape) != 2:
        raise ValueError("Sherry quantization expects a 2-D weight")
    n, k = int(shape[0]), int(shape[1])
    if n <= 0 or k <= 0:
        raise ValueError("weight dimensions must be positive")
    if k % BLOCK != 0:
        raise ValueError(f"K={k} is not divisible by the block size {BLOCK}")
    if granularity not in GRANULARITIES:
        raise ValueError(f"unsupported granularity: {granularity!r}")
    if granularity == "per_group":
        if group_size <= 0 or k % group_size != 0:
            raise ValueError("per_group needs 0 < group_size dividing K")
        if group_size % BLOCK != 0:
            raise ValueError("per_group needs group_size % 4 == 0")


# --------------------------------------------------------------------------
# a1: block selection and signs  [P2 format; P1 1.1 topk / mask / sign]
# --------------------------------------------------------------------------
def select_zero(w: np.ndarray) -> np.ndarray:
    """Index (0..3) of the zeroed weight in every block of 4 along K.

    The smallest |w| of the block is zeroed [P2 format].  ``np.argmin``
    returns the first occurrence of the minimum, which is the lowest-index
    tie-break (reading 2).  |w| is taken in fp32; ``np.abs`` maps -0 to +0.
    Returns int64 ``[N, K/4]``.
    """
    w = np.asarray(w, dtype=np.float32)
    n, k = w.shape
    a = np.abs(w).reshape(n, k // BLOCK, BLOCK)
    return np.argmin(a, axis=-1)


def kept_signs(w: np.ndarray) -> np.ndarray:
    """+1 where w > 0, else -1, for every weight (reading 3).  int8 [N, K]."""
    w = np.asarray(w, dtype=np.float32)
    return np.where(w > 0, 1, -1).astype(np.int8)


def ternary(w: np.ndarray) -> np.ndarray:
    """T in {-1, 0, +1}: the signs with the selected weight of each block set
    to 0 (one zero and three +-1 per block [P2 format]).  int8 [N, K]."""
    w = np.asarray(w, dtype=np.float32)
    n, k = w.shape
    z = select_zero(w)
    t = kept_signs(w).reshape(n, k // BLOCK, BLOCK).copy()
    np.put_along_axis(t, z[..., None], 0, axis=-1)
    return t.reshape(n, k)


# --------------------------------------------------------------------------
# a3: the 5-bit code  [P2 format: 32 states, sign bit + 4 lookup bits]
# --------------------------------------------------------------------------
def encode_block(z: int, signs) -> int:
    """Code of one block from its zero position ``z`` and the signs (+-1) of
    its three kept weights in ascending position order (reading 5)."""
    s0, s1, s2 = (int(v) for v in signs)
    s = 1 if s0 == -1 else 0
    p0 = 1 if s1 != s0 else 0
    p1 = 1 if s2 != s0 else 0
    return (s << 4) | (int(z) << 2) | (p1 << 1) | p0


def decode_code(code: int):
    """Inverse of :func:`encode_block`: the 4 ternary values of a block."""
    code = int(code)
    s = (code >> 4) & 1
    z = (code >> 2) & 3
    p1 = (code >> 1) & 1
    p0 = code & 1
    first = -1 if s else 1
    kept = [first, -first if p0 else first, -first if p1 else first]
    out, it = [], iter(kept)
    for pos in range(BLOCK):
        out.append(0 if pos == z else next(it))
    return out


def encode(w: np.ndarray) -> np.ndarray:
    """5-bit code of every block of ``w``: uint8 ``[N, K/4]``.

    Vectorised form of :func:`encode_block`: the kept positions in ascending
    order are the three positions other than z.
    """
    w = np.asarray(w, dtype=np.float32)
    n, k = w.shape
    z = select_zero(w)
    sg = kept_signs(w).reshape(n, k // BLOCK, BLOCK)
    # kept positions for each z, ascending
    kept_pos = np.array([[1, 2, 3], [0, 2, 3], [0, 1, 3], [0, 1, 2]])
    kp = kept_pos[z]                                   # [N, K/4, 3]
    ks = np.take_along_axis(sg, kp, axis=-1)           # signs of k0, k1, k2
    s = (ks[..., 0] == -1).astype(np.uint8)
    p0 = (ks[..., 1] != ks[..., 0]).astype(np.uint8)
    p1 = (ks[..., 2] != ks[..., 0]).astype(np.uint8)
    return (s << 4) | (z.astype(np.uint8) << 2) | (p1 << 1) | p0


def decode_codes(codes: np.ndarray) -> np.ndarray:
    """T (int8 ``[N, 4*C]``) from codes ``[N, C]``, through the 32-entry
    decode of :func:`decode_code`."""
    table = np.array([decode_code(c) for c in range(32)], dtype=np.int8)
    codes = np.asarray(codes, dtype=np.uint8)
    n, c = codes.shape
    return table[codes].reshape(n, c * BLOCK)


# --------------------------------------------------------------------------
# a3: byte layout (fixed by this implementation; the pages give none)
# --------------------------------------------------------------------------
def packed_bytes(n: int, k: int) -> int:
    """5 bits per 4 weights: N*K*5/32 bytes [P2 format; P4 abstract]."""
    return n * k * 5 // 32


def pack(codes: np.ndarray) -> np.ndarray:
    """Pack codes ``[N, K/4]`` into the byte layout (uint8, N*K*5/32 bytes).

    K is cut into superblocks of 128 weights (32 blocks).  Block j of
    superblock g has nibble ``code & 15`` and sign bit ``code >> 4``.

    * nibble plane, first N*K/8 bytes: 16 bytes per (g, n), ordered g-major
      then n.  The 16 bytes are 4 little-endian dwords d = 0..3; byte b of
      dword d holds block 2d + 8b in its low nibble and block 2d + 1 + 8b in
      its high nibble.
    * sign plane, next N*K/32 bytes: one little-endian dword per (g, n),
      g-major then n; bit j is the sign bit of block j.
    """
    codes = np.asarray(codes, dtype=np.uint8)
    n, nb = codes.shape
    k = nb * BLOCK
    if k % SUPERBLOCK:
        raise ValueError("the byte layout needs K % 128 == 0")
    nsb = k // SUPERBLOCK
    c = codes.reshape(n, nsb, 32).transpose(1, 0, 2)  # [g, n, j]
    nib = (c & 15).astype(np.uint8)
    sgn = (c >> 4).astype(np.uint32)

    nib_plane = np.zeros((nsb, n, 16), dtype=np.uint8)
    for j in range(32):
        d, h, b = (j & 7) >> 1, j & 1, j >> 3
        nib_plane[:, :, 4 * d + b] |= (nib[:, :, j] << (4 * h)).astype(np.uint8)

    sign_words = np.zeros((nsb, n), dtype=np.uint32)
    for j in range(32):
        sign_words |= sgn[:, :, j] << np.uint32(j)
    sign_plane = sign_words.astype("<u4").view(np.uint8).reshape(nsb, n, 4)

    out = np.concatenate([nib_plane.reshape(-1), sign_plane.reshape(-1)])
    assert out.size == packed_bytes(n, k)
    return out


def unpack(packed: np.ndarray, n: int, k: int) -> np.ndarray:
    """Inverse of :func:`pack`: codes ``[N, K/4]`` (uint8)."""
    packed = np.asarray(packed, dtype=np.uint8)
    if packed.size != packed_bytes(n, k):
        raise ValueError("packed size does not match N*K*5/32")
    nsb = k // SUPERBLOCK
    nib_plane = packed[: n * k // 8].reshape(nsb, n, 16)
    sign_words = packed[n * k // 8:].view("<u4").reshape(nsb, n)
    c = np.zeros((nsb, n, 32), dtype=np.uint8)
    for j in range(32):
        d, h, b = (j & 7) >> 1, j & 1, j >> 3
        lo = (nib_plane[:, :, 4 * d + b] >> (4 * h)) & 15
        hi = ((sign_words >> np.uint32(j)) & 1).astype(np.uint8)
        c[:, :, j] = lo | (hi << 4)
    return c.transpose(1, 0, 2).reshape(n, k // BLOCK)


# --------------------------------------------------------------------------
# a2: the scale  [P1 1.1 denom / scale; P2 format: mean |w| of kept weights]
# --------------------------------------------------------------------------
def pairwise_sum_f32(v: np.ndarray) -> np.ndarray:
    """Sum along the last axis by a pairwise tree of fp32 adds.

    The axis is padded with +0 to a power of two; each level adds element 2i
    and 2i+1 with one IEEE fp32 add (NumPy elementwise float32 add), until one
    value remains (reading 4).
    """
    v = np.asarray(v, dtype=np.float32)
    length = v.shape[-1]
    width = 1
    while width < length:
        width *= 2
    buf = np.zeros(v.shape[:-1] + (width,), dtype=np.float32)
    buf[..., :length] = v
    while buf.shape[-1] > 1:
        buf = buf[..., 0::2] + buf[..., 1::2]
    return buf[..., 0]


def _granules(a: np.ndarray, granularity: str, group_size: int) -> np.ndarray:
    """View of ``a`` [N, K] as [num_granules, L] in the order of
    ``_reshape_by_granularity`` [P1 1.1]."""
    n, k = a.shape
    if granularity == "per_tensor":
        return a.reshape(1, n * k)
    if granularity == "per_channel":
        return a.reshape(n, k)
    return a.reshape(n, k // group_size, group_size).reshape(-1, group_size)


def alpha(w: np.ndarray, granularity: str = "per_group",
          group_size: int = 128) -> np.ndarray:
    """Scale of every granule, fp32, in the stored layout.

    ``S`` = pairwise fp32 sum of kept |w| (pruned weights count as +0),
    ``D = max(L/4*3, 1)`` the nominal kept count, ``alpha = fp32(S/D)`` with
    the quotient taken in fp64 [P1 1.1; P2 format].

    Layout: per_group ``[K/G, N]`` (group-major), per_channel ``[N]``,
    per_tensor ``[1]``.
    """
    w = np.asarray(w, dtype=np.float32)
    validate(w.shape, granularity, group_size)
    n, k = w.shape
    t = ternary(w)
    v = np.where(t != 0, np.abs(w), np.float32(0)).astype(np.float32)
    g = _granules(v, granularity, group_size)
    length = g.shape[-1]
    s = pairwise_sum_f32(g)
    d = max(float(length) / float(BLOCK) * float(KEEP), 1.0)
    a = (s.astype(np.float64) / np.float64(d)).astype(np.float32)
    if granularity == "per_group":
        return np.ascontiguousarray(a.reshape(n, k // group_size).T)
    return a


def alpha_per_weight(a: np.ndarray, n: int, k: int, granularity: str,
                     group_size: int = 128) -> np.ndarray:
    """Broadcast stored scales to ``[N, K]`` (the scale of each weight's
    granule)."""
    a = np.asarray(a, dtype=np.float32)
    if granularity == "per_tensor":
        return np.full((n, k), a.reshape(-1)[0], dtype=np.float32)
    if granularity == "per_channel":
        return np.repeat(a.reshape(n, 1), k, axis=1)
    return np.repeat(a.reshape(k // group_size, n).T, group_size, axis=1)


def dequant(t: np.ndarray, a: np.ndarray, granularity: str,
            group_size: int = 128) -> np.ndarray:
    """W_q = T * alpha in fp64 (exact) [P1 1.1, ``signed*scale``]."""
    n, k = t.shape
    return t.astype(np.float64) * alpha_per_weight(
        a, n, k, granularity, group_size).astype(np.float64)


def quantize_pack(w: np.ndarray, granularity: str = "per_group",
                  group_size: int = 128):
    """Offline pack of a latent weight: (packed bytes, alpha) [P2 inference]."""
    w = np.asarray(w, dtype=np.float32)
    validate(w.shape, granularity, group_size)
    return pack(encode(w)), alpha(w, granularity, group_size)


def fake_quant(w: np.ndarray, granularity: str = "per_group",
               group_size: int = 128):
    """Quantization-aware training forward: (T * alpha in fp64, alpha)
    [P1 1.1 SherryNMQuant.forward returns ``signed*scale``].  Its backward is
    the identity (straight-through), which has no arithmetic to check."""
    w = np.asarray(w, dtype=np.float32)
    validate(w.shape, granularity, group_size)
    a = alpha(w, granularity, group_size)
    return dequant(ternary(w), a, granularity, group_size), a


def arenas_lambda(step: int, total_steps: int, lambda0: float) -> float:
    """Cosine-annealed residual weight [P2 weight-trapping paragraph: lambda_t
    decays to 0 on a cosine schedule]: lambda0 * (1 + cos(pi t / T)) / 2 for
    0 <= t < T, and 0 from T on (the residual is gone at inference)."""
    if total_steps <= 0 or step >= total_steps:
        return 0.0
    return lambda0 * 0.5 * (1.0 + math.cos(math.pi * step / total_steps))


def arenas_forward(x: np.ndarray, wq: np.ndarray, w: np.ndarray,
                   lam: float) -> np.ndarray:
    """Arenas training forward Y = X (T alpha)^T + lambda X W^T in fp64
    [P2 weight-trapping paragraph]: ``wq`` the dequantized weight, ``w`` the
    latent weight as the kernel reads it (bf16 values)."""
    x = np.asarray(x, dtype=np.float64)
    return x @ np.asarray(wq, dtype=np.float64).T + float(lam) * (x @ np.asarray(w, dtype=np.float64).T)


# --------------------------------------------------------------------------
# a5 / a6: the layer  [P1 1.1 SherryLinear.forward: F.linear(x, W_q)]
# --------------------------------------------------------------------------
def gemv(x: np.ndarray, wq: np.ndarray, rows=None) -> np.ndarray:
    """y = x @ W_q^T in fp64.  ``x`` [B, K] (bf16 values held in fp32, so the
    cast is exact), ``wq`` [N, K] fp64.  ``rows`` restricts the output to a
    subset of output rows (for sampled checks at full size)."""
    x64 = np.asarray(x, dtype=np.float64)
    w64 = np.asarray(wq, dtype=np.float64)
    if rows is not None:
        w64 = w64[np.asarray(rows)]
    return x64 @ w64.T


gemm = gemv  # the prefill product is the same definition with M rows of x


def tolerance_bound(x: np.ndarray, alpha_w: np.ndarray, y_ref=None) -> np.ndarray:
    """Per-element bound ``1e-3 * sum_k |x_k * alpha(n, k)|`` over all k,
    pruned positions included.  ``x`` [B, K], ``alpha_w`` [N, K]; returns
    [B, N].

    The 1e-3 term bounds the accumulation against the fp64 product.  When the
    output is stored in bf16, pass the fp64 result as ``y_ref``: rounding to
    bf16 adds at most half a bf16 ulp of the result, which is added to the
    bound (reading: the bf16 output format is part of the workload, and its
    final rounding can exceed 1e-3 * sum|x*alpha| whenever |y| is a large
    fraction of sum|x*alpha|, e.g. short K or x correlated with the weights).
    """
    x64 = np.abs(np.asarray(x, dtype=np.float64))
    a64 = np.abs(np.asarray(alpha_w, dtype=np.float64))
    bound = 1e-3 * (x64 @ a64.T)
    if y_ref is not None:
        bound = bound + bf16_half_ulp(y_ref)
    return bound


def bf16_half_ulp(y: np.ndarray) -> np.ndarray:
    """Half the bf16 spacing at |y| (8 significant bits): 2^(floor(log2|y|) - 8);
    0 where y == 0."""
    a = np.abs(np.asarray(y, dtype=np.float64))
    out = np.zeros_like(a)
    nz = a > 0
    out[nz] = np.exp2(np.floor(np.log2(a[nz])) - 8.0)
    return out


# --------------------------------------------------------------------------
# bf16 helpers used to state expected bf16 outputs
# --------------------------------------------------------------------------
def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round to nearest, ties to even); returns the
    16-bit patterns.  Inputs are finite."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return (r & np.uint64(0xFFFF)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)
