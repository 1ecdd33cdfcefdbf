"""Plain CPU oracle for the two comparison packings of a ternary matrix.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  It shares
no code with the HIP path and imports nothing from it.

The pages set 1.25-bit Sherry packing against two ways of storing a ternary
matrix ("Sherry: Hardware-Efficient 1.25-Bit Ternary Quantization via
Fine-grained Sparsification", agihunt digest, problem paragraph, and its
results table, which times the 1.67-bit "TL2" kernels):

* padded 2-bit: every weight in 2 bits, one state unused;
* about 1.67-bit: three weights in 5 bits (3^3 = 27 <= 32 states), groups of
  three that do not fall on power-of-two boundaries.

The pages fix neither bit layout; the readings taken here:

* 2-bit: weight value v in {0, +1, -1} is the code 0, 1, 2 (3 unused).  K runs
  in superblocks of 128 weights; the 32-byte record of (superblock g, row n)
  sits at byte (g*N + n)*32, weight j of the superblock in bits 2(j%4) of
  byte j//4.
* 3-in-5: digits d = v + 1 in {0, 1, 2}; the triple (v0, v1, v2) is the code
  d0 + 3 d1 + 9 d2 (0..26).  K runs in superblocks of 192 weights (64
  triples), zero-padded to a multiple of 192; the 40-byte record of
  (superblock g, row n) sits at byte (g*N + n)*40 and holds code t in bits
  [5t, 5t + 5) of its 320 bits, little-endian.

Both formats store the same ternary matrix T; the product is the same
``x @ (T*alpha)^T`` as for Sherry (see ``sherry_oracle.gemv``).
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "CMP_2BIT", "CMP_TL2", "SB_2BIT", "SB_TL2",
    "k_padded", "compare_bytes", "encode_2bit", "decode_2bit", "encode_tl2", "decode_tl2",
]

CMP_2BIT, CMP_TL2 = 0, 1
SB_2BIT = 128      # weights per 2-bit superblock (32 bytes)
SB_TL2 = 192       # weights per 3-in-5 superblock (64 triples, 40 bytes)
_V2CODE = {0: 0, 1: 1, -1: 2}


def k_padded(fmt: int, k: int) -> int:
    """K rounded up to the format's superblock."""
    sb = SB_2BIT if fmt == CMP_2BIT else SB_TL2
    return -(-k // sb) * sb


def compare_bytes(fmt: int, n: int, k: int) -> int:
    """Bytes of the packed planes: N*K/4 (2-bit), N*K_pad*40/192 (3-in-5)."""
    if fmt == CMP_2BIT:
        return n * k_padded(fmt, k) // 4
    return n * (k_padded(fmt, k) // SB_TL2) * 40


def encode_2bit(t: np.ndarray) -> np.ndarray:
    """Padded 2-bit packing of a ternary [N, K] matrix, written as a plain bit
    loop over the layout above."""
    t = np.asarray(t)
    n, k = t.shape
    kp = k_padded(CMP_2BIT, k)
    out = np.zeros(n * kp // 4, dtype=np.uint8)
    for row in range(n):
        for col in range(k):
            g, j = divmod(col, SB_2BIT)
            byte = (g * n + row) * 32 + j // 4
            out[byte] |= np.uint8(_V2CODE[int(t[row, col])] << (2 * (j % 4)))
    return out


def decode_2bit(packed: np.ndarray, n: int, k: int) -> np.ndarray:
    packed = np.asarray(packed, dtype=np.uint8)
    vals = {0: 0, 1: 1, 2: -1}
    t = np.zeros((n, k), dtype=np.int8)
    for row in range(n):
        for col in range(k):
            g, j = divmod(col, SB_2BIT)
            code = (int(packed[(g * n + row) * 32 + j // 4]) >> (2 * (j % 4))) & 3
            t[row, col] = vals[code]
    return t


def encode_tl2(t: np.ndarray) -> np.ndarray:
    """Three weights in 5 bits, written as a plain loop over the layout above
    (positions past K are weight 0, digit 1)."""
    t = np.asarray(t)
    n, k = t.shape
    kp = k_padded(CMP_TL2, k)
    nsb = kp // SB_TL2
    out = np.zeros(n * nsb * 40, dtype=np.uint8)
    for row in range(n):
        for g in range(nsb):
            bits = 0
            for tri in range(64):
                code = 0
                for i in range(3):
                    col = g * SB_TL2 + 3 * tri + i
                    v = int(t[row, col]) if col < k else 0
                    code += (v + 1) * (3 ** i)
                bits |= code << (5 * tri)
            base = (g * n + row) * 40
            out[base:base + 40] = np.frombuffer(bits.to_bytes(40, "little"), dtype=np.uint8)
    return out


def decode_tl2(packed: np.ndarray, n: int, k: int) -> np.ndarray:
    packed = np.asarray(packed, dtype=np.uint8)
    kp = k_padded(CMP_TL2, k)
    t = np.zeros((n, k), dtype=np.int8)
    for row in range(n):
        for g in range(kp // SB_TL2):
            base = (g * n + row) * 40
            bits = int.from_bytes(packed[base:base + 40].tobytes(), "little")
            for tri in range(64):
                code = (bits >> (5 * tri)) & 31
                for i in range(3):
                    col = g * SB_TL2 + 3 * tri + i
                    if col < k:
                        t[row, col] = (code // (3 ** i)) % 3 - 1
    return t
