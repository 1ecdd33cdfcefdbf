"""Pins for the oracle's block selection, code and byte layout (CPU only).

Each check here is independent of the formula it pins: exhaustive enumeration
with a known answer by construction, hand-worked fixtures under
``tests/golden/``, closed forms (counts, sizes), or round trips.
"""

import itertools
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle as O
from conftest import GOLDEN


def _read_blocks():
    rows, alpha_line = [], None
    with open(os.path.join(GOLDEN, "blocks_hand.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if line.startswith("ALPHA_PER_TENSOR"):
                _, s, d = line.split()
                alpha_line = (float(s), float(d))
                continue
            w, z, t, code, ksum = [p.strip() for p in line.split("|")]
            rows.append((
                [float(v) for v in w.split()], int(z),
                [int(v) for v in t.split()], int(code), float(ksum)))
    return rows, alpha_line


def _read_layout():
    out = {}
    with open(os.path.join(GOLDEN, "layout_hand.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            key, *vals = line.split()
            out[key] = vals
    return out


# ---------------------------------------------------------------- selection
def test_hand_blocks_select_sign_code():
    rows, _ = _read_blocks()
    w = np.array([r[0] for r in rows], dtype=np.float32).reshape(1, -1)
    z = O.select_zero(w)[0]
    t = O.ternary(w).reshape(-1, 4)
    codes = O.encode(w)[0]
    for i, (_, zz, tt, code, _) in enumerate(rows):
        assert z[i] == zz, i
        assert list(t[i]) == tt, i
        assert codes[i] == code, i
        assert O.encode_block(zz, [v for p, v in enumerate(tt) if p != zz]) == code


def test_hand_blocks_alpha_per_tensor():
    rows, (s, d) = _read_blocks()
    w = np.array([r[0] for r in rows], dtype=np.float32).reshape(1, -1)
    assert sum(r[4] for r in rows) == s
    assert O.alpha(w, "per_tensor")[0] == np.float32(s / d)


def test_exhaustive_distinct_magnitudes():
    """All 24 orderings of 4 distinct magnitudes x 16 sign patterns: the zero
    lands on the smallest magnitude, the rest keep their sign."""
    mags = np.array([0.125, 0.5, 1.5, 3.0], dtype=np.float32)
    blocks, expect_t = [], []
    for perm in itertools.permutations(range(4)):
        for sg in itertools.product((1, -1), repeat=4):
            m = mags[list(perm)]
            blocks.append(m * np.array(sg, dtype=np.float32))
            smallest = perm.index(0)
            expect_t.append([0 if p == smallest else sg[p] for p in range(4)])
    w = np.concatenate(blocks).reshape(1, -1)
    t = O.ternary(w).reshape(-1, 4)
    assert np.array_equal(t, np.array(expect_t))


def test_tie_patterns_lowest_index():
    cases = [
        ([1, 1, 2, 3], 0), ([2, 1, 1, 3], 1), ([3, 2, 1, 1], 2),
        ([4, 4, 4, 1], 3), ([5, 5, 5, 5], 0), ([2, 1, 3, 1], 1),
        ([-0.0, 0.0, 1, 1], 0), ([1, -0.0, 0.0, 2], 1), ([1, 2, -0.0, 0.0], 2),
        ([-2, 2, -2, 2], 0), ([3, -1, 2, 1], 1),
    ]
    w = np.array([c for c, _ in cases], dtype=np.float32).reshape(1, -1)
    z = O.select_zero(w)[0]
    assert list(z) == [e for _, e in cases]


def test_brute_force_random_ties():
    """bf16-like inputs with many exact ties, against a first-minimum loop."""
    g = np.random.default_rng(7)
    w = (g.integers(-3, 4, size=(16, 64)) * 0.25).astype(np.float32)
    z = O.select_zero(w)
    for r in range(w.shape[0]):
        for b in range(w.shape[1] // 4):
            blk = [abs(float(v)) for v in w[r, 4 * b:4 * b + 4]]
            best = 0
            for i in range(1, 4):
                if blk[i] < blk[best]:
                    best = i
            assert z[r, b] == best


@given(st.integers(1, 6), st.integers(1, 12), st.integers(0, 2**31 - 1))
@settings(max_examples=40, deadline=None)
def test_one_zero_per_block(n, kb, seed):
    w = np.random.default_rng(seed).standard_normal((n, 4 * kb)).astype(np.float32)
    t = O.ternary(w).reshape(n, kb, 4)
    assert np.all((t == 0).sum(-1) == 1)
    assert np.all(np.isin(t, (-1, 0, 1)))
    assert int((t != 0).sum()) == 3 * n * kb


# ---------------------------------------------------------------- the code
def test_code_bijection_32_states():
    seen = {}
    for z in range(4):
        for signs in itertools.product((1, -1), repeat=3):
            c = O.encode_block(z, signs)
            assert 0 <= c < 32
            assert c not in seen
            seen[c] = (z, signs)
            dec = O.decode_code(c)
            assert dec[z] == 0
            assert [v for p, v in enumerate(dec) if p != z] == list(signs)
    assert len(seen) == 32  # C(4,3) * 2^3 states fill 5 bits


def test_code_mirror_sign_bit():
    """Flipping the sign bit negates the block, so 16 lookup entries plus a
    sign cover all 32 states."""
    for c in range(32):
        assert O.decode_code(c ^ 16) == [-v for v in O.decode_code(c)]
        first_kept = next(v for v in O.decode_code(c) if v != 0)
        assert (first_kept == -1) == bool(c >> 4)


def test_every_code_has_one_zero():
    for c in range(32):
        d = O.decode_code(c)
        assert d.count(0) == 1 and all(v in (-1, 0, 1) for v in d)


@given(st.integers(0, 2**31 - 1))
@settings(max_examples=25, deadline=None)
def test_vectorised_encode_matches_scalar(seed):
    w = np.random.default_rng(seed).standard_normal((3, 32)).astype(np.float32)
    codes = O.encode(w)
    t = O.ternary(w).reshape(3, 8, 4)
    for r in range(3):
        for b in range(8):
            zz = int(np.flatnonzero(t[r, b] == 0)[0])
            kept = [int(v) for p, v in enumerate(t[r, b]) if p != zz]
            assert codes[r, b] == O.encode_block(zz, kept)
    assert np.array_equal(O.decode_codes(codes), O.ternary(w))


# ---------------------------------------------------------------- layout
def test_layout_hand_single_superblock():
    lay = _read_layout()
    codes = np.array([int(v) for v in lay["CODES"]], dtype=np.uint8).reshape(1, 32)
    expect = np.array([int(v, 16) for v in lay["BYTES"]], dtype=np.uint8)
    got = O.pack(codes)
    assert got.size == O.packed_bytes(1, 128) == 20
    assert np.array_equal(got, expect)
    assert np.array_equal(O.unpack(expect, 1, 128), codes)


def test_layout_hand_two_rows_two_superblocks():
    lay = _read_layout()
    base = np.arange(32, dtype=np.uint8)
    codes = np.stack([np.tile(base, 2), np.tile(base ^ 16, 2)])
    expect = np.array([int(v, 16) for v in lay["BYTES2"]], dtype=np.uint8)
    got = O.pack(codes)
    assert got.size == O.packed_bytes(2, 256) == 80
    assert np.array_equal(got, expect)


@given(st.integers(1, 9), st.integers(1, 4), st.integers(0, 2**31 - 1))
@settings(max_examples=40, deadline=None)
def test_pack_round_trip(n, nsb, seed):
    codes = np.random.default_rng(seed).integers(0, 32, size=(n, 32 * nsb)).astype(np.uint8)
    p = O.pack(codes)
    assert p.size == n * 128 * nsb * 5 // 32
    assert np.array_equal(O.unpack(p, n, 128 * nsb), codes)


def test_packed_size_is_1_25_bits():
    for n, k in [(256, 512), (2048, 2048), (8192, 8192), (3072, 3072)]:
        assert O.packed_bytes(n, k) * 8 / (n * k) == 1.25


# ---------------------------------------------------------------- validation
@pytest.mark.parametrize("shape,gran,g", [
    ((4,), "per_group", 128), ((2, 3, 4), "per_group", 128),
    ((4, 6), "per_tensor", 128), ((4, 128), "per_block", 128),
    ((4, 128), "per_group", 0), ((4, 128), "per_group", -4),
    ((4, 128), "per_group", 96), ((4, 128), "per_group", 126),
    ((0, 128), "per_tensor", 128),
])
def test_validation_errors(shape, gran, g):
    with pytest.raises(ValueError):
        O.validate(shape, gran, g)


def test_validation_accepts_page_rules():
    O.validate((3, 12), "per_tensor", 0)
    O.validate((3, 12), "per_channel", 0)
    O.validate((3, 24), "per_group", 12)
    O.validate((3, 24), "per_group", 4)


# ---------------------------------------------------------------- fake quant
def test_hand_blocks_fake_quant():
    """T * alpha of the hand-worked row, per_tensor (alpha = 38.5 / 27) and
    per_group G = 12 (three blocks per group, denominator 9, group sums
    from the hand-worked kept sums)."""
    rows, (s_tensor, d_tensor) = _read_blocks()
    w = np.array([r[0] for r in rows], dtype=np.float32).reshape(1, -1)
    t = np.array([r[2] for r in rows], dtype=np.float64).reshape(1, -1)
    out, a = O.fake_quant(w, "per_tensor")
    expect_a = np.float32(s_tensor / d_tensor)
    assert a.reshape(-1)[0] == expect_a
    assert np.array_equal(out, t * np.float64(expect_a))
    ksum = [r[4] for r in rows]
    out, a = O.fake_quant(w, "per_group", 12)
    for g in range(3):
        ag = np.float32(sum(ksum[3 * g:3 * g + 3]) / 9.0)
        assert a.reshape(-1)[g] == ag
        assert np.array_equal(out[0, 12 * g:12 * g + 12], t[0, 12 * g:12 * g + 12] * np.float64(ag))
