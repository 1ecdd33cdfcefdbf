"""Pins for the oracle's scale (alpha) and its pairwise fp32 sum (CPU only).

Pins: the exact rational mean (fractions) within the tree's error bound,
special cases that come out exactly, invariances (scaling by 2^p, negation),
identities between granularities, and a hand-worked sum where the tree order
gives a different fp32 result from a left-to-right sum.
"""

import math
from fractions import Fraction

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle as O


def test_pairwise_tree_order_hand():
    # [2^24, 1, 1, 1, 1, 1, 1, 1]: the tree gives (2^24+1 -> 2^24) + 2 + (2+2)
    # = 2^24 + 6 exactly; a left-to-right fp32 sum stays at 2^24; exact is 2^24+7.
    v = np.array([2.0**24] + [1.0] * 7, dtype=np.float32)
    assert float(O.pairwise_sum_f32(v)) == 2.0**24 + 6
    seq = np.float32(0)
    for e in v:
        seq = np.float32(seq + e)
    assert float(seq) == 2.0**24


def test_pairwise_tree_padding():
    # 5 values pad to 8 with +0: ((1+2)+(3+4)) + ((5+0)+(0+0)) = 15
    assert float(O.pairwise_sum_f32(np.arange(1, 6, dtype=np.float32))) == 15.0
    assert float(O.pairwise_sum_f32(np.array([7.0], dtype=np.float32))) == 7.0


def _exact_mean(w, t):
    s = Fraction(0)
    for v, tt in zip(w.reshape(-1), t.reshape(-1)):
        if tt != 0:
            s += Fraction(abs(float(v)))
    return s / Fraction(t.size * 3, 4)


@pytest.mark.parametrize("gran,g", [("per_group", 128), ("per_group", 32),
                                    ("per_channel", 0), ("per_tensor", 0)])
def test_alpha_close_to_exact_rational_mean(gran, g):
    w = np.random.default_rng(3).standard_normal((6, 256)).astype(np.float32) * 0.02
    a = O.alpha(w, gran, g or 128)
    t = O.ternary(w)
    n, k = w.shape
    if gran == "per_group":
        granules = [(r, c) for c in range(k // g) for r in range(n)]
        vals = a.reshape(-1)
        for idx, (r, c) in enumerate(granules):
            ex = _exact_mean(w[r, c * g:(c + 1) * g], t[r, c * g:(c + 1) * g])
            length = g
            bound = (math.ceil(math.log2(length)) + 2) * 2.0**-24
            assert abs(Fraction(float(vals[idx])) - ex) <= Fraction(bound) * ex
    elif gran == "per_channel":
        for r in range(n):
            ex = _exact_mean(w[r], t[r])
            bound = (math.ceil(math.log2(k)) + 2) * 2.0**-24
            assert abs(Fraction(float(a[r])) - ex) <= Fraction(bound) * ex
    else:
        ex = _exact_mean(w, t)
        bound = (math.ceil(math.log2(n * k)) + 2) * 2.0**-24
        assert abs(Fraction(float(a[0])) - ex) <= Fraction(bound) * ex


def test_alpha_exact_when_sums_are_exact():
    # dyadic magnitudes with few bits: every tree add is exact, so alpha is
    # the correctly rounded fp32 of the exact mean
    g = np.random.default_rng(11)
    w = (g.integers(-64, 65, size=(4, 256)) / 64.0).astype(np.float32)
    t = O.ternary(w)
    a = O.alpha(w, "per_group", 128)
    for c in range(2):
        for r in range(4):
            ex = _exact_mean(w[r, c * 128:(c + 1) * 128], t[r, c * 128:(c + 1) * 128])
            assert a[c, r] == np.float32(float(ex))


def test_alpha_constant_power_of_two():
    for c in (0.125, 2.0**-10, 4.0):
        w = np.full((3, 256), c, dtype=np.float32)
        w[1] *= -1
        for gran in ("per_group", "per_channel", "per_tensor"):
            assert np.all(O.alpha(w, gran, 128) == np.float32(c))


def test_alpha_all_zero_granule():
    w = np.zeros((2, 256), dtype=np.float32)
    w[1, 128:] = 1.0
    a = O.alpha(w, "per_group", 128)
    assert a[0, 0] == 0 and a[1, 0] == 0 and a[0, 1] == 0
    assert a[1, 1] == 1.0
    codes = O.encode(w)
    assert np.all(codes[0] == 16)  # z = 0, every kept sign -1


@given(st.integers(-20, 20), st.integers(0, 2**31 - 1))
@settings(max_examples=30, deadline=None)
def test_scaling_by_power_of_two(p, seed):
    w = np.random.default_rng(seed).standard_normal((3, 256)).astype(np.float32) * 0.02
    w2 = (w * np.float32(2.0**p)).astype(np.float32)
    assert np.array_equal(O.encode(w), O.encode(w2))
    for gran in ("per_group", "per_channel", "per_tensor"):
        assert np.array_equal(O.alpha(w2, gran, 128),
                              (O.alpha(w, gran, 128) * np.float32(2.0**p)).astype(np.float32))


@given(st.integers(0, 2**31 - 1))
@settings(max_examples=30, deadline=None)
def test_negation_flips_sign_bit_only(seed):
    w = np.random.default_rng(seed).standard_normal((3, 256)).astype(np.float32)
    w[w == 0] = 1.0  # negating an exact zero keeps sign -1, excluded here
    c1, c2 = O.encode(w), O.encode(-w)
    assert np.array_equal(c1 ^ 16, c2)
    assert np.array_equal(O.select_zero(w), O.select_zero(-w))
    for gran in ("per_group", "per_channel", "per_tensor"):
        assert np.array_equal(O.alpha(w, gran, 128), O.alpha(-w, gran, 128))


def test_granularity_identities():
    w = np.random.default_rng(5).standard_normal((4, 512)).astype(np.float32)
    # one group spanning K is one channel
    assert np.array_equal(O.alpha(w, "per_group", 512).reshape(-1),
                          O.alpha(w, "per_channel"))
    # one row: per_channel == per_tensor
    assert O.alpha(w[:1], "per_channel")[0] == O.alpha(w[:1], "per_tensor")[0]
    # codes do not depend on the granularity: quantize_pack bytes agree
    p1, _ = O.quantize_pack(w, "per_group", 128)
    p2, _ = O.quantize_pack(w, "per_tensor", 128)
    assert np.array_equal(p1, p2)


def test_denominator_is_nominal_kept_count():
    # a granule whose kept weights include exact zeros still divides by L/4*3
    w = np.zeros((1, 128), dtype=np.float32)
    w[0, 1::4] = 3.0  # one nonzero per block: two kept exact zeros per block
    a = O.alpha(w, "per_group", 128)
    assert a[0, 0] == np.float32(3.0 * 32 / 96)


def test_dequant_is_sign_times_scale():
    w = np.random.default_rng(9).standard_normal((5, 256)).astype(np.float32)
    t = O.ternary(w)
    for gran in ("per_group", "per_channel", "per_tensor"):
        a = O.alpha(w, gran, 128)
        wq = O.dequant(t, a, gran, 128)
        aw = O.alpha_per_weight(a, 5, 256, gran, 128)
        assert np.array_equal(np.abs(wq[t != 0]), aw[t != 0].astype(np.float64))
        assert np.all(wq[t == 0] == 0)
        assert np.array_equal(np.sign(wq), t.astype(np.float64) * (aw > 0))


def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    g = np.random.default_rng(1)
    x = np.concatenate([
        g.standard_normal(10000).astype(np.float32),
        np.array([1.0 + 2.0**-8, 1.0 + 3 * 2.0**-8, -(1.0 + 2.0**-8), 0.0, -0.0,
                  3.0e38, 1e-40], dtype=np.float32)])
    ours = O.round_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_alpha_uses_the_pairwise_tree_hand():
    """Hand-worked: row of 8 blocks, block 0 = [0, 2^24, 1, 1], blocks 1..7 =
    [0, 1, 1, 1].  Zeros are pruned (+0 in the sum).  Tree: block 0 ->
    (0+2^24) + (1+1) = 2^24+2; block 1 -> 1 + 2 = 3; (2^24+2)+3 = 2^24+5 rounds
    to 2^24+4 (tie to even); blocks 2..3 -> 6, 4..7 -> 12; then 2^24+4+6 =
    2^24+10 and 2^24+10+12 = 2^24+22.  A left-to-right sum would give 2^24
    and the exact sum is 2^24+23.  D = 32/4*3 = 24."""
    row = [0.0, 2.0**24, 1.0, 1.0] + [0.0, 1.0, 1.0, 1.0] * 7
    w = np.array(row, dtype=np.float32).reshape(1, 32)
    expect = np.float32(np.float64(2.0**24 + 22) / 24.0)
    assert O.alpha(w, "per_tensor")[0] == expect
    assert O.alpha(w, "per_group", 32)[0, 0] == expect
    assert O.alpha(w, "per_channel")[0] == expect
    assert expect != np.float32(np.float64(2.0**24 + 23) / 24.0)
