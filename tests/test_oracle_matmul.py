"""Pins for the oracle's layer product y = x @ (T*alpha)^T (CPU only).

Pins: a pure-Python triple loop on tiny shapes (no BLAS), one-hot inputs that
read back T[n, k] * alpha exactly, the full pack/unpack path against the
direct ternary, and the tolerance bound against a bf16-rounded output.
"""

import math

import numpy as np
import pytest

import oracle as O
import workloads as WL


def _loop_gemv(x, t, a_w):
    b_rows, k = x.shape
    n = t.shape[0]
    y = [[0.0] * n for _ in range(b_rows)]
    for b in range(b_rows):
        for r in range(n):
            acc = 0.0
            for kk in range(k):
                if t[r, kk] != 0:
                    acc += float(x[b, kk]) * float(t[r, kk]) * float(a_w[r, kk])
            y[b][r] = acc
    return np.array(y)


@pytest.mark.parametrize("gran", ["per_group", "per_channel", "per_tensor"])
def test_gemv_against_python_loop(gran):
    w = WL.latent_weight(6, 256, seed=42)
    _, x = WL.activations_bf16(2, 256, seed=43)
    packed, a = O.quantize_pack(w, gran, 128)
    t = O.decode_codes(O.unpack(packed, 6, 256))
    wq = O.dequant(t, a, gran, 128)
    y = O.gemv(x, wq)
    y_loop = _loop_gemv(x, t, O.alpha_per_weight(a, 6, 256, gran, 128))
    assert np.allclose(y, y_loop, rtol=1e-12, atol=1e-12)


def test_pack_path_matches_direct_ternary():
    w = WL.latent_weight(256, 512, seed=0)
    packed, _ = O.quantize_pack(w)
    assert packed.size == 256 * 512 * 5 // 32
    t = O.decode_codes(O.unpack(packed, 256, 512))
    assert np.array_equal(t, O.ternary(w))


def test_one_hot_reads_back_weight():
    w = WL.latent_weight(8, 256, seed=3)
    packed, a = O.quantize_pack(w, "per_group", 128)
    t = O.ternary(w)
    wq = O.dequant(t, a, "per_group", 128)
    for k in (0, 5, 127, 128, 255):
        x = np.zeros((1, 256), dtype=np.float32)
        x[0, k] = 1.0
        y = O.gemv(x, wq)[0]
        expect = t[:, k].astype(np.float64) * a[k // 128].astype(np.float64)
        assert np.array_equal(y, expect)


def test_rows_subset():
    w = WL.latent_weight(16, 128, seed=8)
    _, x = WL.activations_bf16(1, 128, seed=9)
    _, a = O.quantize_pack(w)
    wq = O.dequant(O.ternary(w), a, "per_group", 128)
    rows = [0, 7, 15]
    assert np.array_equal(O.gemv(x, wq, rows=rows), O.gemv(x, wq)[:, rows])


def test_bf16_output_within_tolerance():
    """Rounding the fp64 result to bf16 stays inside 1e-3 * sum|x*alpha| at
    the small workload, so a bf16 output can pass the bound."""
    w = WL.latent_weight(256, 512, seed=0)
    _, x = WL.activations_bf16(1, 512, seed=1)
    _, a = O.quantize_pack(w)
    t = O.ternary(w)
    wq = O.dequant(t, a, "per_group", 128)
    y = O.gemv(x, wq)
    yb = O.bf16_bits_to_f32(O.round_to_bf16_bits(y.astype(np.float32)))
    bound = O.tolerance_bound(x, O.alpha_per_weight(a, 256, 512, "per_group"))
    assert np.all(np.abs(yb - y) <= bound)
    assert np.max(np.abs(yb - y) / bound) < 0.5


def test_bf16_half_ulp_bounds_rounding():
    """Half-ulp values at powers of two, and the bound holds (and is reached
    at ties) for torch's bf16 rounding."""
    torch = pytest.importorskip("torch")
    assert O.bf16_half_ulp(np.array([1.0]))[0] == 2.0**-8
    assert O.bf16_half_ulp(np.array([1.99]))[0] == 2.0**-8
    assert O.bf16_half_ulp(np.array([-4.0]))[0] == 2.0**-6
    assert O.bf16_half_ulp(np.array([0.0]))[0] == 0.0
    g = np.random.default_rng(3)
    y = np.concatenate([g.standard_normal(20000) * 10.0 ** g.integers(-3, 4, 20000),
                        [1.0 + 2.0**-8, 3.0 * (1.0 + 2.0**-8)]])
    yb = torch.from_numpy(y.astype(np.float32)).to(torch.bfloat16).double().numpy()
    err = np.abs(yb - y.astype(np.float32).astype(np.float64))
    hu = O.bf16_half_ulp(y)
    assert np.all(err <= hu * (1 + 1e-12))
    assert err[-2] == hu[-2]


# ---------------------------------------------------------------- Arenas
def test_arenas_lambda_cosine_values():
    """Cosine annealing from lambda0 to 0: exact ends, the half-way value, the
    value at a quarter (which tells a cosine from a linear decay: 1/2 + sqrt(2)/4,
    not 3/4), the mirror symmetry of the half wave, and monotone decay."""
    lam0, T = 0.75, 1000
    assert O.arenas_lambda(0, T, lam0) == lam0
    assert O.arenas_lambda(T, T, lam0) == 0.0 and O.arenas_lambda(T + 5, T, lam0) == 0.0
    assert abs(O.arenas_lambda(T // 2, T, lam0) - lam0 / 2) < 1e-15
    assert abs(O.arenas_lambda(T // 4, T, lam0) - lam0 * (0.5 + math.sqrt(2.0) / 4)) < 1e-15
    for t in range(0, T + 1, 37):
        assert abs(O.arenas_lambda(t, T, lam0) + O.arenas_lambda(T - t, T, lam0) - lam0) < 1e-15 or t == 0
    vals = [O.arenas_lambda(t, T, lam0) for t in range(T + 1)]
    assert all(a >= b for a, b in zip(vals, vals[1:]))


def test_arenas_forward_one_hot_and_zero_lambda():
    """One-hot activations pick column k of T*alpha + lambda*W exactly; with
    lambda = 0 the forward is the Sherry product."""
    rng = np.random.default_rng(3)
    n, k = 6, 8
    w = rng.standard_normal((n, k)).astype(np.float32)
    wq = np.where(rng.random((n, k)) < 0.25, 0.0, np.sign(rng.standard_normal((n, k)))) * 0.125
    lam = 0.3
    for c in (0, 5, 7):
        x = np.zeros((1, k))
        x[0, c] = 1.0
        y = O.arenas_forward(x, wq, w, lam)
        assert np.array_equal(y[0], wq[:, c] + lam * w[:, c].astype(np.float64))
    x = rng.standard_normal((3, k))
    assert np.array_equal(O.arenas_forward(x, wq, w, 0.0), O.gemm(x, wq))


# ---------------------------------------------------------------- tolerance pin
def _tolerance_fixture():
    import os
    from conftest import GOLDEN
    w, x, alpha, bound, y, bound_bf16 = [], [], {}, {}, {}, {}
    for line in open(os.path.join(GOLDEN, "tolerance_hand.txt")):
        line = line.split("#")[0].split()
        if not line:
            continue
        tag, rest = line[0], line[1:]
        if tag == "W":
            w.append([float(v) for v in rest])
        elif tag == "X":
            x.append([float(v) for v in rest])
        else:
            key = (rest[0], int(rest[1]))
            vals = [float(v) for v in rest[2:]]
            {"ALPHA": alpha, "BOUND": bound, "Y": y, "BOUND_BF16": bound_bf16}[tag][key] = vals
    return (np.array(w, dtype=np.float32), np.array(x, dtype=np.float32), alpha, bound, y, bound_bf16)


@pytest.mark.parametrize("gran,g", [("per_group", 4), ("per_channel", 8), ("per_tensor", 8)])
def test_tolerance_bound_hand_worked(gran, g):
    """The bound 1e-3 * sum_k |x_k| alpha(n, k) on a hand-worked 2 x 8 case
    (tests/golden/tolerance_hand.txt): the scales of all three granularities
    exactly (two distinct per_channel scales, four per_group scales in their
    group-major layout), then the bound of every (row of x, output) pair.  The
    values change if the factor, either absolute value, the granule broadcast
    or the range of the sum (all k, pruned positions included) changes."""
    w, x, alpha, bound, _, _ = _tolerance_fixture()
    a = O.alpha(w, gran, g)
    assert np.array_equal(a.reshape(-1), np.array(alpha[(gran, g)], dtype=np.float32))
    got = O.tolerance_bound(x, O.alpha_per_weight(a, 2, 8, gran, g))
    want = np.array(bound[(gran, g)]).reshape(2, 2)
    assert got.shape == (2, 2)
    assert np.allclose(got, want, rtol=1e-12, atol=0)


def test_tolerance_bound_bf16_term_hand_worked():
    """With the fp64 result passed in, half a bf16 ulp of it is added: the
    hand-worked per_group output y[0, 0] = 5.75 and its bound 0.0255."""
    w, x, _, _, y, bound_bf16 = _tolerance_fixture()
    a = O.alpha(w, "per_group", 4)
    t = O.ternary(w)
    y_ref = O.gemv(x, O.dequant(t, a, "per_group", 4))
    b, n, yv = y[("per_group", 4)]
    assert y_ref[int(b), int(n)] == yv
    got = O.tolerance_bound(x, O.alpha_per_weight(a, 2, 8, "per_group", 4), y_ref)
    b2, n2, bv = bound_bf16[("per_group", 4)]
    assert abs(got[int(b2), int(n2)] - bv) <= 1e-15


def test_alpha_per_weight_per_channel_two_rows():
    """per_channel broadcast: every weight of row n gets that row's scale
    (0.75 and 1.125 in the hand-worked case), and the dequantized weight is
    T times it, exactly."""
    w, _, alpha, _, _, _ = _tolerance_fixture()
    a = O.alpha(w, "per_channel", 8)
    aw = O.alpha_per_weight(a, 2, 8, "per_channel")
    assert np.array_equal(aw[0], np.full(8, 0.75, dtype=np.float32))
    assert np.array_equal(aw[1], np.full(8, 1.125, dtype=np.float32))
    wq = O.dequant(O.ternary(w), a, "per_channel")
    assert np.array_equal(wq[0], np.array([1, -1, 1, 0, -1, 0, 1, -1]) * 0.75)
    assert np.array_equal(wq[1], np.array([1, -1, 0, 1, 1, -1, 0, 1]) * 1.125)
