"""Pins for the comparison packings (padded 2-bit, three weights in 5 bits):
hand-worked bytes under tests/golden/, exhaustive code tables, sizes and
round trips.  CPU only."""

import itertools
import os

import numpy as np

import oracle as O
from conftest import GOLDEN


def _golden():
    out = {}
    with open(os.path.join(GOLDEN, "compare_hand.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            key, *vals = line.split()
            out[key] = vals
    return out


def test_2bit_hand_bytes():
    g = _golden()
    row = np.array([[int(v) for v in g["ROW8"]]], dtype=np.int8)
    packed = O.encode_2bit(row)
    assert packed.size == 32  # one 128-weight superblock record
    assert packed[0] == int(g["BYTES2"][0], 16) and packed[1] == int(g["BYTES2"][1], 16)
    assert not packed[2:].any()
    assert np.array_equal(O.decode_2bit(packed, 1, 8), row)


def test_tl2_hand_codes():
    g = _golden()
    row = np.array([[int(v) for v in g["ROW6"]]], dtype=np.int8)
    packed = O.encode_tl2(row)
    assert packed.size == 40
    bits = int.from_bytes(packed.tobytes(), "little")
    tri = [int(v) for v in g["TRIPLES"]]
    assert bits & 31 == tri[0] and (bits >> 5) & 31 == tri[1]
    pad = int(g["PAD_TRIPLE"][0])
    assert all((bits >> (5 * t)) & 31 == pad for t in range(2, 64))
    assert np.array_equal(O.decode_tl2(packed, 1, 6), row)


def test_tl2_codes_are_a_bijection_on_27_triples():
    codes = set()
    for v in itertools.product((-1, 0, 1), repeat=3):
        p = O.encode_tl2(np.array([v], dtype=np.int8))
        c = int.from_bytes(p.tobytes(), "little") & 31
        assert c < 27
        codes.add(c)
        assert tuple(O.decode_tl2(p, 1, 3)[0]) == v
    assert codes == set(range(27))


def test_sizes_and_round_trip_random():
    rng = np.random.default_rng(11)
    for n, k in ((3, 128), (5, 384), (2, 256)):
        t = rng.integers(-1, 2, size=(n, k)).astype(np.int8)
        p2 = O.encode_2bit(t)
        assert p2.size == O.compare_bytes(O.CMP_2BIT, n, k) == n * k // 4
        assert np.array_equal(O.decode_2bit(p2, n, k), t)
        p3 = O.encode_tl2(t)
        kp = O.k_padded(O.CMP_TL2, k)
        assert kp % 192 == 0 and kp - k < 192
        assert p3.size == O.compare_bytes(O.CMP_TL2, n, k) == n * kp * 5 // 24
        assert np.array_equal(O.decode_tl2(p3, n, k), t)
