"""Pins for the oracle's counter-based dropout (CPU only)."""
import os
from fractions import Fraction

import numpy as np

from oracle import philox

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "philox4x32_10_kat.txt")


def _kat():
    """Known-answer vectors of Philox4x32-10 distributed with its authors' Random123
    library (Salmon et al., SC'11), from tests/golden: (counter, key) -> output."""
    out = []
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        w = [int(x, 16) for x in line.split()]
        assert len(w) == 10
        out.append((tuple(w[0:4]), tuple(w[4:6]), tuple(w[6:10])))
    return out


KAT = _kat()


def _round_f32(q: Fraction) -> np.float32:
    """Exact rational -> nearest fp32, ties to even (checked against both neighbours)."""
    c = np.float32(float(q))
    best = None
    for cand in (np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))):
        d = abs(Fraction(float(cand)) - q)
        even = (int(np.array(cand, np.float32).view(np.uint32)) & 1) == 0
        if best is None or d < best[0] or (d == best[0] and even):
            best = (d, cand)
    return np.float32(best[1])


def test_known_answers():
    assert len(KAT) == 3
    for ctr, key, want in KAT:
        got = philox.philox4x32_10(ctr, key)
        assert tuple(int(g) for g in got) == want


def test_vectorised_equals_scalar():
    rng = np.random.default_rng(0)
    ctr = [rng.integers(0, 2**32, 50, dtype=np.uint64) for _ in range(4)]
    key = (0x12345678, 0x9ABCDEF0)
    vec = philox.philox4x32_10(ctr, key)
    for i in range(50):
        one = philox.philox4x32_10(tuple(int(c[i]) for c in ctr), key)
        assert tuple(int(v[i]) for v in vec) == tuple(int(o) for o in one)


def test_threshold_and_scale():
    assert philox.drop_threshold(0.0) == 0
    assert philox.drop_threshold(0.5) == 2**31
    assert philox.drop_threshold(0.25) == 2**30
    # p = 0.1 as fp32 is 13421773 / 2^27
    assert philox.drop_threshold(0.1) == (13421773 * 2**32) // 2**27
    for p in (0.0, 0.1, 0.25, 0.3, 0.5, 0.9):
        p32 = Fraction(float(np.float32(p)))
        one_minus = _round_f32(1 - p32)
        assert philox.drop_scale(p) == _round_f32(1 / Fraction(float(one_minus)))
    assert philox.drop_scale(0.0) == np.float32(1.0)
    assert philox.drop_scale(0.5) == np.float32(2.0)


def test_mask_layout_matches_counter_definition():
    T, K = 5, 96
    seed, layer, proj, step, micro = 0x1_0000_0002, 3, 5, 7, 1
    keep = philox.keep_mask(T, K, 0.3, seed, layer, proj, step, micro)
    thr = philox.drop_threshold(0.3)
    for t, k in [(0, 0), (0, 3), (1, 17), (4, 95), (2, 64)]:
        e = t * K + k
        words = philox.philox4x32_10((e >> 2, (layer << 4) | proj, step, micro),
                                     (seed & 0xFFFFFFFF, seed >> 32))
        assert keep[t, k] == (int(words[e & 3]) >= thr)


def test_mask_statistics_and_keys():
    T, K, p = 512, 896, 0.1
    keep = philox.keep_mask(T, K, p, 0, 0, 0, 0, 0)
    n = T * K
    dropped = n - int(keep.sum())
    sd = np.sqrt(n * p * (1 - p))
    assert abs(dropped - n * p) < 5 * sd
    other = philox.keep_mask(T, K, p, 0, 0, 1, 0, 0)       # another projection
    assert not np.array_equal(keep, other)
    again = philox.keep_mask(T, K, p, 0, 0, 0, 0, 0)       # replay
    assert np.array_equal(keep, again)


def test_zero_dropout_keeps_everything():
    keep = philox.keep_mask(64, 128, 0.0, 99, 1, 2, 3, 4)
    assert keep.all()
