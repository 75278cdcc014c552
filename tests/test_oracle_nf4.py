"""Pins for the oracle's NF4 codebook, quantizer and dequantizer (CPU only).

Each test checks the oracle against something other than itself: a second
inverse-normal routine, published codebook values, exact rational brute force,
closed-form special cases and an independently written rounding path.
"""
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.special as sp

from oracle import nf4

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "nf4_levels_qlora.txt")


def _published_levels():
    """The NF4 values printed in the QLoRA paper (Dettmers et al. 2023, the appendix that
    lists the NormalFloat data type), from tests/golden.  They were computed from fp32
    probabilities, so they agree with a float64 construction to a few fp32 ulps, not
    bitwise."""
    vals = {}
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        i, v = line.split()
        vals[int(i)] = float(v)
    assert sorted(vals) == list(range(16))
    return [vals[i] for i in range(16)]


QLORA_PUBLISHED = _published_levels()


def test_codebook_invariants():
    L = nf4.codebook()
    assert L.dtype == np.float32 and L.shape == (16,)
    assert np.all(np.diff(L.astype(np.float64)) > 0)
    assert L[0] == -1.0 and L[7] == 0.0 and L[15] == 1.0
    assert np.sum(L < 0) == 7 and np.sum(L > 0) == 8
    assert not np.signbit(L[7])


def test_codebook_second_inverse_cdf():
    # scipy's ndtri (Cephes) instead of statistics.NormalDist (Wichura AS241)
    d = 1.0 - 0.5 * (1.0 / 32 + 1.0 / 30)
    top = sp.ndtri(d)
    pos = [sp.ndtri(0.5 + j * (d - 0.5) / 8) / top for j in range(1, 9)]
    neg = [-sp.ndtri(0.5 + j * (d - 0.5) / 7) / top for j in range(1, 8)]
    L2 = np.array(sorted(neg + [0.0] + pos)).astype(np.float32)
    assert np.array_equal(L2.view(np.uint32), nf4.codebook().view(np.uint32))


def test_codebook_matches_published_qlora_values():
    L = nf4.codebook().astype(np.float64)
    assert np.max(np.abs(L - np.array(QLORA_PUBLISHED))) < 5e-7


def _bf16_values(lo_bits, hi_bits):
    b = np.arange(lo_bits, hi_bits, dtype=np.uint32)
    return (b << 16).view(np.float32)


def _argmin_fraction(w: float, a: float):
    """Nearest level of w/a by exact rationals, ties to the lower code."""
    if a == 0.0:
        return 7
    L = [Fraction(float(v)) for v in nf4.codebook()]
    x = Fraction(float(w)) / Fraction(float(a))
    best, bd = None, None
    for i, l in enumerate(L):
        dd = abs(x - l)
        if bd is None or dd < bd:
            best, bd = i, dd
    return best


def test_quantize_random_blocks_bruteforce():
    rng = np.random.default_rng(11)
    w = rng.standard_normal((40, 64 * 6)).astype(np.float32) * rng.uniform(1e-3, 10, (40, 1)).astype(np.float32)
    w = nf4.bf16_round(w)
    codes, a = nf4.quantize_codes(w)
    wb = w.reshape(40, 6, 64)
    cb = codes.reshape(40, 6, 64)
    for i in range(40):
        for j in range(6):
            aa = float(a[i, j])
            assert aa == float(np.max(np.abs(wb[i, j])))
            for e in range(64):
                assert cb[i, j, e] == _argmin_fraction(wb[i, j, e], aa)


def test_quantize_every_bf16_value_unit_absmax():
    # every bf16 w with |w| <= 1, in blocks whose first element is 1.0 (absmax 1)
    pos = _bf16_values(0x0000, 0x3F81)  # +0 .. 1.0
    vals = np.concatenate([pos, -pos])
    n_per = 63
    nblk = -(-vals.size // n_per)
    pad = np.zeros(nblk * n_per, dtype=np.float32)
    pad[: vals.size] = vals
    w = np.concatenate([np.ones((nblk, 1), np.float32), pad.reshape(nblk, n_per)], axis=1)
    codes, a = nf4.quantize_codes(w)
    assert np.all(a == 1.0)
    L = [Fraction(float(v)) for v in nf4.codebook()]
    flat_w = w[:, 1:].reshape(-1)[: vals.size]
    flat_c = codes[:, 1:].reshape(-1)[: vals.size]
    # exact check: the code's level is nearest, and strictly nearer than any lower code
    for wv, c in zip(flat_w.tolist(), flat_c.tolist()):
        x = Fraction(wv)
        d = abs(x - L[c])
        if c > 0:
            assert abs(x - L[c - 1]) > d
        if c < 15:
            assert abs(x - L[c + 1]) >= d


def test_quantize_exact_ties_go_to_lower_code():
    L = nf4.codebook().astype(np.float64)
    m = (L[:-1] + L[1:]) / 2
    hit = 0
    for i in range(15):
        if np.float64(np.float32(m[i])) != m[i]:
            continue  # this midpoint is not an fp32 value; no fp32 input can tie
        for a in (1.0, 0.5, 4.0):
            t = np.float32(m[i] * a)
            blk = np.zeros((1, 64), np.float32)
            blk[0, 0] = a
            blk[0, 1] = t
            blk[0, 2] = np.nextafter(t, np.float32(np.inf))
            blk[0, 3] = np.nextafter(t, np.float32(-np.inf))
            codes, _ = nf4.quantize_codes(blk)
            assert codes[0, 1] == i          # exact tie -> lower code
            assert codes[0, 2] == i + 1      # just above the midpoint -> upper
            assert codes[0, 3] == i          # just below -> lower
            hit += 1
    assert hit >= 3


def test_exact_zero_maps_to_zero():
    rng = np.random.default_rng(3)
    w = nf4.bf16_round(rng.standard_normal((4, 128)).astype(np.float32))
    w[:, 5] = 0.0
    w[:, 77] = -0.0
    packed, a = nf4.quantize(w)
    codes = nf4.unpack(packed)
    assert np.all(codes[:, 5] == 7) and np.all(codes[:, 77] == 7)
    deq = nf4.dequantize(packed, a)
    assert np.all(deq[:, 5] == 0.0) and np.all(deq[:, 77] == 0.0)


def test_block_max_maps_to_end_levels_exactly():
    rng = np.random.default_rng(4)
    w = nf4.bf16_round(rng.standard_normal((8, 64)).astype(np.float32))
    w[:4, 9] = 50.0
    w[4:, 9] = -50.0
    packed, a = nf4.quantize(w)
    codes = nf4.unpack(packed)
    assert np.all(a == 50.0)
    assert np.all(codes[:4, 9] == 15) and np.all(codes[4:, 9] == 0)
    deq = nf4.dequantize(packed, a)
    assert np.all(deq[:4, 9] == 50.0) and np.all(deq[4:, 9] == -50.0)


def test_all_zero_block():
    w = np.zeros((2, 128), np.float32)
    w[1, 64:] = 1.0
    packed, a = nf4.quantize(w)
    codes = nf4.unpack(packed)
    assert a[0, 0] == 0 and a[0, 1] == 0 and a[1, 0] == 0 and a[1, 1] == 1.0
    assert np.all(codes[0] == 7) and np.all(codes[1, :64] == 7)
    deq = nf4.dequantize(packed, a)
    assert np.all(deq[0] == 0) and np.all(deq[1, :64] == 0) and np.all(deq[1, 64:] == 1.0)


def test_pack_nibble_order():
    codes = np.array([[1, 2, 15, 0] + [7] * 60], dtype=np.uint8)
    p = nf4.pack(codes)
    assert p[0, 0] == 0x12 and p[0, 1] == 0xF0 and p[0, 2] == 0x77
    assert np.array_equal(nf4.unpack(p), codes)


def test_round_trip_is_idempotent():
    rng = np.random.default_rng(5)
    w = nf4.bf16_round((0.02 * rng.standard_normal((64, 256))).astype(np.float32))
    p1, a1 = nf4.quantize(w)
    p2, a2 = nf4.quantize(nf4.dequantize(p1, a1))
    assert np.array_equal(p1, p2) and np.array_equal(a1.view(np.uint32), a2.view(np.uint32))


def _rne_bits_from_f32(f32: np.ndarray) -> np.ndarray:
    """Independent RNE to bf16 on the fp32 bit pattern (finite inputs)."""
    u = f32.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    return (((u + 0x7FFF + lsb) >> 16) & 0xFFFF).astype(np.uint16)


def test_bf16_round_hand_cases():
    one = 1.0
    cases = {
        one + 2.0 ** -8: one,                       # tie, even neighbour is 1
        one + 3 * 2.0 ** -8: one + 2.0 ** -6,       # tie, even neighbour is above
        one + 2.0 ** -8 + 2.0 ** -20: one + 2.0 ** -7,
        -(one + 2.0 ** -8): -one,
        2.0 ** -130 + 2.0 ** -140: 2.0 ** -130,     # subnormal stays subnormal
    }
    for x, want in cases.items():
        got = nf4.bf16_round(np.array([x], np.float32))[0]
        assert got == np.float32(want), (x, got, want)


def test_dequant_every_code_every_bf16_absmax():
    a_bits = np.arange(0x0000, 0x7F80, dtype=np.uint32)   # all finite non-negative bf16
    a = (a_bits << 16).view(np.float32)
    n = a.size
    codes = np.tile(np.arange(16, dtype=np.uint8), (n, 4))      # [n, 64]
    packed = nf4.pack(codes)
    deq = nf4.dequantize(packed, a.reshape(n, 1))
    L = nf4.codebook().astype(np.float64)
    exact = L[codes] * a.astype(np.float64)[:, None]            # exact: 24 x 8 bits
    want = _rne_bits_from_f32(exact.astype(np.float32))         # one rounding to fp32, then RNE
    assert np.array_equal(nf4.bf16_to_bits(deq), want)
