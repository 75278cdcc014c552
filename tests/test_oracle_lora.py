"""Pins for the oracle's NF4 + LoRA linear (CPU only): special cases, brute
force on tiny integer inputs, and central finite differences."""
import itertools

import numpy as np

from oracle import lora, nf4


def _setup(T=6, K=128, N=64, r=4, seed=0, w_std=0.05, bias=True):
    rng = np.random.default_rng(seed)
    w = nf4.bf16_round((w_std * rng.standard_normal((N, K))).astype(np.float32))
    codes, a = nf4.quantize(w)
    x = nf4.bf16_round(rng.standard_normal((T, K)).astype(np.float32))
    A = rng.uniform(-1 / np.sqrt(K), 1 / np.sqrt(K), (r, K)).astype(np.float32)
    B = (0.3 * rng.standard_normal((N, r))).astype(np.float32)
    b = nf4.bf16_round((0.02 * rng.standard_normal(N)).astype(np.float32)) if bias else None
    dy = nf4.bf16_round(rng.standard_normal((T, N)).astype(np.float32))
    return x, codes, a, b, A, B, dy


def test_b_zero_gives_base_output():
    x, codes, a, b, A, B, _ = _setup()
    key = lora.RngKey(seed=3, layer=1, proj=2)
    y0, _ = lora.fwd(x, codes, a, b, A, np.zeros_like(B), 32.0, 0.1, key)
    ybase, _ = lora.fwd(x, codes, a, b, A[:0], B[:, :0], 32.0, 0.1, key)   # r = 0
    assert np.array_equal(y0, ybase)
    W = nf4.dequantize(codes, a).astype(np.float64)
    # base output by brute force on a few entries
    for t, n in [(0, 0), (3, 17), (5, 63)]:
        s = sum(float(x[t, k]) * float(W[n, k]) for k in range(x.shape[1])) + float(b[n])
        assert abs(ybase[t, n] - s) < 1e-12


def test_zero_weight_is_pure_lora_bruteforce():
    T, K, N, r = 3, 64, 5, 2
    x, _, _, _, A, B, _ = _setup(T, K, N, r, bias=False)
    codes, a = nf4.quantize(np.zeros((N, K), np.float32))
    p = 0.25
    key = lora.RngKey(seed=7, step=2, layer=4, proj=6)
    y, u = lora.fwd(x, codes, a, None, A, B, 32.0, p, key)
    from oracle import philox
    keep = philox.keep_mask(T, K, p, 7, 4, 6, 2, 0)
    sig = float(philox.drop_scale(p))
    s = 32.0 / r
    for t in range(T):
        uu = [sum((float(x[t, k]) * sig if keep[t, k] else 0.0) * float(A[j, k]) for k in range(K))
              for j in range(r)]
        for j in range(r):
            assert abs(u[t, j] - uu[j]) < 1e-12
        for n in range(N):
            want = s * sum(uu[j] * float(B[n, j]) for j in range(r))
            assert abs(y[t, n] - want) < 1e-12


def test_exact_integer_case_bruteforce():
    """W in {-1,0,1}*2^e per block (codes 0/7/15 exactly), integer x, A, B:
    every value is an integer, so the result must match integer arithmetic."""
    rng = np.random.default_rng(9)
    T, K, N, r = 4, 128, 6, 2
    e = rng.integers(-3, 3, size=(N, K // 64))
    sgn = rng.integers(-1, 2, size=(N, K)).astype(np.float32)
    sgn[:, 0] = 1.0
    sgn[:, 64] = -1.0                                     # every block reaches its absmax
    w = sgn * np.repeat(2.0 ** e, 64, axis=1).astype(np.float32)
    codes, a = nf4.quantize(w)
    cu = nf4.unpack(codes)
    assert set(np.unique(cu).tolist()) <= {0, 7, 15}
    assert np.array_equal(nf4.dequantize(codes, a), w)
    x = rng.integers(-4, 5, size=(T, K)).astype(np.float32)
    A = rng.integers(-2, 3, size=(r, K)).astype(np.float32)
    B = rng.integers(-2, 3, size=(N, r)).astype(np.float32)
    dy = rng.integers(-3, 4, size=(T, N)).astype(np.float32)
    key = lora.RngKey()
    y, u = lora.fwd(x, codes, a, None, A, B, 4.0, 0.0, key)          # s = 2
    dx, dA, dB = lora.bwd(dy, x, codes, a, A, B, 4.0, 0.0, key)
    from fractions import Fraction as F
    W = [[F(float(v)) for v in row] for row in w]
    X = [[int(v) for v in row] for row in x]
    for t, n in itertools.product(range(T), range(N)):
        uu = [sum(X[t][k] * int(A[j, k]) for k in range(K)) for j in range(r)]
        want = sum(X[t][k] * W[n][k] for k in range(K)) + 2 * sum(uu[j] * int(B[n, j]) for j in range(r))
        assert F(float(y[t, n])) == want
    for t, k in itertools.product(range(T), range(0, K, 7)):
        du = [2 * sum(int(dy[t, n]) * int(B[n, j]) for n in range(N)) for j in range(r)]
        want = sum(int(dy[t, n]) * W[n][k] for n in range(N)) + sum(du[j] * int(A[j, k]) for j in range(r))
        assert F(float(dx[t, k])) == want


def test_zero_dropout_ignores_key():
    x, codes, a, b, A, B, dy = _setup()
    y1, _ = lora.fwd(x, codes, a, b, A, B, 32.0, 0.0, lora.RngKey(seed=1, layer=2))
    y2, _ = lora.fwd(x, codes, a, b, A, B, 32.0, 0.0, lora.RngKey(seed=5, step=9, proj=3))
    assert np.array_equal(y1, y2)
    g1 = lora.bwd(dy, x, codes, a, A, B, 32.0, 0.0, lora.RngKey(seed=1))
    g2 = lora.bwd(dy, x, codes, a, A, B, 32.0, 0.0, lora.RngKey(seed=8, micro=3))
    for u, v in zip(g1, g2):
        assert np.array_equal(u, v)


def test_finite_differences():
    T, K, N, r = 3, 64, 64, 4
    x, codes, a, b, A, B, dy = _setup(T, K, N, r)
    x = x.astype(np.float64)
    A = A.astype(np.float64)
    B = B.astype(np.float64)
    alpha, p = 8.0, 0.3
    key = lora.RngKey(seed=11, step=1, layer=2, proj=4)
    dyd = dy.astype(np.float64)

    def loss(xx, AA, BB):
        y, _ = lora.fwd(xx, codes, a, b, AA, BB, alpha, p, key)
        return float(np.sum(y * dyd))

    dx, dA, dB = lora.bwd(dy, x, codes, a, A, B, alpha, p, key)
    h = 1e-5
    rng = np.random.default_rng(0)
    for arr, grad, which in ((x, dx, 0), (A, dA, 1), (B, dB, 2)):
        for _ in range(12):
            idx = tuple(int(rng.integers(0, s)) for s in arr.shape)
            args = [x, A, B]
            plus = [v.copy() for v in args]
            minus = [v.copy() for v in args]
            plus[which][idx] += h
            minus[which][idx] -= h
            fd = (loss(*plus) - loss(*minus)) / (2 * h)
            assert abs(fd - grad[idx]) <= 1e-6 * max(1.0, abs(fd)), (which, idx, fd, grad[idx])
