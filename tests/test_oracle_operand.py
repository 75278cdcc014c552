"""Pins for the oracle's reading of the frozen-base product's operands (CPU only).

operand="bf16": the activation entering x W^T and the gradient entering dy W are rounded to
bf16 (round to nearest, ties to even); the rank-r adapter products keep the unrounded
values.  Pinned by hand-worked bf16 roundings through an identity base (every expected
value below is written out, not computed by a rounding routine), by the identity on
bf16-valued inputs, and by agreement with an independently written rounding of the
same two operands inside a whole stack step.  dx_cols (dx on a subset of input columns)
and row subsets of the forward are pinned against the full evaluation."""
import numpy as np
import pytest

import msq_inputs as mi
from oracle import block, lora, nf4, step

# (fp32 input, its bf16 rounding): ties to even, just above a tie, below half a spacing,
# a non-bf16 fraction, a subnormal; worked by hand from the bit patterns
CASES = [
    (1.0 + 2.0 ** -8, 1.0),                           # tie between 1 and 1 + 2^-7 -> even (1)
    (1.0 + 3 * 2.0 ** -8, 1.015625),                   # tie between 1 + 2^-7 (odd) and 1 + 2^-6 -> 1 + 2^-6
    (1.0 + 2.0 ** -8 + 2.0 ** -20, 1.0078125),         # just above the tie -> up
    (-(3.0 + 2.0 ** -10), -3.0),                       # below half the 2^-6 spacing at 3 -> down
    (np.float32(0.1), 0.10009765625),                  # 0x3DCCCCCD -> 0x3DCD
    (np.float32(1e-40), 2.0 ** -133),                  # subnormal 0x000116C2 -> 0x0001
    (-(2.0 ** -7 + 2.0 ** -15), -(2.0 ** -7)),         # negative tie at 2^-7 (spacing 2^-14) -> even
    (65792.0, 65536.0),                                # tie between 65536 (even) and 66048 -> 65536
]


def _identity_base(K):
    """The NF4 round trip of the identity is the identity (block max 1 -> code 15 -> 1.0,
    zeros -> code 7 -> 0.0)."""
    codes, a = nf4.quantize(np.eye(K, dtype=np.float32))
    W = nf4.dequantize(codes, a)
    assert np.array_equal(W, np.eye(K, dtype=np.float32))
    return W


def test_forward_rounds_the_base_operand_only():
    K = 64
    W = _identity_base(K)
    x = np.zeros((1, K), np.float32)
    for i, (v, _) in enumerate(CASES):
        x[0, i] = v
    want = np.zeros(K)
    for i, (_, r) in enumerate(CASES):
        want[i] = r
    A = np.zeros((2, K), np.float32)
    A[0, 0] = 1.0      # u[:, 0] = x[:, 0], unrounded
    A[1, 4] = 1.0      # u[:, 1] = x[:, 4]
    B0 = np.zeros((K, 2), np.float32)
    y, u = lora.fwd_dense(x, W, None, A, B0, 32.0, 0.0, lora.RngKey(), operand="bf16")
    assert np.array_equal(y[0], want)
    assert u[0, 0] == np.float32(1.0 + 2.0 ** -8) and u[0, 1] == np.float32(0.1)
    ye, _ = lora.fwd_dense(x, W, None, A, B0, 32.0, 0.0, lora.RngKey(), operand="exact")
    assert np.array_equal(ye[0], x[0].astype(np.float64))
    # the adapter term is added to the rounded base product, from unrounded u
    B = np.zeros((K, 2), np.float32)
    B[5, 0] = 1.0
    y2, _ = lora.fwd_dense(x, W, None, A, B, 32.0, 0.0, lora.RngKey(), operand="bf16")
    assert y2[0, 5] == 2.0 ** -133 + 16.0 * (1.0 + 2.0 ** -8)


def test_backward_rounds_the_base_operand_only():
    K = 64
    W = _identity_base(K)
    dy = np.zeros((1, K), np.float32)
    for i, (v, _) in enumerate(CASES):
        dy[0, i] = v
    want = np.zeros(K)
    for i, (_, r) in enumerate(CASES):
        want[i] = r
    x = np.zeros((1, K), np.float32)
    x[0, 3] = 1.0
    A = np.zeros((1, K), np.float32)
    A[0, 3] = 1.0                                          # u = x[:, 3] = 1
    B0 = np.zeros((K, 1), np.float32)
    dx, dA, dB = lora.bwd_dense(dy, x, W, A, B0, 2.0, 0.0, lora.RngKey(), operand="bf16")
    assert np.array_equal(dx[0], want)                     # du = 0: dx is the base term alone
    assert dB[0, 0] == 2.0 * (1.0 + 2.0 ** -8)             # s dy^T u with the unrounded dy
    assert dB[4, 0] == 2.0 * float(np.float32(0.1))
    # du = s dy B reads the unrounded dy too, and enters dx through A unrounded
    B = np.zeros((K, 1), np.float32)
    B[0, 0] = 1.0
    dx2, dA2, _ = lora.bwd_dense(dy, x, W, A, B, 2.0, 0.0, lora.RngKey(), operand="bf16")
    assert dx2[0, 3] == want[3] + 2.0 * (1.0 + 2.0 ** -8)
    assert dA2[0, 3] == 2.0 * (1.0 + 2.0 ** -8)


def test_bf16_inputs_are_unchanged_by_the_operand_rounding():
    rng = np.random.default_rng(5)
    T, K, N, r = 9, 128, 64, 4
    x = nf4.bf16_round(rng.standard_normal((T, K)).astype(np.float32))
    dy = nf4.bf16_round(rng.standard_normal((T, N)).astype(np.float32))
    W = nf4.bf16_round((0.05 * rng.standard_normal((N, K))).astype(np.float32))
    A = rng.uniform(-0.1, 0.1, (r, K)).astype(np.float32)
    B = (0.1 * rng.standard_normal((N, r))).astype(np.float32)
    key = lora.RngKey(seed=2, layer=1, proj=3)
    for a, b in zip(lora.fwd_dense(x, W, None, A, B, 8.0, 0.2, key, "exact"),
                    lora.fwd_dense(x, W, None, A, B, 8.0, 0.2, key, "bf16")):
        assert np.array_equal(a, b)
    for a, b in zip(lora.bwd_dense(dy, x, W, A, B, 8.0, 0.2, key, "exact"),
                    lora.bwd_dense(dy, x, W, A, B, 8.0, 0.2, key, "bf16")):
        assert np.array_equal(a, b)
    with pytest.raises(ValueError):
        lora.base_operand(x, "fp8")


def test_column_subsets_equal_the_full_evaluation():
    rng = np.random.default_rng(8)
    T, K, N, r = 7, 192, 128, 8
    x = rng.standard_normal((T, K)).astype(np.float32)
    dy = rng.standard_normal((T, N)).astype(np.float32)
    W = nf4.bf16_round((0.05 * rng.standard_normal((N, K))).astype(np.float32))
    A = rng.uniform(-0.1, 0.1, (r, K)).astype(np.float32)
    B = (0.1 * rng.standard_normal((N, r))).astype(np.float32)
    bias = nf4.bf16_round((0.02 * rng.standard_normal(N)).astype(np.float32))
    key = lora.RngKey(seed=9, step=4, layer=2, proj=5)
    for operand in ("exact", "bf16"):
        y, u = lora.fwd_dense(x, W, bias, A, B, 16.0, 0.3, key, operand)
        rows = np.array([0, 5, 64, 127])
        ys, us = lora.fwd_dense(x, W[rows], bias[rows], A, B[rows], 16.0, 0.3, key, operand)
        assert np.allclose(ys, y[:, rows], rtol=0, atol=1e-12) and np.array_equal(us, u)
        dx, dA, dB = lora.bwd_dense(dy, x, W, A, B, 16.0, 0.3, key, operand)
        cols = np.array([1, 63, 64, 150, 191])
        dxs, dAs, dBs = lora.bwd_dense(dy, x, W[:, cols], A, B, 16.0, 0.3, key, operand, dx_cols=cols)
        assert dxs.shape == (T, cols.size)
        assert np.allclose(dxs, dx[:, cols], rtol=0, atol=1e-12)
        assert np.array_equal(dAs, dA) and np.array_equal(dBs, dB)


def _independent_fwd(x, W, bias, A, B, alpha, p, key):
    """The bf16 operand rounding written separately from lora.base_operand."""
    xr = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    xr = ((xr + 0x7FFF + ((xr >> 16) & 1)) >> 16 << 16).astype(np.uint32).view(np.float32)
    y = xr.astype(np.float64) @ W.astype(np.float64).T + (bias.astype(np.float64) if bias is not None else 0.0)
    h, _, _ = lora.lora_input(x, p, key)
    u = h @ A.astype(np.float64).T
    return y + alpha / A.shape[0] * (u @ B.astype(np.float64).T), u


def _independent_bwd(dy, x, W, A, B, alpha, p, key):
    dr = np.asarray(dy, np.float32).view(np.uint32).astype(np.uint64)
    dr = ((dr + 0x7FFF + ((dr >> 16) & 1)) >> 16 << 16).astype(np.uint32).view(np.float32)
    s = alpha / A.shape[0]
    h, keep, sig = lora.lora_input(x, p, key)
    A64, B64 = A.astype(np.float64), B.astype(np.float64)
    u = h @ A64.T
    du = s * dy.astype(np.float64) @ B64
    return dr.astype(np.float64) @ W.astype(np.float64) + sig * np.where(keep, du @ A64, 0.0), du.T @ h, s * dy.T @ u


def test_stack_with_bf16_operands_matches_an_independent_rounding(monkeypatch):
    """A 3-layer stack step with operand="bf16" equals the same step with the two roundings
    inserted by separately written code (integer RNE on the fp32 bit patterns).  The
    activations are float64 in the oracle; both routes take them to fp32 first."""
    TINY = mi.BlockShape(hidden=128, heads=2, kv_heads=1, head_dim=64, inter=256, layers=3, vocab=512)
    lo, seed, T = mi.LoraSpec(8, 16.0, 0.1), 1, 32
    layers = [block.quantize_params(mi.block_params(seed, 3, l, TINY, lo)) for l in range(3)]
    glob = mi.stack_globals(seed, 3, TINY, T)
    toks = mi.tokens(seed, 3, 0, T, TINY.vocab)
    loss_b, got_b = step.forward_backward(layers, glob, toks, TINY, lo.alpha, lo.p_drop, seed, 0, operand="bf16")
    monkeypatch.setattr(block.lora, "fwd_dense", lambda x, W, b, A, B, al, p, k, op: _independent_fwd(
        x, W, b, A, B, al, p, k))
    monkeypatch.setattr(block.lora, "bwd_dense", lambda dy, x, W, A, B, al, p, k, op: _independent_bwd(
        dy, x, W, A, B, al, p, k))
    loss_i, got_i = step.forward_backward(layers, glob, toks, TINY, lo.alpha, lo.p_drop, seed, 0)
    assert loss_b == loss_i
    for l in range(3):
        for p in block.PROJS:
            for w in (0, 1):
                assert np.allclose(got_b[l][p][w], got_i[l][p][w], rtol=1e-12, atol=0)
