"""Sensitivity of the stack's adapter gradients to bf16 operand rounding (CPU only).

The library runs the frozen-base product on bf16 MFMA: activations are rounded to
bf16 for that product in the forward, and incoming gradients are rounded to bf16 for
the dx product in the backward; everything else (LoRA products, glue) keeps fp32
values.  Re-running the oracle with exactly those two roundings inserted -- and
nothing else changed -- measures how far that arithmetic alone moves the results.
The GPU stack test uses twice this envelope as its tolerance for a 3-layer chain.
"""
import numpy as np

import msq_inputs as mi
import oracle.lora as OL
from oracle import block, nf4, step

TINY = mi.BlockShape(hidden=128, heads=2, kv_heads=1, head_dim=64, inter=256, layers=3, vocab=512)


def _r16(x):
    return nf4.bf16_round(np.asarray(x, np.float32)).astype(np.float64)


def _fwd(x, W, bias, A, B, alpha, p, key):
    W = W.astype(np.float64)
    y = _r16(x) @ W.T + (bias.astype(np.float64) if bias is not None else 0.0)
    h, _, _ = OL.lora_input(x, p, key)
    u = h @ A.astype(np.float64).T
    return y + alpha / A.shape[0] * (u @ B.astype(np.float64).T), u


def _bwd(dy, x, W, A, B, alpha, p, key):
    W = W.astype(np.float64)
    s = alpha / A.shape[0]
    h, keep, sig = OL.lora_input(x, p, key)
    A64, B64 = A.astype(np.float64), B.astype(np.float64)
    u = h @ A64.T
    du = s * dy @ B64
    return _r16(dy) @ W + sig * np.where(keep, du @ A64, 0.0), du.T @ h, s * dy.T @ u


def test_bf16_operand_rounding_envelope(monkeypatch):
    lo, seed, T = mi.LoraSpec(8, 16.0, 0.1), 1, 32
    layers = [block.quantize_params(mi.block_params(seed, 3, l, TINY, lo)) for l in range(3)]
    glob = mi.stack_globals(seed, 3, TINY, T)
    toks = mi.tokens(seed, 3, 0, T, TINY.vocab)
    ref_loss, ref = step.forward_backward(layers, glob, toks, TINY, lo.alpha, lo.p_drop, seed, 0)
    monkeypatch.setattr(block.lora, "fwd_dense", _fwd)
    monkeypatch.setattr(block.lora, "bwd_dense", _bwd)
    loss, got = step.forward_backward(layers, glob, toks, TINY, lo.alpha, lo.p_drop, seed, 0)
    worst = max(np.max(np.abs(got[l][p][w] - ref[l][p][w])) / np.sqrt(np.mean(ref[l][p][w] ** 2))
                for l in range(3) for p in block.PROJS for w in (0, 1))
    assert abs(loss - ref_loss) < 1e-3 * abs(ref_loss)
    assert 1e-2 < worst <= 2.7e-2, worst
