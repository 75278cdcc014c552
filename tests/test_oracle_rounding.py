"""How far the bf16 operands of the frozen-base product move a stack's adapter gradients
(CPU only).

The library runs the frozen-base product on bf16 matrix cores: a stack that keeps its
activations in fp32 feeds that product bf16(x) forward and bf16(dy) backward, while the
rank-r adapter products see the fp32 values.  The oracle states this as operand="bf16"
(oracle/lora.py, pinned in test_oracle_operand.py).  Through a 3-layer chain at 32 tokens
those two roundings alone move some adapter gradients by more than 1e-2 * RMS of the
exact-operand result, so the GPU stack is held to the 2e-2 * RMS bar against the
operand="bf16" oracle, the computation it actually performs.
"""
import numpy as np

import msq_inputs as mi
from oracle import block, step

TINY = mi.BlockShape(hidden=128, heads=2, kv_heads=1, head_dim=64, inter=256, layers=3, vocab=512)


def test_bf16_operand_rounding_envelope():
    lo, seed, T = mi.LoraSpec(8, 16.0, 0.1), 1, 32
    layers = [block.quantize_params(mi.block_params(seed, 3, l, TINY, lo)) for l in range(3)]
    glob = mi.stack_globals(seed, 3, TINY, T)
    toks = mi.tokens(seed, 3, 0, T, TINY.vocab)
    ref_loss, ref = step.forward_backward(layers, glob, toks, TINY, lo.alpha, lo.p_drop, seed, 0)
    loss, got = step.forward_backward(layers, glob, toks, TINY, lo.alpha, lo.p_drop, seed, 0, operand="bf16")
    worst = max(np.max(np.abs(got[l][p][w] - ref[l][p][w])) / np.sqrt(np.mean(ref[l][p][w] ** 2))
                for l in range(3) for p in block.PROJS for w in (0, 1))
    assert abs(loss - ref_loss) < 1e-3 * abs(ref_loss)
    assert 1e-2 < worst <= 2.7e-2, worst
