"""One training step of the Qwen2.5-shaped stack (oracle).

The step the pages describe ("Poros" research post, the paragraph on the
training step): the forward runs the blocks in order keeping activations at
block boundaries; the backward walks the blocks in reverse, recomputes each
block's forward with the restored RNG, and propagates gradients to the adapters
and block inputs only; then one optimizer step, identical to a resident run's.
The learning problem is unchanged by streaming (same paragraph group: same
attention kernels, optimizer, LoRA configuration, data order, loss).

Readings (the pages name none of these):
  * frozen bf16 token embedding and untied lm_head, neither quantized nor
    adapted; a final RMSNorm (eps 1e-6) before the lm_head
  * loss = mean next-token cross-entropy over the T-1 positions that have a
    target
  * global gradient norm over all adapter gradients, float64
  * AdamW with decoupled weight decay and bias correction (Loshchilov and
    Hutter, "Decoupled Weight Decay Regularization", ICLR 2019):
    lr 2e-4, betas (0.9, 0.999), eps 1e-8, weight decay 0.01, constant
    schedule, no clipping.

Parity status: the loss of a random-weight stack has no printed value on the
pages, so this composition is parity unpinned against absolute values; its
parts are pinned individually and the whole is pinned by finite differences.
"""
from __future__ import annotations

from typing import Dict, List

import numpy as np

from . import block, lora

LR, BETA1, BETA2, ADAM_EPS, WD = 2e-4, 0.9, 0.999, 1e-8, 0.01


def loss_and_dlogits(logits: np.ndarray, tokens: np.ndarray):
    """Mean CE over positions 0..T-2 predicting tokens[1..T-1]."""
    T = logits.shape[0]
    z = logits[:-1]
    tgt = tokens[1:]
    zmax = z.max(axis=1, keepdims=True)
    lse = zmax[:, 0] + np.log(np.exp(z - zmax).sum(axis=1))
    loss = float(np.mean(lse - z[np.arange(T - 1), tgt]))
    P = np.exp(z - lse[:, None])
    P[np.arange(T - 1), tgt] -= 1.0
    d = np.zeros_like(logits)
    d[:-1] = P / (T - 1)
    return loss, d


def forward_backward(layers: List[Dict[str, object]], glob: Dict[str, np.ndarray],
                     toks: np.ndarray, shape, alpha: float, p: float, seed: int, step: int,
                     micro: int = 0, operand: str = "exact", trace: bool = False):
    """Returns (loss, grads[layer][proj] = (dA, dB)).  layers hold quantized params.
    operand: how activations and gradients enter the frozen-base products
    (lora.base_operand); "bf16" is the stack with fp32 activations on bf16 matrix cores.
    trace: also return {"inputs", "outputs", "d_outputs", "d_inputs"}, per layer: the
    block's input and output activations and the loss gradients at its output and input
    (the values this composition already forms, kept for layer-by-layer comparisons)."""
    rk = lora.RngKey(seed=seed, step=step, micro=micro)
    h = glob["emb"][toks].astype(np.float64)
    bounds = []
    outputs = []
    for li, qp in enumerate(layers):
        bounds.append(h)
        h, _ = block.forward(h, qp, shape, li, alpha, p, rk, operand)
        outputs.append(h)
    hn, rinv = block.rmsnorm(h, glob["lnf"].astype(np.float64))
    logits = hn @ glob["lm"].astype(np.float64).T
    loss, dlog = loss_and_dlogits(logits, toks)
    dhn = dlog @ glob["lm"].astype(np.float64)
    dh = block.rmsnorm_bwd(h, glob["lnf"].astype(np.float64), rinv, dhn)
    grads: List[Dict[str, tuple]] = [None] * len(layers)
    d_out, d_in = [None] * len(layers), [None] * len(layers)
    for li in reversed(range(len(layers))):
        qp = layers[li]
        _, cache = block.forward(bounds[li], qp, shape, li, alpha, p, rk, operand)  # recompute
        d_out[li] = dh
        dh, grads[li] = block.backward(dh, cache, qp, shape, li, alpha, p, rk, operand)
        d_in[li] = dh
    if trace:
        return loss, grads, {"inputs": bounds, "outputs": outputs, "d_outputs": d_out, "d_inputs": d_in}
    return loss, grads


def accumulated(layers: List[Dict[str, object]], glob: Dict[str, np.ndarray], toks_list,
                shape, alpha: float, p: float, seed: int, step: int, operand: str = "exact"):
    """Gradient accumulation over M micro-batches ("Poros" research post and "Current
    limitations", "What 0.00e+00 means": accumulation at 2 and 4 micro-batches is part of
    the parity surface).  Reading: one optimizer step sees the mean of the micro-batch
    losses and its gradient, the mean of the micro-batch gradients; micro-batch m keys its
    dropout masks with micro = m.  The order in which the micro-batches and blocks are
    visited is not part of the definition.  Returns (mean loss, grads)."""
    M = len(toks_list)
    total, acc = 0.0, None
    for m, toks in enumerate(toks_list):
        loss, g = forward_backward(layers, glob, toks, shape, alpha, p, seed, step, micro=m, operand=operand)
        total += loss
        if acc is None:
            acc = [{proj: (dA.astype(np.float64), dB.astype(np.float64)) for proj, (dA, dB) in gl.items()}
                   for gl in g]
        else:
            acc = [{proj: (a[proj][0] + gl[proj][0], a[proj][1] + gl[proj][1]) for proj in a}
                   for a, gl in zip(acc, g)]
    return total / M, [{proj: (dA / M, dB / M) for proj, (dA, dB) in a.items()} for a in acc]


def grad_norm(grads) -> float:
    s = 0.0
    for g in grads:
        for proj in block.PROJS:
            dA, dB = g[proj]
            s += float(np.sum(dA.astype(np.float64) ** 2) + np.sum(dB.astype(np.float64) ** 2))
    return float(np.sqrt(s))


def adamw(param: np.ndarray, grad: np.ndarray, m: np.ndarray, v: np.ndarray, t: int,
          lr: float = LR, b1: float = BETA1, b2: float = BETA2, eps: float = ADAM_EPS,
          wd: float = WD):
    """One AdamW update (t counts from 1); float64; returns (param, m, v)."""
    param = param.astype(np.float64) * (1.0 - lr * wd)
    m = b1 * m + (1.0 - b1) * grad
    v = b2 * v + (1.0 - b2) * grad * grad
    mhat = m / (1.0 - b1 ** t)
    vhat = v / (1.0 - b2 ** t)
    return param - lr * mhat / (np.sqrt(vhat) + eps), m, v
