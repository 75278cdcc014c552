"""NF4-quantized frozen linear layer with a LoRA adapter: forward and backward (oracle).

What is computed follows the problem the pages state: the base is frozen and
4-bit, read block by block, and only the adapters are trained; the backward
"propagates gradients only to the adapters and block inputs", frozen weights
are never differentiated ("Poros" research post, the paragraph describing the
training step; package README, "How it works").

Readings (the pages give only r and alpha -- rank 16, alpha 32 in the README
"Quickstart" and the A100 "Configuration" table -- and say dropout exists):
  * y  = x W^T + b + s * (drop(x) A^T) B^T, with s = alpha / r (standard LoRA
    scaling), dropout on the LoRA input only (inverted dropout, see philox.py)
  * u  = drop(x) A^T                       (saved for the backward)
  * du = s * dy B
  * dB = s * dy^T u
  * dA = du^T drop(x)
  * dx = dy W + sigma * keep (.) (du A)
  * no gradient for W, its absmax, or the bias (frozen).
W here is the dequantized NF4 matrix, or for a bf16 base ("Current limitations",
"bf16 LoRA": the same streaming with the frozen base kept in bf16) the bf16 matrix
itself.  All contractions run in float64 on exactly-represented inputs (bf16 x, fp32 A
and B, bf16 W).

Operands of the frozen-base product (reading).  The dequantized base is a bf16 matrix,
and the product that consumes it is a bf16 matrix-core product: both of its operands
are bf16, accumulated in fp32 (the pages gate their parity with bf16 products switched
on, "Poros" research post, bitwise-parity paragraph, mode sweep with bf16 autocast).
With bf16 activations -- the single-layer and single-block workloads -- this changes
nothing.  A stack that keeps its activations between projections in fp32 feeds the base
product bf16(x) in the forward and bf16(dy) in the input gradient, while the rank-r
adapter products see the fp32 values.  operand="bf16" states exactly that: the
activation entering x W^T, and the gradient entering dy W, are rounded to bf16
(round to nearest, ties to even) first; nothing else changes.  operand="exact" (the
default) takes them as given.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

from . import nf4, philox


@dataclass(frozen=True)
class RngKey:
    seed: int = 0
    step: int = 0
    micro: int = 0
    layer: int = 0
    proj: int = 0


OPERANDS = ("exact", "bf16")


def base_operand(a: np.ndarray, operand: str) -> np.ndarray:
    """The activation (or gradient) as the frozen-base product receives it, float64:
    unchanged ("exact") or rounded to bf16 ("bf16", see the module docstring).  A float64
    value is first taken to fp32, the type the activations have between projections."""
    if operand not in OPERANDS:
        raise ValueError(f"operand must be one of {OPERANDS}, got {operand!r}")
    if operand == "bf16":
        a = nf4.bf16_round(np.asarray(a, dtype=np.float32))
    return np.asarray(a).astype(np.float64)


def lora_input(x: np.ndarray, p: float, key: RngKey) -> np.ndarray:
    """drop(x) = keep (.) x * sigma in float64."""
    T, K = x.shape
    keep = philox.keep_mask(T, K, p, key.seed, key.layer, key.proj, key.step, key.micro)
    sigma = float(philox.drop_scale(p))
    return np.where(keep, x.astype(np.float64) * sigma, 0.0), keep, sigma


def fwd_dense(x: np.ndarray, W: np.ndarray, bias: Optional[np.ndarray], A: np.ndarray, B: np.ndarray,
              alpha: float, p: float, key: RngKey, operand: str = "exact"):
    """The layer with its frozen base given as values (bf16 W [N, K], or the dequantized
    NF4 matrix).  Returns (y, u) in float64.  r = A.shape[0]; r = 0 means base only.

    Output columns are independent: rows n of W, bias and B give columns n of y, so a
    caller may pass those rows alone to evaluate y on a subset of its columns (u needs
    all of x and A either way)."""
    W = W.astype(np.float64)
    y = base_operand(x, operand) @ W.T
    if bias is not None:
        y = y + bias.astype(np.float64)[None, :]
    r = A.shape[0]
    if r == 0:
        return y, np.zeros((x.shape[0], 0))
    s = alpha / r
    h, _, _ = lora_input(x, p, key)
    u = h @ A.astype(np.float64).T
    y = y + s * (u @ B.astype(np.float64).T)
    return y, u


def bwd_dense(dy: np.ndarray, x: np.ndarray, W: np.ndarray, A: np.ndarray, B: np.ndarray,
              alpha: float, p: float, key: RngKey, operand: str = "exact",
              dx_cols: Optional[np.ndarray] = None):
    """Returns (dx, dA, dB) in float64, replaying the forward's mask from the key.

    dx_cols: evaluate dx only on these input columns.  W is then the matching columns
    W[:, dx_cols] of the frozen base; x, A and B stay whole (dA, dB and the mask's
    element indices need them) and dx comes back as [T, len(dx_cols)]."""
    W = W.astype(np.float64)
    dy64 = dy.astype(np.float64)
    dx = base_operand(dy, operand) @ W
    r = A.shape[0]
    if r == 0:
        return dx, np.zeros((0, x.shape[1])), np.zeros((B.shape[0], 0))
    s = alpha / r
    h, keep, sigma = lora_input(x, p, key)
    A64 = A.astype(np.float64)
    u = h @ A64.T
    du = s * (dy64 @ B.astype(np.float64))
    dB = s * (dy64.T @ u)
    dA = du.T @ h
    if dx_cols is None:
        dx = dx + sigma * np.where(keep, du @ A64, 0.0)
    else:
        dx = dx + sigma * np.where(keep[:, dx_cols], du @ A64[:, dx_cols], 0.0)
    return dx, dA, dB


def fwd(x: np.ndarray, codes: np.ndarray, absmax: np.ndarray, bias: Optional[np.ndarray],
        A: np.ndarray, B: np.ndarray, alpha: float, p: float, key: RngKey):
    """The NF4 layer: W is the dequantized matrix."""
    return fwd_dense(x, nf4.dequantize(codes, absmax), bias, A, B, alpha, p, key)


def bwd(dy: np.ndarray, x: np.ndarray, codes: np.ndarray, absmax: np.ndarray,
        A: np.ndarray, B: np.ndarray, alpha: float, p: float, key: RngKey):
    return bwd_dense(dy, x, nf4.dequantize(codes, absmax), A, B, alpha, p, key)
