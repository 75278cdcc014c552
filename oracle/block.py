"""Qwen2.5-shaped decoder block with seven NF4 + LoRA projections (oracle).

The pages validate the Qwen2.5 family ("Poros" research post, the list of
families with bitwise parity; package README, "Supported models") and name the
pointwise pieces of its block -- SwiGLU multiply, residual adds, rotary
embeddings with precomputed tables ("Limitations", "Roadmap", the paragraph on
the Poros kernel).  Block math is a reading of the Qwen2 architecture:

  xn  = RMSNorm(x; w1, eps 1e-6)
  q,k,v = NF4-LoRA projections of xn (with bias)
  q,k   = RoPE (rotate-half form, base theta = 1e6, positions 0..T-1)
  att   = causal grouped-query attention, softmax scale 1/sqrt(head_dim), query
          head h reads kv head h // (heads / kv_heads)
  x1  = x + o(att)
  xn2 = RMSNorm(x1; w2)
  out = x1 + down(SiLU(gate(xn2)) * up(xn2))

The frozen base of each projection is NF4 (quantize_params) or kept in bf16
(bf16_params, the pages' bf16 streaming variant).  Each projection draws its dropout
mask from the key (seed, step, micro, layer, proj), so the recompute in the backward
replays it ("Poros" research post, RNG
state capture).  The backward is derived by hand and differentiates only the
adapters and the block input (frozen norms, frozen base).
"""
from __future__ import annotations

from typing import Dict

import numpy as np

from . import lora, nf4

PROJS = ("q", "k", "v", "o", "gate", "up", "down")
PROJ_ID = {p: i for i, p in enumerate(PROJS)}
EPS = 1e-6
THETA = 1.0e6


def quantize_params(params: Dict[str, object]) -> Dict[str, object]:
    """Replace each projection's bf16 W by its NF4 (codes, absmax)."""
    q = {}
    for proj in PROJS:
        pp = params[proj]
        codes, a = nf4.quantize(pp["W"])
        q[proj] = {"codes": codes, "absmax": a, "bias": pp["bias"], "A": pp["A"], "B": pp["B"]}
    q["ln1"] = params["ln1"]
    q["ln2"] = params["ln2"]
    return q


def bf16_params(params: Dict[str, object]) -> Dict[str, object]:
    """Keep each projection's bf16 W as the frozen base (no quantization)."""
    q = {proj: {k: params[proj][k] for k in ("W", "bias", "A", "B")} for proj in PROJS}
    q["ln1"] = params["ln1"]
    q["ln2"] = params["ln2"]
    return q


def rmsnorm(x, w):
    rinv = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + EPS)
    return x * rinv * w, rinv


def rmsnorm_bwd(x, w, rinv, dy):
    g = dy * w
    n = x.shape[-1]
    return rinv * g - x * (rinv ** 3) * np.sum(x * g, axis=-1, keepdims=True) / n


def rope_tables(T: int, D: int):
    inv_freq = THETA ** (-np.arange(0, D, 2, dtype=np.float64) / D)
    ang = np.arange(T, dtype=np.float64)[:, None] * inv_freq[None, :]
    cos = np.concatenate([np.cos(ang), np.cos(ang)], axis=1)
    sin = np.concatenate([np.sin(ang), np.sin(ang)], axis=1)
    return cos, sin


def rotate_half(x):
    h = x.shape[-1] // 2
    return np.concatenate([-x[..., h:], x[..., :h]], axis=-1)


def rotate_half_T(g):
    h = g.shape[-1] // 2
    return np.concatenate([g[..., h:], -g[..., :h]], axis=-1)


def rope(x, cos, sin):
    """x: [T, H, D]"""
    return x * cos[:, None, :] + rotate_half(x) * sin[:, None, :]


def rope_bwd(g, cos, sin):
    return g * cos[:, None, :] + rotate_half_T(g * sin[:, None, :])


def attention(q, k, v, heads, kv_heads):
    """Causal GQA; q [T,H,D], k/v [T,KV,D] -> out [T,H,D], probs [H,T,T]."""
    T, H, D = q.shape
    grp = heads // kv_heads
    out = np.empty_like(q)
    probs = np.empty((H, T, T))
    causal = np.triu(np.ones((T, T), dtype=bool), 1)
    for h in range(H):
        g = h // grp
        s = q[:, h, :] @ k[:, g, :].T / np.sqrt(D)
        s = np.where(causal, -np.inf, s)
        s = s - s.max(axis=1, keepdims=True)
        e = np.exp(s)
        P = e / e.sum(axis=1, keepdims=True)
        probs[h] = P
        out[:, h, :] = P @ v[:, g, :]
    return out, probs


def attention_bwd(dout, q, k, v, probs, heads, kv_heads):
    T, H, D = q.shape
    grp = heads // kv_heads
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for h in range(H):
        g = h // grp
        P = probs[h]
        do = dout[:, h, :]
        dv[:, g, :] += P.T @ do
        dP = do @ v[:, g, :].T
        dS = P * (dP - np.sum(dP * P, axis=1, keepdims=True))
        dq[:, h, :] = dS @ k[:, g, :] / np.sqrt(D)
        dk[:, g, :] += dS.T @ q[:, h, :] / np.sqrt(D)
    return dq, dk, dv


def silu(g):
    return g / (1.0 + np.exp(-g))


def silu_grad(g):
    sg = 1.0 / (1.0 + np.exp(-g))
    return sg * (1.0 + g * (1.0 - sg))


def base_weight(pp: Dict[str, object]) -> np.ndarray:
    """A projection's frozen base as values: the bf16 W, or the dequantized NF4 codes."""
    if "W" in pp:
        return pp["W"]
    return nf4.dequantize(pp["codes"], pp["absmax"])


def _key(rk: lora.RngKey, layer: int, proj: str) -> lora.RngKey:
    return lora.RngKey(seed=rk.seed, step=rk.step, micro=rk.micro, layer=layer,
                       proj=PROJ_ID[proj])


def forward(x, qp, shape, layer: int, alpha: float, p: float, rk: lora.RngKey, operand: str = "exact"):
    """x: [T, hidden] (float values) -> (out float64 [T, hidden], cache).  operand: how the
    activations enter the frozen-base products (lora.base_operand)."""
    H, KV, D = shape.heads, shape.kv_heads, shape.head_dim
    T = x.shape[0]
    x = x.astype(np.float64)
    c = {"x": x}
    xn, c["rinv1"] = rmsnorm(x, qp["ln1"].astype(np.float64))
    c["xn"] = xn

    def lin(inp, proj):
        pp = qp[proj]
        y, _ = lora.fwd_dense(inp, base_weight(pp), pp["bias"], pp["A"], pp["B"], alpha, p,
                              _key(rk, layer, proj), operand)
        return y

    q = lin(xn, "q").reshape(T, H, D)
    k = lin(xn, "k").reshape(T, KV, D)
    v = lin(xn, "v").reshape(T, KV, D)
    cos, sin = rope_tables(T, D)
    c["cos"], c["sin"] = cos, sin
    qr, kr = rope(q, cos, sin), rope(k, cos, sin)
    att, probs = attention(qr, kr, v, H, KV)
    c.update(qr=qr, kr=kr, v=v, probs=probs)
    att2 = att.reshape(T, H * D)
    c["att"] = att2
    x1 = x + lin(att2, "o")
    c["x1"] = x1
    xn2, c["rinv2"] = rmsnorm(x1, qp["ln2"].astype(np.float64))
    c["xn2"] = xn2
    g = lin(xn2, "gate")
    u = lin(xn2, "up")
    a = silu(g) * u
    c.update(g=g, u=u, a=a)
    out = x1 + lin(a, "down")
    return out, c


def backward(dout, c, qp, shape, layer: int, alpha: float, p: float, rk: lora.RngKey,
             operand: str = "exact"):
    """Returns (dx float64 [T, hidden], grads {proj: (dA, dB)}).  operand: how the incoming
    gradients enter the frozen-base products (lora.base_operand)."""
    H, KV, D = shape.heads, shape.kv_heads, shape.head_dim
    T = dout.shape[0]
    dout = dout.astype(np.float64)
    grads = {}

    def lin_bwd(dy, inp, proj):
        pp = qp[proj]
        dx, dA, dB = lora.bwd_dense(dy, inp, base_weight(pp), pp["A"], pp["B"], alpha, p,
                                    _key(rk, layer, proj), operand)
        grads[proj] = (dA, dB)
        return dx

    dx1 = dout.copy()
    da = lin_bwd(dout, c["a"], "down")
    g, u = c["g"], c["u"]
    dg = da * u * silu_grad(g)
    du = da * silu(g)
    dxn2 = lin_bwd(dg, c["xn2"], "gate") + lin_bwd(du, c["xn2"], "up")
    dx1 = dx1 + rmsnorm_bwd(c["x1"], qp["ln2"].astype(np.float64), c["rinv2"], dxn2)
    datt = lin_bwd(dx1, c["att"], "o").reshape(T, H, D)
    dqr, dkr, dv = attention_bwd(datt, c["qr"], c["kr"], c["v"], c["probs"], H, KV)
    dq = rope_bwd(dqr, c["cos"], c["sin"]).reshape(T, H * D)
    dk = rope_bwd(dkr, c["cos"], c["sin"]).reshape(T, KV * D)
    dv = dv.reshape(T, KV * D)
    dxn = lin_bwd(dq, c["xn"], "q") + lin_bwd(dk, c["xn"], "k") + lin_bwd(dv, c["xn"], "v")
    dx = dx1 + rmsnorm_bwd(c["x"], qp["ln1"].astype(np.float64), c["rinv1"], dxn)
    return dx, grads
