"""Seeded synthetic input generators shared by the oracle, the tests and the bench.

This module holds no arithmetic of the method (no quantization, no LoRA, no
dropout): it only draws the random tensors that both sides consume, so that the
HIP path and the CPU oracle see identical inputs.  Every tensor is drawn from
``numpy.random.default_rng([seed, cfg_id, layer, tensor_id])`` so that drawing
order never matters.

The workloads follow the pages' synthetic recipe ("synthetic (deterministic,
license-free random tokens)" in the Configuration table of the official A100
results page) at the shapes of the Qwen2.5 family the pages validate.

bf16 inputs are returned as their float32 values (exactly representable in
bf16) together with the raw uint16 bit patterns.  The float32 -> bf16 rounding
of a freshly drawn sample is round-to-nearest-even, done by torch's CPU cast.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np

# tensor ids used in the seed tuple
PROJS = ("q", "k", "v", "o", "gate", "up", "down")
PROJ_ID = {p: i for i, p in enumerate(PROJS)}
T_W, T_BIAS, T_A, T_B, T_X, T_DY, T_LN1, T_LN2, T_TOK, T_EMB, T_LM, T_LNF = range(12)


def rng_for(seed: int, cfg_id: int, layer: int, tensor_id: int) -> np.random.Generator:
    return np.random.default_rng([int(seed), int(cfg_id), int(layer), int(tensor_id)])


def round_to_bf16(x32: np.ndarray) -> np.ndarray:
    """Round float32 samples to bf16-representable float32 values (RNE, via torch CPU)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def bf16_bits(x_bf16_valued: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of float32 values that are exactly bf16."""
    u = np.ascontiguousarray(x_bf16_valued, dtype=np.float32).view(np.uint32)
    if np.any(u & 0xFFFF):
        raise ValueError("value is not exactly representable in bf16")
    return (u >> 16).astype(np.uint16)


def normal_bf16(rng: np.random.Generator, shape, std: float, mean: float = 0.0) -> np.ndarray:
    return round_to_bf16((mean + std * rng.standard_normal(shape)).astype(np.float32))


def uniform_f32(rng: np.random.Generator, shape, bound: float) -> np.ndarray:
    return rng.uniform(-bound, bound, size=shape).astype(np.float32)


def normal_f32(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    return (std * rng.standard_normal(shape)).astype(np.float32)


@dataclasses.dataclass(frozen=True)
class BlockShape:
    """Qwen2.5-family decoder block geometry."""

    hidden: int
    heads: int
    kv_heads: int
    head_dim: int
    inter: int
    layers: int = 1
    vocab: int = 152064

    def proj_shape(self, proj: str):
        """(K = in_features, N = out_features) of one projection."""
        h, q, kv = self.hidden, self.heads * self.head_dim, self.kv_heads * self.head_dim
        return {
            "q": (h, q), "k": (h, kv), "v": (h, kv), "o": (q, h),
            "gate": (h, self.inter), "up": (h, self.inter), "down": (self.inter, h),
        }[proj]


# Qwen2.5 shapes named by the pages' validated family (0.5B, 7B, 32B, 72B)
QWEN25_05B = BlockShape(hidden=896, heads=14, kv_heads=2, head_dim=64, inter=4864, layers=24)
QWEN25_7B = BlockShape(hidden=3584, heads=28, kv_heads=4, head_dim=128, inter=18944, layers=28)
QWEN25_32B = BlockShape(hidden=5120, heads=40, kv_heads=8, head_dim=128, inter=27648, layers=64)
QWEN25_72B = BlockShape(hidden=8192, heads=64, kv_heads=8, head_dim=128, inter=29568, layers=80)
# a tiny block for finite differences and fast CPU tests
TINY = BlockShape(hidden=64, heads=2, kv_heads=1, head_dim=32, inter=128, layers=2, vocab=97)


@dataclasses.dataclass(frozen=True)
class LoraSpec:
    r: int = 16
    alpha: float = 32.0
    p_drop: float = 0.0


def linear_inputs(seed: int, cfg_id: int, layer: int, proj: str, K: int, N: int, T: int,
                  lora: LoraSpec, w_std: float = 0.02, with_bias: bool = False,
                  x_std: float = 1.0) -> Dict[str, np.ndarray]:
    """One NF4 + LoRA linear: W bf16 [N,K] ~N(0,w_std), A f32 [r,K] ~U(+-1/sqrt(K)),
    B f32 [N,r] ~N(0,0.01), x bf16 [T,K] ~N(0,x_std), dy bf16 [T,N] ~N(0,1), optional
    bias bf16 [N] ~N(0,0.02)."""
    pid = PROJ_ID[proj]
    base = 16 * pid
    out = {
        "W": normal_bf16(rng_for(seed, cfg_id, layer, base + T_W), (N, K), w_std),
        "A": uniform_f32(rng_for(seed, cfg_id, layer, base + T_A), (lora.r, K), 1.0 / np.sqrt(K)),
        "B": normal_f32(rng_for(seed, cfg_id, layer, base + T_B), (N, lora.r), 0.01),
        "x": normal_bf16(rng_for(seed, cfg_id, layer, base + T_X), (T, K), x_std),
        "dy": normal_bf16(rng_for(seed, cfg_id, layer, base + T_DY), (T, N), 1.0),
    }
    out["bias"] = (normal_bf16(rng_for(seed, cfg_id, layer, base + T_BIAS), (N,), 0.02)
                   if with_bias else None)
    return out


def cfg1_inputs(seed: int = 0) -> Dict[str, np.ndarray]:
    """Single 896x896 NF4 linear + LoRA r=16 alpha=32, 512 tokens, dropout 0.0."""
    return linear_inputs(seed, 1, 0, "q", 896, 896, 512, LoraSpec(16, 32.0, 0.0))


def block_params(seed: int, cfg_id: int, layer: int, shape: BlockShape, lora: LoraSpec,
                 w_std: float = 0.02) -> Dict[str, object]:
    """Weights of one decoder block: 7 projections (W, A, B, bias on q/k/v), two
    RMSNorm weights ~1+N(0,0.02)."""
    p: Dict[str, object] = {}
    for proj in PROJS:
        K, N = shape.proj_shape(proj)
        pid = PROJ_ID[proj]
        base = 16 * pid
        p[proj] = {
            "W": normal_bf16(rng_for(seed, cfg_id, layer, base + T_W), (N, K), w_std),
            "A": uniform_f32(rng_for(seed, cfg_id, layer, base + T_A), (lora.r, K), 1.0 / np.sqrt(K)),
            "B": normal_f32(rng_for(seed, cfg_id, layer, base + T_B), (N, lora.r), 0.01),
            "bias": (normal_bf16(rng_for(seed, cfg_id, layer, base + T_BIAS), (N,), 0.02)
                     if proj in ("q", "k", "v") else None),
        }
    p["ln1"] = normal_bf16(rng_for(seed, cfg_id, layer, 200 + T_LN1), (shape.hidden,), 0.02, 1.0)
    p["ln2"] = normal_bf16(rng_for(seed, cfg_id, layer, 200 + T_LN2), (shape.hidden,), 0.02, 1.0)
    return p


def block_io(seed: int, cfg_id: int, shape: BlockShape, T: int) -> Dict[str, np.ndarray]:
    """Block input (random token embeddings, bf16 ~N(0,1)) and output cotangent."""
    return {
        "x": normal_bf16(rng_for(seed, cfg_id, 9999, T_X), (T, shape.hidden), 1.0),
        "dy": normal_bf16(rng_for(seed, cfg_id, 9999, T_DY), (T, shape.hidden), 1.0),
    }


def stack_globals(seed: int, cfg_id: int, shape: BlockShape, T: int, step: int = 0
                  ) -> Dict[str, np.ndarray]:
    """Frozen embedding / lm_head (bf16 ~N(0,0.02)), final norm and one step's tokens."""
    return {
        "emb": normal_bf16(rng_for(seed, cfg_id, 10000, T_EMB), (shape.vocab, shape.hidden), 0.02),
        "lm": normal_bf16(rng_for(seed, cfg_id, 10000, T_LM), (shape.vocab, shape.hidden), 0.02),
        "lnf": normal_bf16(rng_for(seed, cfg_id, 10000, T_LNF), (shape.hidden,), 0.02, 1.0),
    }


def tokens(seed: int, cfg_id: int, step: int, T: int, vocab: int) -> np.ndarray:
    """Random tokens, uniform over the vocabulary, for one step."""
    return rng_for(seed, cfg_id, 20000 + step, T_TOK).integers(0, vocab, size=T, dtype=np.int64)


def seed_int(seed: int, cfg_id: int, layer: int, tensor_id: int) -> int:
    """A 63-bit integer seed for device-side generators, derived from the same tuple."""
    return int(rng_for(seed, cfg_id, layer, tensor_id).integers(0, 2**63 - 1))


def device_normal_bf16(seed: int, cfg_id: int, layer: int, tensor_id: int, shape, std: float, device):
    """A large bf16 ~N(0, std) tensor drawn on the device by a torch generator seeded from
    the same tuple (for matrices too large to draw on the host quickly, such as the 72B
    projections).  The values are plain torch draws rounded to bf16; a test copies back the
    rows or columns it needs."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed_int(seed, cfg_id, layer, tensor_id))
    return (torch.randn(*shape, generator=g, device=device) * std).to(torch.bfloat16)
