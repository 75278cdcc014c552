"""NF4 codebook, blockwise quantization and dequantization (oracle).

The pages name the frozen base's format -- NF4 through bitsandbytes
("Limitations", "What 0.00e+00 means": NF4-only parity; Official A100
results, "Configuration": precision NF4) -- and state that the base is 4-bit
and read-only ("Poros" research post, opening paragraphs: roughly 18 GB of NF4
weights at 32B).  They give no codebook, block size, scale dtype or rounding
rule.  Readings taken here:

  * codebook: the NormalFloat construction of the QLoRA paper (Dettmers et al.
    2023, section 3, "4-bit NormalFloat"): 8 positive and 7 negative normal
    quantiles sharing one exact zero, normalised to [-1, 1], with upper
    probability cut delta = 1 - (1/32 + 1/30)/2.  Computed in float64 and
    rounded once to float32.
  * blocks of 64 consecutive elements of the row-major [N, K] matrix, one fp32
    absmax per block, no double quantization.
  * code = nearest level of w / absmax, decided exactly (no division): the
    number of midpoints m_i = (L_i + L_{i+1}) / 2 with w > absmax * m_i.  Ties go
    to the lower code.  An all-zero block stores absmax 0 and code 7 (the zero
    level).
  * two codes per byte, the element with the even index in the high nibble.
  * dequantized value = bf16_rne(fp32(L[code] * absmax)).
"""
from __future__ import annotations

from statistics import NormalDist

import numpy as np

BLOCK = 64
DELTA = 1.0 - 0.5 * (1.0 / 32.0 + 1.0 / 30.0)
ZERO_CODE = 7


def codebook_f64() -> np.ndarray:
    """The 16 NF4 levels in float64, ascending (QLoRA section 3 construction)."""
    inv = NormalDist().inv_cdf
    top = inv(DELTA)
    pos = [inv(0.5 + j * (DELTA - 0.5) / 8.0) / top for j in range(1, 9)]
    neg = [-inv(0.5 + j * (DELTA - 0.5) / 7.0) / top for j in range(1, 8)]
    levels = sorted(neg + [0.0] + pos)
    return np.array(levels, dtype=np.float64)


def codebook() -> np.ndarray:
    """The 16 NF4 levels rounded once to float32."""
    return codebook_f64().astype(np.float32)


def midpoints() -> np.ndarray:
    """m_i = (L_i + L_{i+1}) / 2 in float64; exact because the L_i are fp32."""
    L = codebook().astype(np.float64)
    return (L[:-1] + L[1:]) / 2.0


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 (round to nearest, ties to even), returned as float32 values.

    Uses torch's CPU cast, a library primitive implementing IEEE RNE."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def bf16_to_bits(x: np.ndarray) -> np.ndarray:
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    assert not np.any(u & 0xFFFF), "not a bf16 value"
    return (u >> 16).astype(np.uint16)


def bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def absmax(w: np.ndarray) -> np.ndarray:
    """Per-64-block max |w| of a row-major [N, K] matrix, float32 [N, K/64]."""
    n, k = w.shape
    assert k % BLOCK == 0
    return np.abs(w.astype(np.float32)).reshape(n, k // BLOCK, BLOCK).max(axis=2)


def quantize_codes(w: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Unpacked codes (uint8 [N, K], values 0..15) and absmax (float32 [N, K/64]).

    w holds float32 values (bf16 inputs are exact in float32).  Each decision
    is an exact float64 comparison w > a * m_i: a has 24 significant bits and
    m_i at most 29, so the product is exact in the 53-bit double."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    assert np.all(np.isfinite(w)), "quantize requires finite inputs"
    n, k = w.shape
    a = absmax(w)
    m = midpoints()
    wb = w.astype(np.float64).reshape(n, k // BLOCK, BLOCK)
    ab = a.astype(np.float64)[:, :, None]
    codes = np.zeros(wb.shape, dtype=np.uint8)
    for i in range(15):
        codes += (wb > ab * m[i]).astype(np.uint8)
    codes[a == 0.0] = ZERO_CODE
    return codes.reshape(n, k), a


def pack(codes: np.ndarray) -> np.ndarray:
    """Two codes per byte, element 2j in the high nibble: [N, K] -> [N, K/2]."""
    c = codes.astype(np.uint8)
    return ((c[:, 0::2] << 4) | c[:, 1::2]).astype(np.uint8)


def unpack(packed: np.ndarray) -> np.ndarray:
    p = packed.astype(np.uint8)
    n, kh = p.shape
    out = np.empty((n, 2 * kh), dtype=np.uint8)
    out[:, 0::2] = p >> 4
    out[:, 1::2] = p & 0xF
    return out


def quantize(w: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """NF4 quantization of a bf16-valued [N, K] matrix -> (packed codes u8 [N, K/2],
    absmax f32 [N, K/64])."""
    codes, a = quantize_codes(w)
    return pack(codes), a


def dequantize(packed: np.ndarray, a: np.ndarray) -> np.ndarray:
    """bf16_rne(fp32(L[code] * absmax)) as float32 values [N, K]."""
    codes = unpack(packed)
    n, k = codes.shape
    L = codebook()
    lv = L[codes].reshape(n, k // BLOCK, BLOCK)
    prod = (lv * a.astype(np.float32)[:, :, None]).astype(np.float32)  # one IEEE fp32 multiply
    return bf16_round(prod.reshape(n, k))
