"""GPU parity of nf4_quantize / nf4_dequantize against the oracle: bit-exact."""
import numpy as np
import pytest
import torch

import msq_inputs as mi
from oracle import nf4 as onf4

from gpu_util import bf16_bits, dev_bf16, dev_u8, dev_f32

pytestmark = pytest.mark.gpu
msq = pytest.importorskip("memory_streamed_qlora_amd")


def _gpu_quant(w32):
    codes, a = msq.nf4_quantize(dev_bf16(w32))
    torch.cuda.synchronize()
    return codes.cpu().numpy(), a.cpu().numpy()


def test_quantize_cfg1_weight_bit_exact():
    w = mi.cfg1_inputs()["W"]
    c, a = _gpu_quant(w)
    oc, oa = onf4.quantize(w)
    assert np.array_equal(c, oc)
    assert np.array_equal(a.view(np.uint32), oa.view(np.uint32))


def test_quantize_bf16_domain_sweep_bit_exact():
    """Every bf16 value w with |w| <= a, for absmax values a spanning the whole
    exponent range (subnormal to large), packed in blocks whose first element is a."""
    a_bits = np.concatenate([np.arange(0x0001, 0x0080, 19), np.arange(0x0080, 0x7F80, 251),
                             np.array([0x3F80, 0x7F7F])]).astype(np.uint32)
    blocks = []
    for ab in a_bits:
        a = (np.array([ab], np.uint32) << 16).view(np.float32)[0]
        pos = (np.arange(0, ab + 1, dtype=np.uint32) << 16).view(np.float32)
        vals = np.concatenate([pos, -pos])
        n_per = 63
        nb = -(-vals.size // n_per)
        pad = np.zeros(nb * n_per, np.float32)
        pad[: vals.size] = vals
        blocks.append(np.concatenate([np.full((nb, 1), a, np.float32), pad.reshape(nb, n_per)], 1))
    w = np.concatenate(blocks, 0)
    rows = -(-w.shape[0] // 8)
    w = np.concatenate([w, np.zeros((rows * 8 - w.shape[0], 64), np.float32)]).reshape(rows, 8 * 64)
    print(f"quantize sweep: {w.size} elements, {a_bits.size} absmax values", flush=True)
    c, a = _gpu_quant(w)
    oc, oa = onf4.quantize(w)
    assert np.array_equal(a.view(np.uint32), oa.view(np.uint32))
    assert np.array_equal(c, oc)


def test_quantize_special_cases():
    w = np.zeros((4, 192), np.float32)
    rng = np.random.default_rng(0)
    w[1] = onf4.bf16_round(rng.standard_normal(192).astype(np.float32))
    w[1, 3] = 0.0
    w[1, 70] = -0.0
    w[2, :64] = 3.0
    w[2, 64:128] = -3.0
    w[3, 128] = onf4.bf16_round(np.array([1e-40], np.float32))[0]  # a subnormal absmax
    c, a = _gpu_quant(w)
    oc, oa = onf4.quantize(w)
    assert np.array_equal(c, oc) and np.array_equal(a.view(np.uint32), oa.view(np.uint32))
    cu = onf4.unpack(c)
    assert np.all(cu[0] == 7) and cu[1, 3] == 7 and cu[1, 70] == 7
    assert np.all(cu[2, :64] == 15) and np.all(cu[2, 64:128] == 0)


def test_dequant_every_code_every_bf16_absmax_bit_exact():
    a_bits = np.arange(0x0000, 0x7F80, dtype=np.uint32)
    a = (a_bits << 16).view(np.float32)
    n = a.size
    codes = onf4.pack(np.tile(np.arange(16, dtype=np.uint8), (n, 4)))
    out = msq.nf4_dequantize(dev_u8(codes), dev_f32(a.reshape(n, 1)))
    torch.cuda.synchronize()
    ref = onf4.bf16_to_bits(onf4.dequantize(codes, a.reshape(n, 1)))
    assert np.array_equal(bf16_bits(out), ref)


def test_round_trip_on_gpu_is_idempotent():
    rng = np.random.default_rng(1)
    w = onf4.bf16_round((0.02 * rng.standard_normal((256, 1024))).astype(np.float32))
    c1, a1 = msq.nf4_quantize(dev_bf16(w))
    deq = msq.nf4_dequantize(c1, a1)
    c2, a2 = msq.nf4_quantize(deq)
    torch.cuda.synchronize()
    assert torch.equal(c1, c2) and torch.equal(a1, a2)
    ref = onf4.bf16_to_bits(onf4.dequantize(c1.cpu().numpy(), a1.cpu().numpy()))
    assert np.array_equal(bf16_bits(deq), ref)


def test_empty_and_codebook():
    e = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    c, a = msq.nf4_quantize(e)
    assert c.shape == (0, 32) and a.shape == (0, 1)
    assert np.array_equal(msq.nf4_codebook().numpy().view(np.uint32), onf4.codebook().view(np.uint32))
