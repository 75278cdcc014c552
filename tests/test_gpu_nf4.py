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


def _unpack_dev(codes: torch.Tensor) -> torch.Tensor:
    """[n, k/2] packed codes -> [n, k] (element 2j in the high nibble), on the device."""
    c = codes.to(torch.int32)
    return torch.stack([c >> 4, c & 15], dim=2).reshape(codes.shape[0], -1)


def test_quantize_exhaustive_over_every_bf16_pair():
    """Every pair of bf16 values (w, a) with 0 < a finite and |w| <= a (1.07e9 pairs), packed
    as blocks whose first element is a, through nf4_quantize.  For each a the oracle's code is
    a nondecreasing function of w (a count of thresholds below w), so the GPU's codes equal
    the oracle's for every w when (1) the GPU's codes are nondecreasing in w too and (2) the
    two agree at both ends and on both sides of every place where the GPU's code steps.  (1)
    and the step places are computed on the device; (2) evaluates the oracle's quantizer on
    exactly those points.  Every block's absmax must be a."""
    dev = "cuda"
    a_all = np.arange(1, 0x7F80, dtype=np.int64)               # positive finite bf16 bit patterns
    n_all = 2 * (a_all + 1)                                    # w = -a .. -0, +0 .. +a
    chunks, cur, acc = [], [], 0
    for i, n in enumerate(n_all):
        cur.append(i)
        acc += n
        if acc >= (96 << 20):
            chunks.append(np.array(cur))
            cur, acc = [], 0
    if cur:
        chunks.append(np.array(cur))
    total, points = 0, []
    for ci, idx in enumerate(chunks):
        A = torch.from_numpy(a_all[idx]).to(dev)
        n = 2 * (A + 1)
        nb = (n + 62) // 63                                   # blocks of 63 w values after a
        blk_a = torch.repeat_interleave(A, nb)
        first = torch.repeat_interleave(torch.cumsum(nb, 0) - nb, nb)
        j = torch.arange(blk_a.numel(), device=dev) - first   # block index within its a
        i = j[:, None] * 63 + torch.arange(63, device=dev)[None, :]   # w index within its a
        na = torch.repeat_interleave(n, nb)[:, None]
        half = (blk_a + 1)[:, None]
        bits = torch.where(i < half, 0x8000 | (blk_a[:, None] - i), i - half)  # -a..-0, then +0..+a
        valid = i < na
        bits = torch.where(valid, bits, torch.zeros_like(bits))
        blocks = torch.cat([blk_a[:, None], bits], 1).to(torch.int32).to(torch.int16)
        w = blocks.view(torch.bfloat16).contiguous()
        codes, absmax = msq.nf4_quantize(w)
        assert torch.equal(absmax.view(torch.int32), (blk_a.to(torch.int32) << 16).view(1, -1).t().contiguous()
                           .view(-1, 1)), f"chunk {ci}: absmax != a"
        c = _unpack_dev(codes)[:, 1:][valid]                  # each a's codes, w ascending
        seg = torch.repeat_interleave(torch.arange(idx.size, device=dev), n)
        step = c[1:] - c[:-1]
        same = seg[1:] == seg[:-1]
        assert bool(torch.all(step[same] >= 0)), f"chunk {ci}: codes not monotone in w"
        # the first index with code >= lvl, per a and level (from the counts, codes monotone)
        cnt = torch.zeros(idx.size, 16, dtype=torch.int64, device=dev)
        for lvl in range(1, 16):
            cnt[:, lvl].index_add_(0, seg, (c >= lvl).to(torch.int64))
        starts = n[:, None] - cnt[:, 1:]                      # [n_a, 15]
        # GPU code at w index q, and the points to check: both ends and both sides of every step
        pts = torch.cat([torch.zeros_like(starts[:, :1]), n[:, None] - 1,
                         (starts - 1).clamp(min=0), starts.clamp(max=(n - 1)[:, None])], 1)
        gcode = (starts[:, None, :] <= pts[:, :, None]).sum(2)
        points.append((A.cpu().numpy(), n.cpu().numpy(), pts.cpu().numpy(), gcode.cpu().numpy()))
        total += int(n.sum())
        del codes, absmax, blocks, w, c
    assert total == int(n_all.sum())
    print(f"exhaustive quantize: {total} (w, a) pairs over {a_all.size} absmax values", flush=True)
    # the oracle at the check points: one block per a: [a, w at the 32 points]
    A = np.concatenate([p[0] for p in points])
    n = np.concatenate([p[1] for p in points])
    pts = np.concatenate([p[2] for p in points])
    gcode = np.concatenate([p[3] for p in points])
    half = (A + 1)[:, None]
    wb = np.where(pts < half, 0x8000 | (A[:, None] - pts), pts - half).astype(np.uint16)
    blk = np.zeros((A.size, 64), np.uint16)
    blk[:, 0] = A
    blk[:, 1:1 + pts.shape[1]] = wb
    codes, absmax = onf4.quantize_codes(onf4.bits_to_f32(blk))
    assert np.array_equal(absmax[:, 0].view(np.uint32), (A.astype(np.uint32) << 16))
    assert np.array_equal(codes[:, 1:1 + pts.shape[1]].astype(np.int64), gcode)
