"""The small-tile path of the fused linear (one launch per forward, the input gradient and
du in one launch per backward, then the column gradients), beyond the cases
test_gpu_linear.py runs on both paths:

  * the Qwen2.5-0.5B block's projections (q/o 896 x 896, k/v 896 -> 128, gate/up
    896 -> 4864, down 4864 -> 896) at 512 tokens, dropout 0.1, fp32 activations as the
    stack passes them, forward and backward against the oracle, u passed and recomputed;
  * a 32B-shaped projection (5120 -> 1024) forced onto the small tiles: 80 k-steps over
    the four waves of a workgroup;
  * the dropout mask bit for bit: with A = [I | 0] (r = 32, K = 64) and B = 0,
    u = fp32(x * sigma) where the oracle keeps and 0 where it drops; with W = 0, B = I and
    alpha = r, dx = sigma * keep (.) dy;
  * a bf16 base equal to the dequantized NF4 base gives the NF4 call's bits;
  * small and tiled paths within fp32 summation-order noise of each other.
Bar: max |gpu - ref| <= 2e-2 * RMS(ref) per tensor."""
import numpy as np
import pytest
import torch

import msq_inputs as mi
from oracle import lora as olora
from oracle import nf4 as onf4
from oracle import philox as ophilox

from gpu_util import assert_parity, dev_bf16, dev_f32, host_f64

pytestmark = pytest.mark.gpu
msq = pytest.importorskip("memory_streamed_qlora_amd")

QWEN05B = {"q": (896, 896), "k": (896, 128), "gate": (896, 4864), "down": (4864, 896)}


def _case(seed, K, N, T, r, p, f32):
    inp = mi.linear_inputs(seed, 2, 0, "q", K, N, T, mi.LoraSpec(r, 32.0, p), with_bias=True)
    if f32:
        rng = np.random.default_rng(seed + 100)
        inp["x"] = rng.standard_normal((T, K)).astype(np.float32)
        inp["dy"] = rng.standard_normal((T, N)).astype(np.float32)
    codes, a = onf4.quantize(inp["W"])
    return inp, codes, a


def _dev(inp, f32):
    return dev_f32(inp["x"]) if f32 else dev_bf16(inp["x"]), dev_f32(inp["dy"]) if f32 else dev_bf16(inp["dy"])


@pytest.mark.parametrize("proj", list(QWEN05B))
@pytest.mark.parametrize("f32", [True, False], ids=["fp32", "bf16"])
def test_qwen05b_projections_vs_oracle(proj, f32):
    K, N = QWEN05B[proj]
    T, r, p = 512, 16, 0.1
    print(f"[small] 0.5B {proj}: K={K} N={N} {'fp32' if f32 else 'bf16'}", flush=True)
    inp, codes, a = _case(31, K, N, T, r, p, f32)
    key = olora.RngKey(seed=3, step=1, layer=2, proj=msq.ops.PROJ_ID[proj])
    dk = msq.rng_key(key.seed, key.step, key.micro, key.layer, key.proj)
    x, dy = _dev(inp, f32)
    c_d, a_d = torch.from_numpy(codes).cuda(), dev_f32(a)
    A, B, b = dev_f32(inp["A"]), dev_f32(inp["B"]), dev_bf16(inp["bias"])
    cfg = msq.Lora(r, 32.0, p)
    y, u = msq.nf4_lora_fwd(x, c_d, a_d, b, A, B, cfg, dk, out_dtype=torch.float32, path="small")
    dx, dA, dB = msq.nf4_lora_bwd(dy, x, c_d, a_d, A, B, cfg, dk, u=u, out_dtype=torch.float32, path="small")
    dx2, dA2, dB2 = msq.nf4_lora_bwd(dy, x, c_d, a_d, A, B, cfg, dk, out_dtype=torch.float32, path="small")
    torch.cuda.synchronize()
    ry, ru = olora.fwd(inp["x"], codes, a, inp["bias"], inp["A"], inp["B"], 32.0, p, key)
    rdx, rdA, rdB = olora.bwd(inp["dy"], inp["x"], codes, a, inp["A"], inp["B"], 32.0, p, key)
    for nm, g, rf in (("y", y, ry), ("u", u, ru), ("dx", dx, rdx), ("dA", dA, rdA), ("dB", dB, rdB)):
        assert_parity(host_f64(g), rf, name=f"{proj} {nm}")
    # u recomputed inside the backward by the same kernel: the same bits
    for g, h in ((dx, dx2), (dA, dA2), (dB, dB2)):
        assert torch.equal(g.view(torch.int32), h.view(torch.int32))


def test_32b_projection_forced_small():
    K, N, T, r, p = 5120, 1024, 512, 16, 0.0
    print(f"[small] 32B k projection forced small: K={K} N={N}", flush=True)
    inp, codes, a = _case(37, K, N, T, r, p, False)
    key = olora.RngKey(seed=1, layer=4, proj=1)
    dk = msq.rng_key(key.seed, key.step, key.micro, key.layer, key.proj)
    x, dy = _dev(inp, False)
    c_d, a_d = torch.from_numpy(codes).cuda(), dev_f32(a)
    A, B, b = dev_f32(inp["A"]), dev_f32(inp["B"]), dev_bf16(inp["bias"])
    cfg = msq.Lora(r, 32.0, p)
    y, u = msq.nf4_lora_fwd(x, c_d, a_d, b, A, B, cfg, dk, path="small")
    dx, dA, dB = msq.nf4_lora_bwd(dy, x, c_d, a_d, A, B, cfg, dk, u=u, path="small")
    torch.cuda.synchronize()
    ry, ru = olora.fwd(inp["x"], codes, a, inp["bias"], inp["A"], inp["B"], 32.0, p, key)
    rdx, rdA, rdB = olora.bwd(inp["dy"], inp["x"], codes, a, inp["A"], inp["B"], 32.0, p, key)
    for nm, g, rf in (("y", y, ry), ("u", u, ru), ("dx", dx, rdx), ("dA", dA, rdA), ("dB", dB, rdB)):
        assert_parity(host_f64(g), rf, name=f"32B-k {nm}")


@pytest.mark.parametrize("p", [0.1, 0.5])
def test_dropout_mask_bit_exact(p):
    T, K, r = 300, 64, 32
    print(f"[small] mask p={p}", flush=True)
    rng = np.random.default_rng(int(p * 10) + 5)
    x = mi.normal_bf16(rng, (T, K), 1.0)
    key = olora.RngKey(seed=77, step=3, layer=9, proj=5)
    dk = msq.rng_key(key.seed, key.step, key.micro, key.layer, key.proj)
    cfg = msq.Lora(r, float(r), p)  # alpha = r: s = 1
    zero = msq.nf4_quantize(torch.zeros(64, K, dtype=torch.bfloat16, device="cuda"))
    eye = torch.zeros(r, K, device="cuda")
    eye[:, :r] = torch.eye(r, device="cuda")
    xd = dev_bf16(x)
    _, u = msq.nf4_lora_fwd(xd, zero[0], zero[1], None, eye, torch.zeros(64, r, device="cuda"), cfg, dk,
                            path="small")
    keep = ophilox.keep_mask(T, K, p, key.seed, key.layer, key.proj, key.step, key.micro)
    sigma = np.float32(1.0) / np.float32(1.0 - np.float32(p))
    want = np.where(keep[:, :r], x[:, :r].astype(np.float32) * sigma, np.float32(0.0)).astype(np.float32)
    torch.cuda.synchronize()
    assert np.array_equal(u.cpu().numpy().view(np.int32), want.view(np.int32))
    # backward: W = 0, B = [I; 0] (n = 64 rows, the first r of them I), alpha = r:
    # du = dy[:, :r], dx = keep * sigma * (du A) = keep * sigma * [dy[:, :r] | 0]
    Bm = torch.zeros(64, r, device="cuda")
    Bm[:r] = torch.eye(r, device="cuda")
    dy = mi.normal_bf16(rng, (T, 64), 1.0)
    dx, _, _ = msq.nf4_lora_bwd(dev_bf16(dy), xd, zero[0], zero[1], eye, Bm, cfg, dk, out_dtype=torch.float32,
                                path="small")
    torch.cuda.synchronize()
    wdx = np.zeros((T, K), dtype=np.float32)
    wdx[:, :r] = np.where(keep[:, :r], sigma * dy[:, :r].astype(np.float32), np.float32(0.0))
    assert np.array_equal(dx.cpu().numpy().view(np.int32), wdx.view(np.int32))


@pytest.mark.parametrize("K,N,T", [(896, 896, 512), (4864, 896, 77), (896, 4864, 1000)])
def test_bf16_base_equals_nf4_on_dequantized_weights(K, N, T):
    g = torch.Generator(device="cuda").manual_seed(K + N + T)
    W = (torch.randn(N, K, generator=g, device="cuda") * 0.02).to(torch.bfloat16)
    codes, absmax = msq.nf4_quantize(W)
    Wd = msq.nf4_dequantize(codes, absmax)
    x = torch.randn(T, K, generator=g, device="cuda")
    dy = torch.randn(T, N, generator=g, device="cuda")
    A = (torch.rand(16, K, generator=g, device="cuda") * 2 - 1) / K ** 0.5
    B = torch.randn(N, 16, generator=g, device="cuda") * 0.01
    cfg, key = msq.Lora(16, 32.0, 0.1), msq.rng_key(1, 2, 0, 3, 4)
    y4, u4 = msq.nf4_lora_fwd(x, codes, absmax, None, A, B, cfg, key, path="small")
    yb, ub = msq.bf16_lora_fwd(x, Wd, None, A, B, cfg, key, path="small")
    dx4, dA4, dB4 = msq.nf4_lora_bwd(dy, x, codes, absmax, A, B, cfg, key, u=u4, path="small")
    dxb, dAb, dBb = msq.bf16_lora_bwd(dy, x, Wd, A, B, cfg, key, u=ub, path="small")
    torch.cuda.synchronize()
    for a_, b_, nm in ((y4, yb, "y"), (u4, ub, "u"), (dx4, dxb, "dx"), (dA4, dAb, "dA"), (dB4, dBb, "dB")):
        assert torch.equal(a_.view(torch.int32), b_.view(torch.int32)), f"{nm} differs"


@pytest.mark.parametrize("K,N,T", [(896, 896, 512), (896, 128, 300), (4864, 896, 512)])
def test_small_and_tiled_paths_agree(K, N, T):
    g = torch.Generator(device="cuda").manual_seed(K * 3 + N + T)
    W = (torch.randn(N, K, generator=g, device="cuda") * 0.02).to(torch.bfloat16)
    codes, absmax = msq.nf4_quantize(W)
    x = torch.randn(T, K, generator=g, device="cuda")
    dy = torch.randn(T, N, generator=g, device="cuda")
    A = (torch.rand(16, K, generator=g, device="cuda") * 2 - 1) / K ** 0.5
    B = torch.randn(N, 16, generator=g, device="cuda") * 0.01
    bias = (torch.randn(N, generator=g, device="cuda") * 0.02).to(torch.bfloat16)
    cfg, key = msq.Lora(16, 32.0, 0.1), msq.rng_key(2, 1, 0, 1, 3)
    outs = {}
    for path in ("tiled", "small"):
        y, u = msq.nf4_lora_fwd(x, codes, absmax, bias, A, B, cfg, key, out_dtype=torch.float32, path=path)
        dx, dA, dB = msq.nf4_lora_bwd(dy, x, codes, absmax, A, B, cfg, key, u=u, out_dtype=torch.float32, path=path)
        outs[path] = (y, u, dx, dA, dB)
    torch.cuda.synchronize()
    for nm, a_, b_ in zip(("y", "u", "dx", "dA", "dB"), outs["tiled"], outs["small"]):
        d = (a_ - b_).abs().max().item()
        rms = a_.pow(2).mean().sqrt().item()
        print(f"[small vs tiled] K={K} N={N} T={T} {nm}: {d / rms:.2e} RMS", flush=True)
        assert d <= 1e-4 * rms, nm
