"""GPU parity of the fused NF4 + LoRA linear (nf4_lora_fwd / nf4_lora_bwd) against the
oracle, on both the tiled path and the small-tile path (the `path` parameter; "small"
holds r <= 32 with r % 4 == 0).  Bar: max |gpu - ref| <= 2e-2 * RMS(ref) per tensor (fp32 accumulation
on the GPU, float64 in the oracle); exact-integer inputs must match bit for bit."""
import numpy as np
import pytest
import torch

import msq_inputs as mi
from oracle import lora as olora
from oracle import nf4 as onf4

from gpu_util import assert_parity, bf16_bits, dev_bf16, dev_f32, host_f64

pytestmark = pytest.mark.gpu
msq = pytest.importorskip("memory_streamed_qlora_amd")


def _quant(W):
    codes, a = onf4.quantize(W)
    return codes, a


PATHS = ["tiled", "small"]


def _run(inp, codes, a, r, alpha, p, key, bias=None, u_given=True, path="auto"):
    x = dev_bf16(inp["x"])
    dy = dev_bf16(inp["dy"])
    c_d = torch.from_numpy(codes).cuda()
    a_d = dev_f32(a)
    A = dev_f32(inp["A"][:r])
    B = dev_f32(inp["B"][:, :r])
    b = dev_bf16(bias) if bias is not None else None
    cfg = msq.Lora(r, alpha, p)
    k = msq.rng_key(key.seed, key.step, key.micro, key.layer, key.proj)
    y, u = msq.nf4_lora_fwd(x, c_d, a_d, b, A, B, cfg, k, path=path)
    dx, dA, dB = msq.nf4_lora_bwd(dy, x, c_d, a_d, A, B, cfg, k, u=u if u_given else None, path=path)
    torch.cuda.synchronize()
    return y, u, dx, dA, dB


def _check_against_oracle(inp, r=16, alpha=32.0, p=0.0, key=olora.RngKey(), bias=None, u_given=True,
                          name="", path="auto"):
    codes, a = _quant(inp["W"])
    name = f"{name} [{path}]"
    y, u, dx, dA, dB = _run(inp, codes, a, r, alpha, p, key, bias, u_given, path)
    Ar, Br = inp["A"][:r], inp["B"][:, :r]
    ry, ru = olora.fwd(inp["x"], codes, a, bias, Ar, Br, alpha, p, key)
    rdx, rdA, rdB = olora.bwd(inp["dy"], inp["x"], codes, a, Ar, Br, alpha, p, key)
    out = {"y": assert_parity(host_f64(y), ry, name=name + " y"),
           "dx": assert_parity(host_f64(dx), rdx, name=name + " dx")}
    if r > 0:
        out["u"] = assert_parity(host_f64(u), ru, name=name + " u")
        out["dA"] = assert_parity(host_f64(dA), rdA, name=name + " dA")
        out["dB"] = assert_parity(host_f64(dB), rdB, name=name + " dB")
    print(name, {k: f"{v:.2e}" for k, v in out.items()}, flush=True)
    return y, u, dx, dA, dB


@pytest.mark.parametrize("path", PATHS)
def test_cfg1_single_linear(path):
    """896x896 NF4 linear + LoRA r16 alpha32, 512 tokens, dropout 0.0."""
    _check_against_oracle(mi.cfg1_inputs(), name="cfg1", path=path)


@pytest.mark.parametrize("path", PATHS)
def test_ragged_tokens_dropout_bias_several_tiles(path):
    lo = mi.LoraSpec(16, 32.0, 0.1)
    inp = mi.linear_inputs(1, 2, 3, "q", 384, 640, 300, lo, with_bias=True)
    _check_against_oracle(inp, p=0.1, key=olora.RngKey(seed=7, step=3, layer=2, proj=0),
                          bias=inp["bias"], name="ragged+dropout", path=path)
    # u recomputed inside the backward
    _check_against_oracle(inp, p=0.1, key=olora.RngKey(seed=7, step=3, layer=2, proj=0),
                          bias=inp["bias"], u_given=False, name="recompute-u", path=path)


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("T,K,N,r", [(1, 64, 64, 1), (7, 128, 192, 8), (129, 256, 64, 33),
                                     (64, 4864, 896, 64), (1000, 896, 128, 32), (65, 4864, 896, 16)])
def test_odd_shapes(T, K, N, r, path):
    if path == "small" and (r > 32 or r % 4):
        pytest.skip("the small-tile path holds r <= 32 with r % 4 == 0")
    lo = mi.LoraSpec(r, 16.0, 0.2)
    inp = mi.linear_inputs(3, 2, T, "down", K, N, T, lo)
    _check_against_oracle(inp, r=r, alpha=16.0, p=0.2, key=olora.RngKey(seed=1, layer=5, proj=6),
                          name=f"T{T} K{K} N{N} r{r}", path=path)


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_fp32_activations(out_dtype, path):
    """fp32 x and dy (not bf16-representable): the base product sees bf16(x) on MFMA,
    the LoRA products the fp32 values; outputs in fp32 or bf16."""
    rng = np.random.default_rng(21)
    T, K, N, r, p = 300, 512, 384, 16, 0.1
    inp = mi.linear_inputs(2, 2, 7, "gate", K, N, T, mi.LoraSpec(r, 32.0, p), with_bias=True)
    x = rng.standard_normal((T, K)).astype(np.float32)
    dy = rng.standard_normal((T, N)).astype(np.float32)
    codes, a = _quant(inp["W"])
    key = olora.RngKey(seed=3, step=2, layer=1, proj=4)
    c_d, a_d = torch.from_numpy(codes).cuda(), dev_f32(a)
    A, B, b = dev_f32(inp["A"]), dev_f32(inp["B"]), dev_bf16(inp["bias"])
    cfg, k = msq.Lora(r, 32.0, p), msq.rng_key(3, 2, 0, 1, 4)
    y, u = msq.nf4_lora_fwd(dev_f32(x), c_d, a_d, b, A, B, cfg, k, out_dtype=out_dtype, path=path)
    dx, dA, dB = msq.nf4_lora_bwd(dev_f32(dy), dev_f32(x), c_d, a_d, A, B, cfg, k, u=u, out_dtype=out_dtype,
                                  path=path)
    torch.cuda.synchronize()
    assert y.dtype == out_dtype and dx.dtype == out_dtype
    ry, ru = olora.fwd(x, codes, a, inp["bias"], inp["A"], inp["B"], 32.0, p, key)
    rdx, rdA, rdB = olora.bwd(dy, x, codes, a, inp["A"], inp["B"], 32.0, p, key)
    r_ = {n_: assert_parity(host_f64(g), rf, name=n_) for n_, g, rf in
          (("y", y, ry), ("u", u, ru), ("dx", dx, rdx), ("dA", dA, rdA), ("dB", dB, rdB))}
    print("fp32 activations", out_dtype, path, {k_: f"{v:.2e}" for k_, v in r_.items()}, flush=True)
    # the LoRA path sees the fp32 values: u is far more accurate than a bf16 input allows
    assert r_["u"] < 1e-4


@pytest.mark.parametrize("path", PATHS)
def test_b_zero_equals_base_only_call(path):
    inp = mi.cfg1_inputs()
    inp = dict(inp, B=np.zeros_like(inp["B"]))
    codes, a = _quant(inp["W"])
    y0, *_ = _run(inp, codes, a, 16, 32.0, 0.1, olora.RngKey(seed=2), path=path)
    yb, *_ = _run(inp, codes, a, 0, 32.0, 0.1, olora.RngKey(seed=2), path=path)
    assert torch.equal(y0, yb)
    ref, _ = olora.fwd(inp["x"], codes, a, None, inp["A"][:0], inp["B"][:, :0], 32.0, 0.0, olora.RngKey())
    assert_parity(host_f64(yb), ref, name="base")


@pytest.mark.parametrize("path", PATHS)
def test_zero_weight_isolates_lora(path):
    inp = mi.cfg1_inputs()
    inp = dict(inp, W=np.zeros_like(inp["W"]), B=inp["B"] * 10)
    _check_against_oracle(inp, p=0.1, key=olora.RngKey(seed=4, layer=1, proj=2), name="W=0", path=path)


@pytest.mark.parametrize("path", PATHS)
def test_exact_integer_case_bitwise(path):
    """W in {-1,0,1}*2^e per block, integer x, A, B, dy: every sum is exact in fp32, so
    the GPU must equal the (exact) oracle after one rounding to bf16 (y, dx) or exactly
    (u, dA, dB)."""
    rng = np.random.default_rng(9)
    T, K, N, r = 160, 256, 192, 16
    e = rng.integers(-3, 3, size=(N, K // 64))
    sgn = rng.integers(-1, 2, size=(N, K)).astype(np.float32)
    sgn[:, ::64] = 1.0
    W = (sgn * np.repeat(2.0 ** e, 64, axis=1)).astype(np.float32)
    inp = {"W": W,
           "x": rng.integers(-4, 5, size=(T, K)).astype(np.float32),
           "A": rng.integers(-2, 3, size=(r, K)).astype(np.float32),
           "B": rng.integers(-2, 3, size=(N, r)).astype(np.float32),
           "dy": rng.integers(-3, 4, size=(T, N)).astype(np.float32)}
    codes, a = _quant(W)
    y, u, dx, dA, dB = _run(inp, codes, a, r, 32.0, 0.0, olora.RngKey(), path=path)
    ry, ru = olora.fwd(inp["x"], codes, a, None, inp["A"], inp["B"], 32.0, 0.0, olora.RngKey())
    rdx, rdA, rdB = olora.bwd(inp["dy"], inp["x"], codes, a, inp["A"], inp["B"], 32.0, 0.0, olora.RngKey())
    assert np.array_equal(bf16_bits(y), onf4.bf16_to_bits(onf4.bf16_round(ry.astype(np.float32))))
    assert np.array_equal(bf16_bits(dx), onf4.bf16_to_bits(onf4.bf16_round(rdx.astype(np.float32))))
    assert np.array_equal(u.cpu().numpy().astype(np.float64), ru)
    assert np.array_equal(dA.cpu().numpy().astype(np.float64), rdA)
    assert np.array_equal(dB.cpu().numpy().astype(np.float64), rdB)


@pytest.mark.parametrize("path", PATHS)
def test_zero_dropout_ignores_key_and_calls_are_deterministic(path):
    inp = mi.cfg1_inputs()
    codes, a = _quant(inp["W"])
    r1 = _run(inp, codes, a, 16, 32.0, 0.0, olora.RngKey(seed=1, layer=3), path=path)
    r2 = _run(inp, codes, a, 16, 32.0, 0.0, olora.RngKey(seed=99, step=5, proj=4), path=path)
    r3 = _run(inp, codes, a, 16, 32.0, 0.0, olora.RngKey(seed=1, layer=3), path=path)
    for u, v, w in zip(r1, r2, r3):
        assert torch.equal(u, v) and torch.equal(u, w)
    d1 = _run(inp, codes, a, 16, 32.0, 0.3, olora.RngKey(seed=1, layer=3), path=path)
    d2 = _run(inp, codes, a, 16, 32.0, 0.3, olora.RngKey(seed=1, layer=3), path=path)
    d3 = _run(inp, codes, a, 16, 32.0, 0.3, olora.RngKey(seed=1, layer=4), path=path)
    for u, v in zip(d1, d2):
        assert torch.equal(u, v)
    assert not torch.equal(d1[0], d3[0])


@pytest.mark.parametrize("path", PATHS)
def test_accumulate_flags(path):
    inp = mi.linear_inputs(5, 2, 0, "up", 256, 320, 96, mi.LoraSpec(16, 32.0, 0.0))
    codes, a = _quant(inp["W"])
    x, dy = dev_bf16(inp["x"]), dev_bf16(inp["dy"])
    c_d, a_d, A, B = torch.from_numpy(codes).cuda(), dev_f32(a), dev_f32(inp["A"]), dev_f32(inp["B"])
    cfg, key = msq.Lora(16, 32.0, 0.0), msq.rng_key()
    dx1, dA1, dB1 = msq.nf4_lora_bwd(dy, x, c_d, a_d, A, B, cfg, key, path=path)
    dx = torch.zeros_like(dx1)
    dA, dB = dA1.clone(), dB1.clone()
    msq.nf4_lora_bwd(dy, x, c_d, a_d, A, B, cfg, key, dx=dx, dx_accumulate=True, dA=dA, dB=dB,
                     dAB_accumulate=True, path=path)
    torch.cuda.synchronize()
    assert torch.equal(dA, dA1 + dA1) and torch.equal(dB, dB1 + dB1)
    assert torch.equal(dx, dx1)                       # 0 + v rounds like v
    dx2 = dx1.clone()
    msq.nf4_lora_bwd(dy, x, c_d, a_d, A, B, cfg, key, dx=dx2, dx_accumulate=True, dA=dA, dB=dB, path=path)
    torch.cuda.synchronize()
    two = 2.0 * dx1.float()
    assert torch.max(torch.abs(dx2.float() - two)).item() <= 2.0 ** -7 * torch.max(torch.abs(two)).item()


@pytest.mark.parametrize("path", PATHS)
def test_empty_tokens(path):
    inp = mi.linear_inputs(5, 2, 0, "up", 128, 128, 4, mi.LoraSpec(16, 32.0, 0.0))
    codes, a = _quant(inp["W"])
    x = torch.empty((0, 128), dtype=torch.bfloat16, device="cuda")
    dy = torch.empty((0, 128), dtype=torch.bfloat16, device="cuda")
    c_d, a_d, A, B = torch.from_numpy(codes).cuda(), dev_f32(a), dev_f32(inp["A"]), dev_f32(inp["B"])
    y, u = msq.nf4_lora_fwd(x, c_d, a_d, None, A, B, msq.Lora(16, 32.0, 0.0), msq.rng_key(), path=path)
    dA = torch.full((16, 128), 5.0, device="cuda")
    dB = torch.full((128, 16), 5.0, device="cuda")
    dx, dA, dB = msq.nf4_lora_bwd(dy, x, c_d, a_d, A, B, msq.Lora(16, 32.0, 0.0), msq.rng_key(), dA=dA, dB=dB,
                                  path=path)
    torch.cuda.synchronize()
    assert y.shape == (0, 128) and dx.shape == (0, 128)
    assert torch.all(dA == 0) and torch.all(dB == 0)


QWEN32B = mi.QWEN25_32B


@pytest.mark.parametrize("proj", ["q", "k", "gate", "down"])
def test_qwen32b_projection_shapes(proj):
    """One projection of a Qwen2.5-32B-shaped layer at 512 tokens, as the stack runs it."""
    K, N = QWEN32B.proj_shape(proj)
    inp = mi.linear_inputs(0, 4, 0, proj, K, N, 512, mi.LoraSpec(16, 32.0, 0.0),
                           with_bias=proj in ("q", "k"))
    print(f"32B {proj}: K={K} N={N}", flush=True)
    _check_against_oracle(inp, key=olora.RngKey(layer=0, proj=msq.ops.PROJ_ID[proj]),
                          bias=inp["bias"], name=f"32B-{proj}")
