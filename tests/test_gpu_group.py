"""Grouped forward and backward (lora_fwd_group, lora_bwd_group): q/k/v or gate/up of one
input in one pass.

Forward:
  * against the oracle: every projection's y and u within the parity bar, with dropout
    (each projection its own mask) and bias;
  * where the group's split plan and a single call's coincide (no split), each projection's
    output is bit for bit the single nf4_lora_fwd / bf16_lora_fwd output;
  * at the 32B q/k/v and gate/up shapes, against single calls within the fp32
    summation-order noise of the different split plans.
Backward:
  * against the oracle: dx (the sum of the projections' input gradients) and every dA, dB
    within the parity bar, with dropout, u recomputed or passed in, both base formats;
  * every dA and dB bit for bit the single call's, dx within fp32 summation-order noise of
    the single calls' sum, accumulate flags included;
  * at the 32B q/k/v and gate/up shapes, against the single calls' sum."""
import numpy as np
import pytest
import torch

import msq_inputs as mi
from oracle import lora as olora
from oracle import nf4 as onf4

from gpu_util import assert_parity, dev_bf16, dev_f32, host_f64

pytestmark = pytest.mark.gpu
msq = pytest.importorskip("memory_streamed_qlora_amd")


def _proj_inputs(seed, K, ns, r, with_bias=True):
    out = []
    for i, n in enumerate(ns):
        inp = mi.linear_inputs(seed, 2, 1, ("q", "k", "v")[i], K, n, 8, mi.LoraSpec(r, 32.0, 0.1), with_bias=with_bias)
        out.append(inp)
    return out


@pytest.mark.parametrize("T,K,ns", [(512, 896, (896, 128, 128)), (300, 384, (640, 64)), (1, 128, (64, 64, 192))])
def test_group_vs_oracle(T, K, ns):
    print(f"[group] T={T} K={K} ns={ns}", flush=True)
    r, p, alpha = 16, 0.1, 32.0
    ins = _proj_inputs(T + K, K, ns, r)
    x = mi.normal_bf16(mi.rng_for(T, K, 0, 99), (T, K), 1.0)
    projs, refs = [], []
    for i, inp in enumerate(ins):
        codes, a = onf4.quantize(inp["W"])
        key = olora.RngKey(seed=4, step=1, layer=3, proj=i)
        projs.append({"base": (torch.from_numpy(codes).cuda(), dev_f32(a)), "bias": dev_bf16(inp["bias"]),
                      "A": dev_f32(inp["A"]), "B": dev_f32(inp["B"]), "key": msq.rng_key(4, 1, 0, 3, i)})
        refs.append(olora.fwd(x, codes, a, inp["bias"], inp["A"], inp["B"], alpha, p, key))
    outs = msq.lora_fwd_group(dev_bf16(x), projs, msq.Lora(r, alpha, p))
    torch.cuda.synchronize()
    for i, ((y, u), (ry, ru)) in enumerate(zip(outs, refs)):
        assert_parity(host_f64(y), ry, name=f"y{i}")
        assert_parity(host_f64(u), ru, name=f"u{i}")


@pytest.mark.parametrize("fmt", ["nf4", "bf16"])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_group_equals_single_calls_without_split(fmt, out_dtype):
    """K = 256 (4 k-steps): no split in either plan, so every tile does the same
    arithmetic: the group's outputs equal the single calls' bit for bit."""
    T, K, ns, r = 100, 256, (192, 64, 128), 16
    g = torch.Generator(device="cuda").manual_seed(3)
    x = torch.randn(T, K, generator=g, device="cuda")
    cfg = msq.Lora(r, 32.0, 0.1)
    projs = []
    for i, n in enumerate(ns):
        W = (torch.randn(n, K, generator=g, device="cuda") * 0.02).to(torch.bfloat16)
        base = msq.nf4_quantize(W) if fmt == "nf4" else (W,)
        projs.append({"base": base, "bias": (torch.randn(n, generator=g, device="cuda") * 0.02).to(torch.bfloat16),
                      "A": torch.randn(r, K, generator=g, device="cuda") * 0.05,
                      "B": torch.randn(n, r, generator=g, device="cuda") * 0.01,
                      "key": msq.rng_key(9, 2, 1, 5, i),
                      "residual": torch.randn(T, n, generator=g, device="cuda").to(out_dtype) if i == 1 else None})
    outs = msq.lora_fwd_group(x, projs, cfg, out_dtype=out_dtype)
    for i, pr in enumerate(projs):
        if fmt == "nf4":
            y, u = msq.nf4_lora_fwd(x, pr["base"][0], pr["base"][1], pr["bias"], pr["A"], pr["B"], cfg, pr["key"],
                                    out_dtype=out_dtype, residual=pr["residual"], path="tiled")
        else:
            y, u = msq.bf16_lora_fwd(x, pr["base"][0], pr["bias"], pr["A"], pr["B"], cfg, pr["key"],
                                     out_dtype=out_dtype, residual=pr["residual"], path="tiled")
        torch.cuda.synchronize()
        iv = torch.int16 if out_dtype == torch.bfloat16 else torch.int32
        assert torch.equal(outs[i][0].view(iv), y.view(iv)), f"projection {i}: y differs"
        assert torch.equal(outs[i][1].view(torch.int32), u.view(torch.int32)), f"projection {i}: u differs"


@pytest.mark.parametrize("name,K,ns", [("qkv", 5120, (5120, 1024, 1024)), ("gate/up", 5120, (27648, 27648))])
def test_group_at_32b_shapes(name, K, ns):
    print(f"[group 32B] {name}", flush=True)
    T, r = 512, 16
    g = torch.Generator(device="cuda").manual_seed(len(ns))
    x = torch.randn(T, K, generator=g, device="cuda")
    cfg = msq.Lora(r, 32.0, 0.0)
    projs = []
    for i, n in enumerate(ns):
        W = (torch.randn(n, K, generator=g, device="cuda") * 0.02).to(torch.bfloat16)
        projs.append({"base": msq.nf4_quantize(W), "bias": None,
                      "A": (torch.rand(r, K, generator=g, device="cuda") * 2 - 1) / K ** 0.5,
                      "B": torch.randn(n, r, generator=g, device="cuda") * 0.01, "key": msq.rng_key(1, 0, 0, 0, i)})
    outs = msq.lora_fwd_group(x, projs, cfg)
    for i, pr in enumerate(projs):
        y, u = msq.nf4_lora_fwd(x, pr["base"][0], pr["base"][1], None, pr["A"], pr["B"], cfg, pr["key"], path="tiled")
        torch.cuda.synchronize()
        assert torch.equal(outs[i][1], u)
        d = (outs[i][0] - y).abs().max().item()
        rms = y.pow(2).mean().sqrt().item()
        print(f"[group 32B] {name} projection {i}: max|group - single| = {d:.3e} = {d / rms:.2e} RMS", flush=True)
        assert d <= 1e-5 * rms


# ---- backward ---------------------------------------------------------------------------

def _bwd_case(seed, T, K, ns, r, fmt="nf4"):
    """Host inputs of a backward group: x, per projection (W as its codes/absmax or bf16),
    A, B, dy, key."""
    ins = _proj_inputs(seed, K, ns, r, with_bias=False)
    x = mi.normal_bf16(mi.rng_for(T, K, 0, 98), (T, K), 1.0)
    out = []
    for i, inp in enumerate(ins):
        dy = mi.normal_bf16(mi.rng_for(T, ns[i], i, 97), (T, ns[i]), 1.0)
        out.append(dict(inp, dy=dy, key=olora.RngKey(seed=5, step=2, layer=7, proj=i)))
    return x, out


def _dev_projs(cases, fmt, r):
    projs = []
    for i, c in enumerate(cases):
        if fmt == "nf4":
            codes, a = onf4.quantize(c["W"])
            base = (torch.from_numpy(codes).cuda(), dev_f32(a))
            W64 = onf4.dequantize(codes, a)
        else:
            base = (dev_bf16(c["W"]),)
            W64 = np.asarray(c["W"], dtype=np.float64)
        projs.append({"base": base, "A": dev_f32(c["A"]), "B": dev_f32(c["B"]), "dy": dev_bf16(c["dy"]),
                      "key": msq.rng_key(5, 2, 0, 7, i), "W64": W64})
    return projs


@pytest.mark.parametrize("T,K,ns,fmt,pass_u", [(512, 896, (896, 128, 128), "nf4", False),
                                               (300, 384, (640, 64), "nf4", True),
                                               (1, 128, (64, 64, 192), "nf4", False),
                                               (200, 256, (128, 64, 64), "bf16", True)])
def test_group_bwd_vs_oracle(T, K, ns, fmt, pass_u):
    print(f"[group bwd] T={T} K={K} ns={ns} {fmt} u={'passed' if pass_u else 'recomputed'}", flush=True)
    r, p, alpha = 16, 0.1, 32.0
    x, cases = _bwd_case(T + K + 1, T, K, ns, r)
    projs = _dev_projs(cases, fmt, r)
    dx_ref = np.zeros((T, K))
    refs = []
    for c, pr in zip(cases, projs):
        dxi, dA, dB = olora.bwd_dense(c["dy"], x, pr["W64"], c["A"], c["B"], alpha, p, c["key"])
        dx_ref += dxi
        refs.append((dA, dB))
        if pass_u:
            _, u = olora.fwd_dense(x, pr["W64"], None, c["A"], c["B"], alpha, p, c["key"])
            pr["u"] = dev_f32(u)
    dx, grads = msq.lora_bwd_group(dev_bf16(x), projs, msq.Lora(r, alpha, p), out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert_parity(host_f64(dx), dx_ref, name="dx")
    for i, ((dA, dB), (rA, rB)) in enumerate(zip(grads, refs)):
        assert_parity(host_f64(dA), rA, name=f"dA{i}")
        assert_parity(host_f64(dB), rB, name=f"dB{i}")


@pytest.mark.parametrize("fmt", ["nf4", "bf16"])
@pytest.mark.parametrize("p_drop", [0.0, 0.1])
def test_group_bwd_against_single_calls(fmt, p_drop):
    """dA, dB: the same kernels on the same inputs as a single call, so bit for bit; dx: the
    single calls' dx summed in fp32, up to summation order.  Then both accumulate flags:
    dx += the group's sum, dA / dB += their own values."""
    T, K, ns, r = 160, 320, (192, 64, 128), 16
    g = torch.Generator(device="cuda").manual_seed(7)
    x = torch.randn(T, K, generator=g, device="cuda").to(torch.bfloat16)
    cfg = msq.Lora(r, 32.0, p_drop)
    projs = []
    for i, n in enumerate(ns):
        W = (torch.randn(n, K, generator=g, device="cuda") * 0.02).to(torch.bfloat16)
        projs.append({"base": msq.nf4_quantize(W) if fmt == "nf4" else (W,),
                      "A": torch.randn(r, K, generator=g, device="cuda") * 0.05,
                      "B": torch.randn(n, r, generator=g, device="cuda") * 0.01,
                      "dy": torch.randn(T, n, generator=g, device="cuda").to(torch.bfloat16),
                      "key": msq.rng_key(3, 1, 0, 4, i)})
    dx, grads = msq.lora_bwd_group(x, projs, cfg, out_dtype=torch.float32)
    ref = torch.zeros(T, K, device="cuda")
    for pr, (dA, dB) in zip(projs, grads):
        bwd = msq.nf4_lora_bwd if fmt == "nf4" else msq.bf16_lora_bwd
        dxi, sA, sB = bwd(pr["dy"], x, *pr["base"], pr["A"], pr["B"], cfg, pr["key"], out_dtype=torch.float32,
                          path="tiled")
        torch.cuda.synchronize()
        assert torch.equal(dA.view(torch.int32), sA.view(torch.int32))
        assert torch.equal(dB.view(torch.int32), sB.view(torch.int32))
        ref += dxi
    d = (dx - ref).abs().max().item()
    rms = ref.pow(2).mean().sqrt().item()
    print(f"[group bwd] {fmt} p={p_drop}: max|group - sum of singles| = {d / rms:.2e} RMS", flush=True)
    assert d <= 1e-5 * rms
    dx0 = torch.randn(T, K, generator=g, device="cuda")
    A0 = [torch.randn_like(dA) for dA, _ in grads]
    B0 = [torch.randn_like(dB) for _, dB in grads]
    for pr, a0, b0 in zip(projs, A0, B0):
        pr["dA"], pr["dB"] = a0.clone(), b0.clone()
    dx2, grads2 = msq.lora_bwd_group(x, projs, cfg, dx=dx0.clone(), dx_accumulate=True, dAB_accumulate=True)
    torch.cuda.synchronize()
    d = (dx2 - (dx0 + dx)).abs().max().item()
    assert d <= 1e-5 * (dx0 + dx).abs().max().item()
    for (dA, dB), (gA, gB), a0, b0 in zip(grads, grads2, A0, B0):
        torch.testing.assert_close(gA, a0 + dA, rtol=1e-6, atol=1e-7)
        torch.testing.assert_close(gB, b0 + dB, rtol=1e-6, atol=1e-7)


@pytest.mark.parametrize("name,ns", [("qkv", (5120, 1024, 1024)), ("gate/up", (27648, 27648))])
def test_group_bwd_at_32b_shapes(name, ns):
    print(f"[group bwd 32B] {name}", flush=True)
    T, K, r = 512, 5120, 16
    g = torch.Generator(device="cuda").manual_seed(len(ns) + 10)
    x = torch.randn(T, K, generator=g, device="cuda").to(torch.bfloat16)
    cfg = msq.Lora(r, 32.0, 0.0)
    projs = []
    for i, n in enumerate(ns):
        W = (torch.randn(n, K, generator=g, device="cuda") * 0.02).to(torch.bfloat16)
        projs.append({"base": msq.nf4_quantize(W), "A": (torch.rand(r, K, generator=g, device="cuda") * 2 - 1) / K ** 0.5,
                      "B": torch.randn(n, r, generator=g, device="cuda") * 0.01,
                      "dy": torch.randn(T, n, generator=g, device="cuda").to(torch.bfloat16),
                      "key": msq.rng_key(1, 0, 0, 0, i)})
    dx, grads = msq.lora_bwd_group(x, projs, cfg, out_dtype=torch.float32)
    ref = torch.zeros(T, K, device="cuda")
    for pr, (dA, dB) in zip(projs, grads):
        dxi, sA, sB = msq.nf4_lora_bwd(pr["dy"], x, *pr["base"], pr["A"], pr["B"], cfg, pr["key"],
                                       out_dtype=torch.float32, path="tiled")
        torch.cuda.synchronize()
        assert torch.equal(dA, sA) and torch.equal(dB, sB)
        ref += dxi
    d = (dx - ref).abs().max().item()
    rms = ref.pow(2).mean().sqrt().item()
    print(f"[group bwd 32B] {name}: max|group - sum of singles| = {d:.3e} = {d / rms:.2e} RMS", flush=True)
    assert d <= 1e-5 * rms
