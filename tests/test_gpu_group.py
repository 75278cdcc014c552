"""Grouped forward (lora_fwd_group): q/k/v or gate/up of one input in one pass.

  * against the oracle: every projection's y and u within the parity bar, with dropout
    (each projection its own mask) and bias;
  * where the group's split plan and a single call's coincide (no split), each projection's
    output is bit for bit the single nf4_lora_fwd / bf16_lora_fwd output;
  * at the 32B q/k/v and gate/up shapes, against single calls within the fp32
    summation-order noise of the different split plans."""
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
                                    out_dtype=out_dtype, residual=pr["residual"])
        else:
            y, u = msq.bf16_lora_fwd(x, pr["base"][0], pr["bias"], pr["A"], pr["B"], cfg, pr["key"],
                                     out_dtype=out_dtype, residual=pr["residual"])
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
        y, u = msq.nf4_lora_fwd(x, pr["base"][0], pr["base"][1], None, pr["A"], pr["B"], cfg, pr["key"])
        torch.cuda.synchronize()
        assert torch.equal(outs[i][1], u)
        d = (outs[i][0] - y).abs().max().item()
        rms = y.pow(2).mean().sqrt().item()
        print(f"[group 32B] {name} projection {i}: max|group - single| = {d:.3e} = {d / rms:.2e} RMS", flush=True)
        assert d <= 1e-5 * rms
