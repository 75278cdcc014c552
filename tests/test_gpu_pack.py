"""The packing pass over several activations in one launch (the grouped backward packs
every projection's dy together) and its rank-r products, whose column-chunk partials a
second launch sums in chunk order.

  * every call writes its products: outputs filled with NaN beforehand, calls of different
    shapes interleaved (ragged token groups, a ragged last chunk, three rank groups), each
    call equal bit for bit to the first of its shape and that one within the parity bar of
    the oracle's u;
  * a grouped backward whose dy inputs have different widths (one wide, two narrow) packed
    in one launch, into a NaN-filled workspace: dx, dA, dB against the oracle, dA and dB bit
    for bit the single calls', and a second call equal bit for bit to the first."""
import numpy as np
import pytest
import torch

import msq_inputs as mi
from oracle import lora as olora
from oracle import nf4 as onf4

from gpu_util import assert_parity, dev_bf16, dev_f32, host_f64

pytestmark = pytest.mark.gpu
msq = pytest.importorskip("memory_streamed_qlora_amd")

NAN_BYTE = 0xFF  # every fp32 word of a 0xFF-filled buffer is a NaN


def _u_case(T, K, r, p, seed):
    inp = mi.linear_inputs(seed, 1, 0, "q", K, 64, T, mi.LoraSpec(r, 32.0, p))
    codes, a = onf4.quantize(inp["W"])
    key = olora.RngKey(seed=seed, step=3, layer=2, proj=1)
    _, ru = olora.fwd(inp["x"], codes, a, None, inp["A"], inp["B"], 32.0, p, key)
    dev = {"x": dev_bf16(inp["x"]), "codes": torch.from_numpy(codes).cuda(), "absmax": dev_f32(a),
           "A": dev_f32(inp["A"]), "B": dev_f32(inp["B"]), "cfg": msq.Lora(r, 32.0, p),
           "key": msq.rng_key(key.seed, key.step, key.micro, key.layer, key.proj)}
    return dev, ru


def _u_call(c, T, r, path):
    u = torch.full((T, r), float("nan"), device="cuda")
    msq.nf4_lora_fwd(c["x"], c["codes"], c["absmax"], None, c["A"], c["B"], c["cfg"], c["key"], u_out=u,
                     u_only=True, path=path)
    torch.cuda.synchronize()
    return u


@pytest.mark.parametrize("path", ["tiled", "small"])
def test_u_written_on_every_call(path):
    # (T, K, r, p): ragged token groups over a narrow input; a wide input whose last chunk
    # is one k-step, with three rank groups (two ranks blocks, the second partial, on the
    # small-tile path); a single ragged token group over the widest
    shapes = [(1000, 896, 16, 0.1), (1000, 8256, 40 if path == "tiled" else 24, 0.1), (40, 27648, 16, 0.0)]
    cases = []
    for i, (T, K, r, p) in enumerate(shapes):
        print(f"[pack u] T={T} K={K} r={r} p={p}", flush=True)
        cases.append(_u_case(T, K, r, p, 11 + i))
    first = [None] * len(shapes)
    for rnd in range(3):
        for i, ((T, K, r, p), (c, ru)) in enumerate(zip(shapes, cases)):
            u = _u_call(c, T, r, path)
            assert not torch.isnan(u).any(), f"round {rnd} shape {i}: u not written"
            if first[i] is None:
                assert_parity(host_f64(u), ru, name=f"u T={T} K={K} r={r}")
                first[i] = u
            else:
                assert torch.equal(u.view(torch.int32), first[i].view(torch.int32)), f"round {rnd} shape {i}"


def _nan_workspace(nbytes):
    ws = msq.Workspace()
    ws.buf = torch.full((nbytes,), NAN_BYTE, dtype=torch.uint8, device="cuda")
    return ws


def test_grouped_backward_mixed_widths_in_one_launch():
    T, K, ns, r, p, alpha = 300, 256, (8256, 128, 64), 16, 0.1, 32.0
    print(f"[pack group bwd] T={T} K={K} ns={ns}", flush=True)
    x = mi.normal_bf16(mi.rng_for(T, K, 0, 91), (T, K), 1.0)
    cases = []
    for i, n in enumerate(ns):
        inp = mi.linear_inputs(21, 2, 1, ("q", "k", "v")[i], K, n, 8, mi.LoraSpec(r, alpha, p))
        dy = mi.normal_bf16(mi.rng_for(T, n, i, 92), (T, n), 1.0)
        cases.append(dict(inp, dy=dy, key=olora.RngKey(seed=6, step=1, layer=3, proj=i)))
    projs, refs = [], []
    dx_ref = np.zeros((T, K))
    for i, c in enumerate(cases):
        codes, a = onf4.quantize(c["W"])
        W64 = onf4.dequantize(codes, a)
        dxi, dA, dB = olora.bwd_dense(c["dy"], x, W64, c["A"], c["B"], alpha, p, c["key"])
        dx_ref += dxi
        refs.append((dA, dB))
        projs.append({"base": (torch.from_numpy(codes).cuda(), dev_f32(a)), "A": dev_f32(c["A"]),
                      "B": dev_f32(c["B"]), "dy": dev_bf16(c["dy"]), "key": msq.rng_key(6, 1, 0, 3, i)})
    cfg = msq.Lora(r, alpha, p)
    xd = dev_bf16(x)
    ws = _nan_workspace(64 << 20)
    dx, grads = msq.lora_bwd_group(xd, projs, cfg, workspace=ws, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert_parity(host_f64(dx), dx_ref, name="dx")
    for i, ((dA, dB), (rA, rB)) in enumerate(zip(grads, refs)):
        assert_parity(host_f64(dA), rA, name=f"dA{i}")
        assert_parity(host_f64(dB), rB, name=f"dB{i}")
    for pr, (dA, dB) in zip(projs, grads):
        _, sA, sB = msq.nf4_lora_bwd(pr["dy"], xd, *pr["base"], pr["A"], pr["B"], cfg, pr["key"],
                                     out_dtype=torch.float32, path="tiled")
        torch.cuda.synchronize()
        assert torch.equal(dA.view(torch.int32), sA.view(torch.int32))
        assert torch.equal(dB.view(torch.int32), sB.view(torch.int32))
    ws.buf.fill_(NAN_BYTE)
    dx2, grads2 = msq.lora_bwd_group(xd, projs, cfg, workspace=ws, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(dx2.view(torch.int32), dx.view(torch.int32))
    for (dA, dB), (gA, gB) in zip(grads, grads2):
        assert torch.equal(gA.view(torch.int32), dA.view(torch.int32))
        assert torch.equal(gB.view(torch.int32), dB.view(torch.int32))


def test_column_gradient_layouts_agree():
    """dA = du^T x over K = 4096 input columns (a launch of 16-column workgroups) equals the
    first 4096 columns of the same product over K = 32768 (enough columns for 64-column
    workgroups) bit for bit: both widths run each output's products and sums in the same
    order."""
    T, N, r = 512, 256, 16
    g = torch.Generator(device="cuda").manual_seed(41)
    x_wide = torch.randn(T, 32768, generator=g, device="cuda").to(torch.bfloat16)
    dy = torch.randn(T, N, generator=g, device="cuda").to(torch.bfloat16)
    B = torch.randn(N, r, generator=g, device="cuda") * 0.01
    cfg, key = msq.Lora(r, 32.0, 0.0), msq.rng_key(1, 0, 0, 0, 0)
    out = []
    for K in (4096, 32768):
        W = (torch.randn(N, K, generator=g, device="cuda") * 0.02).to(torch.bfloat16)
        A = torch.randn(r, K, generator=g, device="cuda") * 0.01
        u = torch.randn(T, r, generator=g, device="cuda")
        _, dA, dB = msq.nf4_lora_bwd(dy, x_wide[:, :K].contiguous(), *msq.nf4_quantize(W), A, B, cfg, key, u=u,
                                     path="tiled")
        out.append((dA, dB))
    torch.cuda.synchronize()
    assert torch.equal(out[0][0].view(torch.int32), out[1][0][:, :4096].contiguous().view(torch.int32))
