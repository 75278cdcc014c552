"""The bf16-base variant of the path (bf16_lora_fwd / bf16_lora_bwd and a stack streaming
a bf16 base): the pages' bf16 streaming mode, which streams a frozen bf16 base blockwise
at 4x the NF4 bytes and is held to bitwise streamed == resident parity up to the 32B
shape ("Current limitations", "bf16 LoRA").

  * parity with the oracle's dense layer (oracle/lora.py, fwd_dense / bwd_dense), bar
    2e-2 * RMS as for NF4;
  * the bf16 kernels fill the same LDS tiles as the NF4 kernels, only without the
    dequantization: with W equal to the dequantized NF4 matrix both give the same bits,
    which checks the bf16 path at the full 32B projection shapes;
  * streamed == resident bitwise on a tiny stack (dropout on) and on the 64-layer 32B
    stack."""
import dataclasses

import numpy as np
import pytest
import torch

import msq_inputs as mi
from oracle import block as oblock
from oracle import lora as olora
from oracle import step as ostep

from gpu_util import assert_parity, dev_bf16, dev_f32, host_f64
from test_gpu_stack import OPERAND, TINY, _shape, chain_tolerance

pytestmark = pytest.mark.gpu
msq = pytest.importorskip("memory_streamed_qlora_amd")
from memory_streamed_qlora_amd import stack as S  # noqa: E402


def _check(inp, r=16, alpha=32.0, p=0.0, key=olora.RngKey(), bias=None, name=""):
    x, dy = dev_bf16(inp["x"]), dev_bf16(inp["dy"])
    w = dev_bf16(inp["W"])
    A, B = dev_f32(inp["A"][:r]), dev_f32(inp["B"][:, :r])
    b = dev_bf16(bias) if bias is not None else None
    cfg = msq.Lora(r, alpha, p)
    k = msq.rng_key(key.seed, key.step, key.micro, key.layer, key.proj)
    y, u = msq.bf16_lora_fwd(x, w, b, A, B, cfg, k)
    dx, dA, dB = msq.bf16_lora_bwd(dy, x, w, A, B, cfg, k, u=u)
    torch.cuda.synchronize()
    Ar, Br = inp["A"][:r], inp["B"][:, :r]
    ry, ru = olora.fwd_dense(inp["x"], inp["W"], bias, Ar, Br, alpha, p, key)
    rdx, rdA, rdB = olora.bwd_dense(inp["dy"], inp["x"], inp["W"], Ar, Br, alpha, p, key)
    out = {"y": assert_parity(host_f64(y), ry, name=name + " y"),
           "dx": assert_parity(host_f64(dx), rdx, name=name + " dx")}
    if r > 0:
        out["u"] = assert_parity(host_f64(u), ru, name=name + " u")
        out["dA"] = assert_parity(host_f64(dA), rdA, name=name + " dA")
        out["dB"] = assert_parity(host_f64(dB), rdB, name=name + " dB")
    print(name, {k_: f"{v:.2e}" for k_, v in out.items()}, flush=True)


def test_bf16_linear_cfg1_shape():
    _check(mi.cfg1_inputs(), name="bf16 896x896")


def test_bf16_linear_ragged_dropout_bias():
    lo = mi.LoraSpec(16, 32.0, 0.1)
    inp = mi.linear_inputs(1, 2, 3, "q", 384, 640, 300, lo, with_bias=True)
    _check(inp, p=0.1, key=olora.RngKey(seed=7, step=3, layer=2, proj=0), bias=inp["bias"], name="bf16 ragged")


@pytest.mark.parametrize("T,K,N,r", [(1, 64, 64, 1), (129, 256, 64, 33), (64, 4864, 896, 64)])
def test_bf16_linear_odd_shapes(T, K, N, r):
    inp = mi.linear_inputs(3, 2, T, "down", K, N, T, mi.LoraSpec(r, 16.0, 0.2))
    _check(inp, r=r, alpha=16.0, p=0.2, key=olora.RngKey(seed=1, layer=5, proj=6), name=f"bf16 T{T} K{K} N{N}")


# the 32B projection shapes (K, N) at 512 tokens, plus a ragged token count
FULL_SHAPES = [(5120, 5120, 512), (5120, 1024, 512), (5120, 27648, 512), (27648, 5120, 512), (5120, 27648, 77)]


@pytest.mark.parametrize("K,N,T", FULL_SHAPES)
def test_bf16_kernels_equal_nf4_kernels_on_dequantized_weights(K, N, T):
    print(f"[bf16 == nf4] K={K} N={N} T={T}", flush=True)
    g = torch.Generator(device="cuda").manual_seed(K + N + T)
    W = (torch.randn(N, K, generator=g, device="cuda") * 0.02).to(torch.bfloat16)
    codes, absmax = msq.nf4_quantize(W)
    Wd = msq.nf4_dequantize(codes, absmax)
    x = torch.randn(T, K, generator=g, device="cuda")
    dy = torch.randn(T, N, generator=g, device="cuda")
    A = (torch.rand(16, K, generator=g, device="cuda") * 2 - 1) / K ** 0.5
    B = torch.randn(N, 16, generator=g, device="cuda") * 0.01
    cfg, key = msq.Lora(16, 32.0, 0.1), msq.rng_key(1, 2, 0, 3, 4)
    y4, u4 = msq.nf4_lora_fwd(x, codes, absmax, None, A, B, cfg, key)
    yb, ub = msq.bf16_lora_fwd(x, Wd, None, A, B, cfg, key)
    dx4, dA4, dB4 = msq.nf4_lora_bwd(dy, x, codes, absmax, A, B, cfg, key, u=u4)
    dxb, dAb, dBb = msq.bf16_lora_bwd(dy, x, Wd, A, B, cfg, key, u=ub)
    torch.cuda.synchronize()
    for a, b, nm in ((y4, yb, "y"), (u4, ub, "u"), (dx4, dxb, "dx"), (dA4, dAb, "dA"), (dB4, dBb, "dB")):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32)), f"{nm} differs"


def _bf16_stack(layers_np, glob_np, lo, mode, seed, T, window_blocks=1, n_slots=2):
    st = S.Stack(_shape(TINY), T, r=lo.r, alpha=lo.alpha, p_drop=lo.p_drop, window_blocks=window_blocks,
                 mode=mode, seed=seed, n_slots=n_slots, base="bf16")
    for p in layers_np:
        st.add_layer({proj: dev_bf16(p[proj]["W"]) for proj in S.PROJS},
                     {proj: dev_bf16(p[proj]["bias"]) for proj in ("q", "k", "v")},
                     {proj: torch.from_numpy(p[proj]["A"]) for proj in S.PROJS},
                     {proj: torch.from_numpy(p[proj]["B"]) for proj in S.PROJS},
                     torch.from_numpy(p["ln1"]), torch.from_numpy(p["ln2"]))
    st.set_globals(dev_bf16(glob_np["emb"]), dev_bf16(glob_np["lm"]), torch.from_numpy(glob_np["lnf"]))
    st.finalize()
    return st


def test_bf16_stack_streamed_equals_resident_and_oracle():
    lo, seed, T = mi.LoraSpec(8, 16.0, 0.1), 2, 32
    layers = [mi.block_params(seed, 3, l, TINY, lo) for l in range(TINY.layers)]
    glob = mi.stack_globals(seed, 3, TINY, T)
    runs = []
    for mode in ("resident", "streamed"):
        st = _bf16_stack(layers, glob, lo, mode, seed, T)
        losses, first_grads = [], None
        for s in range(6):
            loss, gn = st.train_step(torch.from_numpy(mi.tokens(seed, 3, s, T, TINY.vocab)).cuda())
            losses.append((loss.item(), gn.item()))
            if s == 0:
                first_grads = {k: v.clone() for k, v in st.state_tensors().items() if k.endswith(".grad")}
        torch.cuda.synchronize()
        runs.append((losses, {k: v.clone() for k, v in st.state_tensors().items()}, first_grads))
        st.close()
    (la, sa, ga), (lb, sb, _) = runs
    assert la == lb, "bf16 base: streamed losses differ from resident"
    for k in sa:
        assert torch.equal(sa[k], sb[k]), f"bf16 base: streamed != resident for {k}"
    # the first step's gradients against the oracle's bf16-base step
    bl = [oblock.bf16_params(p) for p in layers]
    rloss, rgrads = ostep.forward_backward(bl, glob, mi.tokens(seed, 3, 0, T, TINY.vocab), TINY, lo.alpha,
                                           lo.p_drop, seed, 0, operand=OPERAND)
    _, exact = ostep.forward_backward(bl, glob, mi.tokens(seed, 3, 0, T, TINY.vocab), TINY, lo.alpha, lo.p_drop, seed, 0)
    tol = chain_tolerance(exact, rgrads)
    assert abs(la[0][0] - rloss) <= 2e-2 * abs(rloss)
    for l in range(TINY.layers):
        for proj in S.PROJS:
            for which, nm in ((0, "A"), (1, "B")):
                assert_parity(host_f64(ga[f"{l}.{proj}.{nm}.grad"]), rgrads[l][proj][which], tol=tol,
                              name=f"bf16 {l}.{proj}.d{nm}")


@pytest.mark.slow
def test_qwen32b_bf16_streamed_equals_resident():
    """32 layers of the Qwen2.5-32B shape with a bf16 base (31.2 GB pinned), window 4 x 3
    slots, dropout 0.0, 2 optimizer steps: streamed == resident on every surface.  Half the
    64 layers: how much host memory a process may pin differs between hosts, and the whole
    bf16 base (62.4 GB) does not fit everywhere.  The lm_head stays on the device."""
    shape = dataclasses.replace(S.QWEN25_32B, layers=32)
    outs = []
    for mode in ("resident", "streamed"):
        print(f"[bf16 32B] building {mode}", flush=True)
        st = S.Stack.random(shape, 512, seed=3, cfg_id=4, r=16, alpha=32.0, p_drop=0.0, window_blocks=4,
                            mode=mode, n_slots=3, base="bf16", lm_stream=False)
        losses = []
        for s in range(2):
            loss, gn = st.train_step(S.random_tokens(3, s, 512, shape.vocab, st.dev))
            losses.append((loss, gn))
        torch.cuda.synchronize()
        outs.append(([(a.item(), b.item()) for a, b in losses], {k: v.clone() for k, v in st.state_tensors().items()}))
        print(f"[bf16 32B] {mode} losses {outs[-1][0]}", flush=True)
        st.close()
        del st
        torch.cuda.empty_cache()
    assert outs[0][0] == outs[1][0]
    for k in outs[0][1]:
        assert torch.equal(outs[0][1][k], outs[1][1][k]), f"bf16 32B: streamed != resident for {k}"
