"""Pointwise block glue in the library: SwiGLU, rotary embedding, RMSNorm's pointwise
tail and the residual add fused into a projection's output pass.

The pages allow a fused kernel around the engine only when it is a pointwise chain that
yields the unfused chain's values ("Poros" README, Roadmap, "The Poros kernel").  So each
fused kernel is held to two bars:
  * bit-exact against the unfused PyTorch chain it replaces, forward and autograd backward
    (the stack's glue="torch"), and a whole training step with glue="native" equal to the
    glue="torch" step on every loss, gradient, adapter weight and AdamW moment;
  * the oracle's fp64 definitions (oracle/block.py) within the parity bar, and within a
    few fp32 roundings (each output is at most five rounded fp32 operations plus one
    exp, so 1e-5 relative to the RMS of the reference is ample)."""
import numpy as np
import pytest
import torch

import msq_inputs as mi
from oracle import block as oblock

from gpu_util import assert_parity, host_f64

pytestmark = pytest.mark.gpu
msq = pytest.importorskip("memory_streamed_qlora_amd")
from memory_streamed_qlora_amd import stack as S  # noqa: E402
from memory_streamed_qlora_amd._abi import MSQ_E_SHAPE, MsqError  # noqa: E402

FP32_CHAIN_TOL = 1e-5


def _bits_equal(a: torch.Tensor, b: torch.Tensor) -> bool:
    return a.shape == b.shape and torch.equal(a.contiguous().view(torch.int32), b.contiguous().view(torch.int32))


def _gate_values(n: int, seed: int) -> torch.Tensor:
    """Gate pre-activations: mostly N(0, 3), a slice spread over +-100 (exp overflows and
    saturates there), and the special values 0, -0, +-1e-30, +-20, +-88, +-89, +-100."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    x = torch.randn(n, generator=g) * 3
    wide = n // 8
    x[:wide] = (torch.rand(wide, generator=g) - 0.5) * 200
    sp = torch.tensor([0.0, -0.0, 1e-30, -1e-30, 20.0, -20.0, 88.0, -88.0, 89.0, -89.0, 100.0, -100.0])
    k = min(n, sp.numel())
    x[n - k:] = sp[:k]
    return x.cuda()


@pytest.mark.parametrize("n", [0, 1, 3, 4, 1027, 512 * 4864])
def test_swiglu_bitwise_unfused_and_oracle(n):
    print(f"[swiglu] n={n}", flush=True)
    gen = torch.Generator(device="cpu").manual_seed(11 + n)
    g = _gate_values(n, 7 + n)
    u = torch.randn(n, generator=gen).cuda()
    da = torch.randn(n, generator=gen).cuda()
    a = msq.swiglu_fwd(g, u)
    dg, du = msq.swiglu_bwd(da, g, u)
    # the unfused chain, forward and its autograd backward
    gr, ur = g.clone().requires_grad_(), u.clone().requires_grad_()
    ref = torch.nn.functional.silu(gr) * ur
    ref.backward(da)
    torch.cuda.synchronize()
    assert _bits_equal(a, ref.detach()), "swiglu_fwd != silu(g) * u"
    assert _bits_equal(dg, gr.grad), "swiglu_bwd dg != autograd of the unfused chain"
    assert _bits_equal(du, ur.grad), "swiglu_bwd du != autograd of the unfused chain"
    # in place: dg over g, du over u, the same bits
    gi, ui = g.clone(), u.clone()
    dgi, dui = msq.swiglu_bwd(da, gi, ui, in_place=True)
    torch.cuda.synchronize()
    assert dgi.data_ptr() == gi.data_ptr() and dui.data_ptr() == ui.data_ptr()
    assert _bits_equal(dgi, dg) and _bits_equal(dui, du), "in-place swiglu_bwd differs"
    if n == 0:
        return
    g64, u64, da64 = host_f64(g), host_f64(u), host_f64(da)
    for got, want, nm in ((a, oblock.silu(g64) * u64, "a"),
                          (dg, da64 * u64 * oblock.silu_grad(g64), "dg"),
                          (du, da64 * oblock.silu(g64), "du")):
        assert_parity(host_f64(got), want, name=nm)
        assert_parity(host_f64(got), want, tol=FP32_CHAIN_TOL, name=nm)


@pytest.mark.parametrize("T,H,D", [(1, 1, 2), (7, 3, 64), (33, 5, 6), (512, 40, 128), (512, 8, 128)])
def test_rope_bitwise_unfused_and_oracle(T, H, D):
    print(f"[rope] T={T} H={H} D={D}", flush=True)
    cos, sin = S.rope_tables(T, D, "cuda")
    gen = torch.Generator(device="cpu").manual_seed(T * 131 + H * 7 + D)
    x = torch.randn(T, H, D, generator=gen).cuda()
    dy = torch.randn(T, H, D, generator=gen).cuda()
    y = msq.rope_fwd(x, cos, sin)
    dx = msq.rope_bwd(dy, cos, sin)
    xr = x.clone().requires_grad_()
    ref = S.rope(xr, cos, sin)
    ref.backward(dy)
    torch.cuda.synchronize()
    assert _bits_equal(y, ref.detach()), "rope_fwd != the unfused chain"
    assert _bits_equal(dx, xr.grad), "rope_bwd != autograd of the unfused chain"
    c64, s64 = host_f64(cos), host_f64(sin)
    want_y = oblock.rope(host_f64(x), c64, s64)
    want_dx = oblock.rope_bwd(host_f64(dy), c64, s64)
    for got, want, nm in ((y, want_y, "y"), (dx, want_dx, "dx")):
        assert_parity(host_f64(got), want, name=nm)
        assert_parity(host_f64(got), want, tol=FP32_CHAIN_TOL, name=nm)


@pytest.mark.parametrize("T,H", [(1, 4), (5, 64), (512, 896), (512, 5120), (77, 8192)])
def test_rmsnorm_apply_bitwise_unfused_and_oracle(T, H):
    """The whole RMSNorm with its pointwise tail fused equals the unfused chain, forward and
    the input gradient through autograd (the mean and its gradient stay in PyTorch)."""
    print(f"[rmsnorm] T={T} H={H}", flush=True)
    gen = torch.Generator(device="cpu").manual_seed(T * 7 + H)
    h = (torch.randn(T, H, generator=gen) * 2).cuda()
    w = (1 + 0.02 * torch.randn(H, generator=gen)).cuda()
    dy = torch.randn(T, H, generator=gen).cuda()
    hn, hr = h.clone().requires_grad_(), h.clone().requires_grad_()
    y = S.rmsnorm_native(hn, w)
    ref = S.rmsnorm(hr, w)
    y.backward(dy)
    ref.backward(dy)
    torch.cuda.synchronize()
    assert _bits_equal(y.detach(), ref.detach()), "fused RMSNorm != the unfused chain"
    assert _bits_equal(hn.grad, hr.grad), "fused RMSNorm backward != autograd of the unfused chain"
    want_y, rinv = oblock.rmsnorm(host_f64(h), host_f64(w))
    want_dx = oblock.rmsnorm_bwd(host_f64(h), host_f64(w), rinv, host_f64(dy))
    for got, want, nm in ((y, want_y, "y"), (hn.grad, want_dx, "dx")):
        assert_parity(host_f64(got), want, name=nm)
        assert_parity(host_f64(got), want, tol=FP32_CHAIN_TOL, name=nm)


def test_glue_rejects_bad_shapes():
    x = torch.zeros(4, 2, 6, device="cuda")
    cs = torch.zeros(4, 6, device="cuda")
    with pytest.raises(ValueError):
        msq.rope_fwd(x, cs[:3].contiguous(), cs)
    with pytest.raises(MsqError) as e:
        msq.rope_fwd(torch.zeros(4, 2, 5, device="cuda"), torch.zeros(4, 5, device="cuda"),
                     torch.zeros(4, 5, device="cuda"))
    assert e.value.code == MSQ_E_SHAPE
    with pytest.raises(TypeError):
        msq.swiglu_fwd(torch.zeros(8, device="cuda", dtype=torch.bfloat16), torch.zeros(8, device="cuda"))
    with pytest.raises(MsqError) as e:
        msq.rmsnorm_apply_fwd(torch.zeros(3, 6, device="cuda"), torch.zeros(3, 1, device="cuda"),
                              torch.zeros(6, device="cuda"))
    assert e.value.code == MSQ_E_SHAPE


# (t, k, n): the first shapes take a single-pass plan (4 k-steps admit no split), the
# others split the reduction (partials + split_reduce)
RES_SHAPES = [(100, 256, 192), (1, 256, 64), (512, 896, 896), (77, 4864, 896)]


@pytest.mark.parametrize("t,k,n", RES_SHAPES)
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_residual_fused_equals_separate_add(t, k, n, out_dtype):
    print(f"[residual] t={t} k={k} n={n} {out_dtype}", flush=True)
    seed = t + k + n
    inp = mi.linear_inputs(seed, 1, 0, "o", k, n, t, mi.LoraSpec(16, 32.0, 0.1))
    W = torch.from_numpy(inp["W"]).cuda().to(torch.bfloat16)
    codes, absmax = msq.nf4_quantize(W)
    gen = torch.Generator(device="cpu").manual_seed(seed)
    x = torch.randn(t, k, generator=gen).cuda()
    A = torch.from_numpy(inp["A"]).cuda()
    B = torch.from_numpy(inp["B"]).cuda()
    bias = (torch.randn(n, generator=gen) * 0.02).cuda().to(torch.bfloat16)
    res = torch.randn(t, n, generator=gen).cuda().to(out_dtype)
    cfg = msq.Lora(16, 32.0, 0.1)
    key = msq.rng_key(seed, 1, 0, 2, 3)
    y, _ = msq.nf4_lora_fwd(x, codes, absmax, bias, A, B, cfg, key, want_u=False, out_dtype=out_dtype)
    fused, _ = msq.nf4_lora_fwd(x, codes, absmax, bias, A, B, cfg, key, want_u=False, out_dtype=out_dtype,
                                residual=res)
    inplace = res.clone()
    msq.nf4_lora_fwd(x, codes, absmax, bias, A, B, cfg, key, y=inplace, want_u=False, residual=inplace)
    torch.cuda.synchronize()
    want = res + y
    iv = torch.int16 if out_dtype == torch.bfloat16 else torch.int32
    assert torch.equal(fused.view(iv), want.view(iv)), "fused residual != separate add"
    assert torch.equal(inplace.view(iv), want.view(iv)), "in-place residual != separate add"


def _stack_run(shape, seq, glue, mode, steps, seed, p_drop, window_blocks=1):
    st = S.Stack.random(shape, seq, seed=seed, r=16, alpha=32.0, p_drop=p_drop, window_blocks=window_blocks,
                        mode=mode, glue=glue)
    losses, norms = [], []
    for s in range(steps):
        toks = S.random_tokens(seed, s, seq, shape.vocab, st.dev)
        loss, gn = st.train_step(toks)
        losses.append(loss)
        norms.append(gn)
    torch.cuda.synchronize()
    out = ([v.item() for v in losses], [v.item() for v in norms],
           {k: v.clone() for k, v in st.state_tensors().items()})
    st.close()
    return out


@pytest.mark.parametrize("name,shape,seq,mode,steps", [
    ("tiny", S.Shape(128, 2, 1, 64, 256, 3, 512), 32, "resident", 4),
    ("qwen05b-2layers", S.Shape(896, 14, 2, 64, 4864, 2), 512, "streamed", 2),
    ("qwen32b-2layers", S.Shape(5120, 40, 8, 128, 27648, 2), 512, "streamed", 2),
])
def test_native_glue_step_equals_torch_glue_bitwise(name, shape, seq, mode, steps):
    """The whole training step (forward, recompute, backward, AdamW) with the fused glue
    equals the step with the unfused PyTorch glue, bit for bit."""
    print(f"[glue step] {name}", flush=True)
    nat = _stack_run(shape, seq, "native", mode, steps, 5, 0.1)
    ref = _stack_run(shape, seq, "torch", mode, steps, 5, 0.1)
    assert nat[0] == ref[0], f"losses differ: {nat[0]} vs {ref[0]}"
    assert nat[1] == ref[1], f"grad norms differ: {nat[1]} vs {ref[1]}"
    assert nat[2].keys() == ref[2].keys()
    for k in nat[2]:
        assert torch.equal(nat[2][k], ref[2][k]), f"native glue != torch glue for {k}"
    assert nat[0][0] != nat[0][-1]
