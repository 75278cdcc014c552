"""The forward with u given (MSQ_U_GIVEN): the recompute of a block uses the u its first
forward kept instead of forming the rank-r product again.

  * single calls on both paths and a group: y with the u the call itself would form equals
    the plain call's y bit for bit, and the given u is not written;
  * the given u is the one used: twice u adds s * u B^T once more (fp32 rounding apart);
  * a stack whose recompute uses the kept u (the default) equals one that forms u again,
    bit for bit on every parity surface: losses, grad norms, adapters, gradients, AdamW
    moments (dropout 0.1, the q/k/v and gate/up groups, the selective recompute of down)."""
import pytest
import torch

pytestmark = pytest.mark.gpu
msq = pytest.importorskip("memory_streamed_qlora_amd")
from memory_streamed_qlora_amd import stack as S  # noqa: E402


def _lin(K, N, T, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    W = (torch.randn(N, K, generator=g, device="cuda") * 0.02).to(torch.bfloat16)
    codes, absmax = msq.nf4_quantize(W)
    x = torch.randn(T, K, generator=g, device="cuda")
    A = (torch.rand(16, K, generator=g, device="cuda") * 2 - 1) / K ** 0.5
    B = torch.randn(N, 16, generator=g, device="cuda") * 0.01
    bias = (torch.randn(N, generator=g, device="cuda") * 0.02).to(torch.bfloat16)
    return codes, absmax, x, A, B, bias


@pytest.mark.parametrize("path", ["tiled", "small"])
@pytest.mark.parametrize("K,N,T", [(896, 896, 512), (896, 128, 300), (1024, 640, 1000)])
def test_single_call_with_given_u(path, K, N, T):
    print(f"[u given] {path} K={K} N={N} T={T}", flush=True)
    codes, absmax, x, A, B, bias = _lin(K, N, T, K + N + T)
    cfg, key = msq.Lora(16, 32.0, 0.1), msq.rng_key(4, 2, 0, 7, 3)
    y, u = msq.nf4_lora_fwd(x, codes, absmax, bias, A, B, cfg, key, out_dtype=torch.float32, path=path)
    u_in = u.clone()
    y2, u2 = msq.nf4_lora_fwd(x, codes, absmax, bias, A, B, cfg, key, u_out=u_in, u_given=True,
                              out_dtype=torch.float32, path=path)
    torch.cuda.synchronize()
    assert u2 is u_in and torch.equal(u_in.view(torch.int32), u.view(torch.int32)), "the given u was written"
    assert torch.equal(y2.view(torch.int32), y.view(torch.int32))
    # twice the u: y moves by s u B^T
    y3, _ = msq.nf4_lora_fwd(x, codes, absmax, bias, A, B, cfg, key, u_out=2 * u, u_given=True,
                             out_dtype=torch.float32, path=path)
    torch.cuda.synchronize()
    want = (cfg.alpha / cfg.r) * (u.double() @ B.double().t())
    d = (y3.double() - y.double()) - want
    assert d.abs().max().item() <= 1e-4 * want.pow(2).mean().sqrt().item() + 1e-6


def test_group_with_given_u():
    T, K = 512, 896
    g = torch.Generator(device="cuda").manual_seed(3)
    x = torch.randn(T, K, generator=g, device="cuda")
    projs = []
    for i, n in enumerate((896, 128, 128)):
        W = (torch.randn(n, K, generator=g, device="cuda") * 0.02).to(torch.bfloat16)
        projs.append({"base": msq.nf4_quantize(W), "bias": None, "key": msq.rng_key(1, 0, 0, 2, i),
                      "A": torch.randn(16, K, generator=g, device="cuda") * 0.03,
                      "B": torch.randn(n, 16, generator=g, device="cuda") * 0.01})
    cfg = msq.Lora(16, 32.0, 0.1)
    outs = msq.lora_fwd_group(x, projs, cfg, out_dtype=torch.float32)
    given = [dict(pr, u=u.clone()) for pr, (_, u) in zip(projs, outs)]
    outs2 = msq.lora_fwd_group(x, given, cfg, u_given=True, out_dtype=torch.float32)
    torch.cuda.synchronize()
    for i, ((y, u), (y2, u2), pr) in enumerate(zip(outs, outs2, given)):
        assert u2 is pr["u"] and torch.equal(u2, u), f"projection {i}: the given u was written"
        assert torch.equal(y2.view(torch.int32), y.view(torch.int32)), f"projection {i}: y differs"


def test_stack_recompute_with_kept_u_bitwise():
    sh = S.Shape(hidden=256, heads=4, kv_heads=2, head_dim=64, inter=512, layers=4, vocab=1024)
    out = []
    for keep in (False, True):
        st = S.Stack.random(sh, 256, seed=5, cfg_id=2, r=16, alpha=32.0, p_drop=0.1, window_blocks=2,
                            mode="streamed", keep_u=keep)
        losses, norms = [], []
        for s in range(3):
            loss, gn = st.train_step(S.random_tokens(5, s, 256, sh.vocab, st.dev))
            losses.append(loss.item())
            norms.append(gn.item())
        assert not st._u_kept
        out.append((losses, norms, {k: v.clone() for k, v in st.state_tensors().items()}))
        st.close()
        del st
        torch.cuda.empty_cache()
    assert out[0][0] == out[1][0] and out[0][1] == out[1][1]
    for k, v in out[0][2].items():
        assert torch.equal(v, out[1][2][k]), k
