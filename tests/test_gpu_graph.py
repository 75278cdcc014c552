"""The fused linear's forward and backward captured in a HIP graph (a caller removing the
per-call host work of latency-bound shapes): each replay, with eager work and
synchronizations between the replays, gives the eager calls' outputs bit for bit, on
both paths, with dropout (the mask replayed from the same key) and with u recomputed."""
import pytest
import torch

pytestmark = pytest.mark.gpu
msq = pytest.importorskip("memory_streamed_qlora_amd")


@pytest.mark.parametrize("path", ["tiled", "small"])
@pytest.mark.parametrize("K,N,T,p", [(896, 896, 512, 0.0), (896, 128, 300, 0.1), (4864, 896, 200, 0.1)])
def test_graph_replays_equal_eager(path, K, N, T, p):
    print(f"[graph] {path} K={K} N={N} T={T} p={p}", flush=True)
    g = torch.Generator(device="cuda").manual_seed(K + N + T)
    W = (torch.randn(N, K, generator=g, device="cuda") * 0.02).to(torch.bfloat16)
    codes, absmax = msq.nf4_quantize(W)
    x = torch.randn(T, K, generator=g, device="cuda").to(torch.bfloat16)
    dy = torch.randn(T, N, generator=g, device="cuda").to(torch.bfloat16)
    A = (torch.rand(16, K, generator=g, device="cuda") * 2 - 1) / K ** 0.5
    B = torch.randn(N, 16, generator=g, device="cuda") * 0.01
    bias = (torch.randn(N, generator=g, device="cuda") * 0.02).to(torch.bfloat16)
    cfg, key = msq.Lora(16, 32.0, p), msq.rng_key(3, 1, 0, 2, 5)

    def step():
        y, u = msq.nf4_lora_fwd(x, codes, absmax, bias, A, B, cfg, key, path=path)
        dx, dA, dB = msq.nf4_lora_bwd(dy, x, codes, absmax, A, B, cfg, key, u=u, path=path)
        dx2, _, _ = msq.nf4_lora_bwd(dy, x, codes, absmax, A, B, cfg, key, path=path)  # u recomputed
        return y, u, dx, dA, dB, dx2

    eager = step()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = step()
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        for nm, a, b in zip(("y", "u", "dx", "dA", "dB", "dx (u recomputed)"), outs, eager):
            iv = torch.int16 if a.dtype == torch.bfloat16 else torch.int32
            assert torch.equal(a.view(iv), b.view(iv)), f"replay {rep}: {nm} differs"
        step()  # eager work between the replays
        torch.cuda.synchronize()
