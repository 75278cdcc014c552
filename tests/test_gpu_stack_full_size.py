"""Full-size streamed == resident parity runs of the training step.

The pages gate streaming on bitwise equality with the fully resident run over 200
optimizer steps ("Poros" research post, correctness paragraph; A100 benchmark matrix):
losses, adapter weights, adapter gradients and optimizer state must match exactly.
These runs use the Qwen2.5 stack shapes of the workloads the pages measure, with
synthetic random weights and tokens.
"""
import time

import pytest
import torch

from memory_streamed_qlora_amd import stack as S

pytestmark = [pytest.mark.gpu, pytest.mark.slow, pytest.mark.timeout(900)]


def _run(sh, mode, steps, window_blocks, n_slots, p_drop, cfg_id, every):
    st = S.Stack.random(sh, 512, seed=0, cfg_id=cfg_id, r=16, alpha=32.0, p_drop=p_drop,
                        window_blocks=window_blocks, n_slots=n_slots, mode=mode)
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    losses, norms = [], []
    t0 = time.perf_counter()
    for s in range(steps):
        loss, gn = st.train_step(S.random_tokens(0, s, 512, sh.vocab, "cpu"))
        losses.append(loss)
        norms.append(gn)
        if (s + 1) % every == 0:
            torch.cuda.synchronize()
            print(f"{mode} step {s + 1}/{steps} loss {loss.item():.6f} "
                  f"{(time.perf_counter() - t0) / (s + 1) * 1e3:.0f} ms/step", flush=True)
    torch.cuda.synchronize()
    secs = time.perf_counter() - t0
    peak = torch.cuda.max_memory_allocated() / 1e9  # before the state copies below
    out = {"losses": [l.item() for l in losses], "norms": [g.item() for g in norms],
           "state": {k: v.clone() for k, v in st.state_tensors().items()},
           "stats": st.window.stats() if st.window else None,
           "ms_per_step": secs / steps * 1e3,
           "peak_gb": peak}
    st.close()
    del st
    torch.cuda.empty_cache()
    return out


def _assert_bitwise(res, stm):
    assert res["losses"] == stm["losses"], "loss stream differs"
    assert res["norms"] == stm["norms"], "grad-norm stream differs"
    assert res["state"].keys() == stm["state"].keys()
    for k in res["state"]:
        assert torch.equal(res["state"][k], stm["state"][k]), f"streamed != resident for {k}"


def test_qwen7b_200_steps_streamed_equals_resident():
    """Qwen2.5-7B-shaped stack, 28 layers streamed in windows of 4 blocks through two
    slots, LoRA r16 alpha32 dropout 0.1, 512 tokens, 200 AdamW steps."""
    sh, steps = S.QWEN25_7B, 200
    res = _run(sh, "resident", steps, 4, 2, 0.1, 3, every=20)
    stm = _run(sh, "streamed", steps, 4, 2, 0.1, 3, every=20)
    _assert_bitwise(res, stm)
    assert res["losses"][0] != res["losses"][-1]
    n_win = 28 // 4
    assert stm["stats"]["windows_copied"] + stm["stats"]["windows_reused"] == steps * 2 * n_win
    print(f"7B: streamed {stm['ms_per_step']:.1f} ms/step, peak {stm['peak_gb']:.2f} GB; "
          f"resident {res['ms_per_step']:.1f} ms/step, peak {res['peak_gb']:.2f} GB", flush=True)


def test_qwen32b_200_steps_streamed_equals_resident():
    """Qwen2.5-32B-shaped stack, 64 layers streamed in windows of 4 blocks through seven
    slots with the lm_head streamed by the loss (the benchmark's configuration), LoRA r16
    alpha32 dropout 0.0, 512 tokens, 200 AdamW steps: every loss, grad norm, adapter,
    gradient and AdamW moment equal."""
    sh, steps = S.QWEN25_32B, 200
    stm = _run(sh, "streamed", steps, 4, 7, 0.0, 4, every=20)
    res = _run(sh, "resident", steps, 4, 7, 0.0, 4, every=20)
    _assert_bitwise(res, stm)
    assert res["losses"][0] != res["losses"][-1]
    print(f"32B: streamed {stm['ms_per_step']:.1f} ms/step, peak {stm['peak_gb']:.2f} GB; "
          f"resident {res['ms_per_step']:.1f} ms/step, peak {res['peak_gb']:.2f} GB", flush=True)


def test_qwen72b_streamed_equals_resident():
    """Qwen2.5-72B-shaped stack, 80 layers streamed in windows of 4 blocks (three
    slots), LoRA r16 alpha32 dropout 0.1 with the masks replayed in the recompute,
    512 tokens: the first 5 AdamW steps bitwise against the resident run."""
    sh, steps = S.QWEN25_72B, 5
    stm = _run(sh, "streamed", steps, 4, 3, 0.1, 5, every=1)
    res = _run(sh, "resident", steps, 4, 3, 0.1, 5, every=1)
    _assert_bitwise(res, stm)
    print(f"72B: streamed {stm['ms_per_step']:.1f} ms/step, peak {stm['peak_gb']:.2f} GB; "
          f"resident {res['ms_per_step']:.1f} ms/step, peak {res['peak_gb']:.2f} GB", flush=True)
