"""Gradient accumulation on the GPU: 2 and 4 micro-batches, micro-batch-major and
block-major loop orders, streamed and resident, with dropout.

The pages gate accumulation at 2 and 4 micro-batches bitwise and have to reject the
block-major order with dropout, since it would reorder their captured RNG state
("Current limitations", "What 0.00e+00 means"; "Poros" research post, RNG state
capture).  Here masks are keyed by (seed, step, micro, layer, proj), so the order does not
matter: every order and residency must give the same bits, and the result must match the
oracle's accumulated step (oracle/step.py, `accumulated`)."""
import numpy as np
import pytest
import torch

import msq_inputs as mi
from oracle import block as oblock
from oracle import step as ostep

from gpu_util import assert_parity, host_f64
from test_gpu_stack import OPERAND, TINY, _build, _tiny, chain_tolerance

pytestmark = pytest.mark.gpu
msq = pytest.importorskip("memory_streamed_qlora_amd")
from memory_streamed_qlora_amd import stack as S  # noqa: E402


def _ga_run(layers, glob, lo, mode, order, M, steps, seed, T=32, window_blocks=1, n_slots=2):
    st = _build(TINY, T, layers, glob, lo, mode, window_blocks, seed, n_slots)
    losses, norms, copies = [], [], []
    for s in range(steps):
        toks = torch.from_numpy(np.stack([mi.tokens(seed, 3, s * 8 + m, T, TINY.vocab) for m in range(M)])).cuda()
        before = st.window.stats()["windows_copied"] if st.window else 0
        loss, gn = st.train_step(toks, order=order)
        losses.append(loss)
        norms.append(gn)
        copies.append((st.window.stats()["windows_copied"] - before) if st.window else 0)
    torch.cuda.synchronize()
    out = ([v.item() for v in losses], [v.item() for v in norms],
           {k: v.clone() for k, v in st.state_tensors().items()}, copies)
    st.close()
    return out


def _assert_same(a, b, what):
    assert a[0] == b[0], f"{what}: losses differ {a[0]} vs {b[0]}"
    assert a[1] == b[1], f"{what}: grad norms differ"
    assert a[2].keys() == b[2].keys()
    for k in a[2]:
        assert torch.equal(a[2][k], b[2][k]), f"{what}: {k} differs"


@pytest.mark.parametrize("M", [2, 4])
def test_ga_orders_and_residency_bitwise(M):
    print(f"[ga] M={M}", flush=True)
    lo, seed = mi.LoraSpec(8, 16.0, 0.1), 4
    layers, glob = _tiny(seed, lo)
    ref = _ga_run(layers, glob, lo, "resident", "micro", M, 3, seed)
    copies = {}
    for mode, order in (("resident", "block"), ("streamed", "block"), ("streamed", "micro")):
        got = _ga_run(layers, glob, lo, mode, order, M, 3, seed)
        _assert_same(ref, got, f"{mode}/{order} vs resident/micro")
        copies[order] = got[3]
    assert ref[0][0] != ref[0][-1]
    # block-major streams the base once per optimizer step, as a single micro-batch does;
    # micro-major streams it once per micro-batch
    single = _ga_run(layers, glob, lo, "streamed", "block", 1, 3, seed)[3]
    assert copies["block"] == single, (copies, single)
    assert all(c > b for c, b in zip(copies["micro"], copies["block"])), copies


def test_ga_step_vs_oracle():
    """Block-major streamed accumulation over 2 micro-batches with dropout against the
    oracle's accumulated step (mean loss, mean gradient)."""
    lo, seed, T, M = mi.LoraSpec(8, 16.0, 0.1), 6, 32, 2
    layers, glob = _tiny(seed, lo)
    toks_np = [mi.tokens(seed, 3, m, T, TINY.vocab) for m in range(M)]
    st = _build(TINY, T, layers, glob, lo, "streamed", 1, seed)
    loss, gn = st.train_step(torch.from_numpy(np.stack(toks_np)).cuda(), order="block")
    torch.cuda.synchronize()
    qlayers = [oblock.quantize_params(p) for p in layers]
    rloss, rgrads = ostep.accumulated(qlayers, glob, toks_np, TINY, lo.alpha, lo.p_drop, seed, 0,
                                     operand=OPERAND)
    _, exact = ostep.accumulated(qlayers, glob, toks_np, TINY, lo.alpha, lo.p_drop, seed, 0)
    tol = chain_tolerance(exact, rgrads)
    assert abs(loss.item() - rloss) <= 2e-2 * abs(rloss)
    assert abs(gn.item() - ostep.grad_norm(rgrads)) <= 2e-2 * ostep.grad_norm(rgrads)
    state = st.state_tensors()
    for l in range(TINY.layers):
        for proj in S.PROJS:
            for which, nm in ((0, "A"), (1, "B")):
                assert_parity(host_f64(state[f"{l}.{proj}.{nm}.grad"]), rgrads[l][proj][which], tol=tol,
                              name=f"{l}.{proj}.d{nm}")
    st.close()


@pytest.mark.slow
def test_qwen7b_ga4_block_major_streamed_equals_micro_major_resident():
    """Real size: the 28-layer Qwen2.5-7B shape, 4 micro-batches of 512 tokens, dropout
    0.1 (masks replayed in the recompute), window 4 x 2 slots; 2 optimizer steps."""
    shape = S.QWEN25_7B
    outs = []
    for mode, order in (("resident", "micro"), ("streamed", "block")):
        print(f"[ga 7B] {mode}/{order}", flush=True)
        st = S.Stack.random(shape, 512, seed=9, cfg_id=2, r=16, alpha=32.0, p_drop=0.1, window_blocks=4,
                            mode=mode, n_slots=2)
        losses, norms = [], []
        for s in range(2):
            toks = torch.stack([S.random_tokens(9, 4 * s + m, 512, shape.vocab, st.dev) for m in range(4)])
            loss, gn = st.train_step(toks, order=order)
            losses.append(loss)
            norms.append(gn)
        torch.cuda.synchronize()
        outs.append(([v.item() for v in losses], [v.item() for v in norms],
                     {k: v.clone() for k, v in st.state_tensors().items()}))
        print(f"[ga 7B] {mode}/{order} losses {outs[-1][0]}", flush=True)
        st.close()
        del st
        torch.cuda.empty_cache()
    _assert_same(outs[0], outs[1], "7B GA4 streamed/block vs resident/micro")
