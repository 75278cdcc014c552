"""Pins for the oracle's training step (CPU only): AdamW against torch's
implementation, the loss against torch's cross-entropy, and finite differences
of the whole stack's loss."""
import numpy as np
import torch

import msq_inputs as mi
from oracle import block, step


def test_adamw_matches_torch():
    rng = np.random.default_rng(0)
    p0 = rng.standard_normal((7, 5))
    tp = torch.nn.Parameter(torch.from_numpy(p0.copy()))
    opt = torch.optim.AdamW([tp], lr=2e-4, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.01)
    p, m, v = p0.copy(), np.zeros_like(p0), np.zeros_like(p0)
    for t in range(1, 4):
        g = rng.standard_normal((7, 5))
        tp.grad = torch.from_numpy(g.copy())
        opt.step()
        p, m, v = step.adamw(p, g, m, v, t)
        assert np.allclose(p, tp.detach().numpy(), rtol=1e-14, atol=1e-15)


def test_loss_matches_torch_cross_entropy():
    rng = np.random.default_rng(1)
    logits = rng.standard_normal((9, 13)) * 3
    toks = rng.integers(0, 13, 9)
    loss, d = step.loss_and_dlogits(logits, toks)
    tl = torch.from_numpy(logits.copy()).requires_grad_()
    ref = torch.nn.functional.cross_entropy(tl[:-1], torch.from_numpy(toks[1:]))
    ref.backward()
    assert abs(loss - ref.item()) < 1e-13
    assert np.allclose(d, tl.grad.numpy(), atol=1e-15)


def test_stack_finite_differences():
    sh = mi.TINY
    alpha, p, seed = 8.0, 0.1, 3
    layers = []
    for li in range(sh.layers):
        prm = mi.block_params(0, 88, li, sh, mi.LoraSpec(4, alpha, p), w_std=0.2)
        for proj in block.PROJS:
            prm[proj]["B"] = (prm[proj]["B"] * 30).astype(np.float32)
        layers.append(block.quantize_params(prm))
    glob = mi.stack_globals(0, 88, sh, 8)
    glob = {k: (v * 10 if k in ("emb", "lm") else v) for k, v in glob.items()}
    toks = mi.tokens(0, 88, 0, 8, sh.vocab)
    loss, grads = step.forward_backward(layers, glob, toks, sh, alpha, p, seed, 0)
    assert np.isfinite(loss)
    h = 1e-6
    rng = np.random.default_rng(2)
    for li, proj, name in [(0, "q", "A"), (0, "down", "B"), (1, "v", "B"), (1, "gate", "A"), (0, "o", "B")]:
        g = grads[li][proj][0 if name == "A" else 1]
        for _ in range(2):
            idx = tuple(int(rng.integers(0, s)) for s in g.shape)

            def with_delta(dlt):
                ls = [dict(l) for l in layers]
                ls[li] = {k: (dict(v) if isinstance(v, dict) else v) for k, v in layers[li].items()}
                arr = layers[li][proj][name].astype(np.float64).copy()
                arr[idx] += dlt
                ls[li][proj][name] = arr
                return step.forward_backward(ls, glob, toks, sh, alpha, p, seed, 0)[0]

            fd = (with_delta(h) - with_delta(-h)) / (2 * h)
            assert abs(fd - g[idx]) <= 1e-6 * max(1e-3, abs(fd)) + 1e-9, (li, proj, name, fd, g[idx])


def test_grad_norm_is_l2_of_everything():
    rng = np.random.default_rng(3)
    grads = [{p: (rng.standard_normal((2, 3)), rng.standard_normal((4, 2))) for p in block.PROJS}
             for _ in range(2)]
    flat = np.concatenate([np.concatenate([g[p][0].ravel(), g[p][1].ravel()])
                           for g in grads for p in block.PROJS])
    assert np.isclose(step.grad_norm(grads), np.linalg.norm(flat), rtol=1e-14)
