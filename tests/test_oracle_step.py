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


def _fd_stack(p_drop=0.1):
    sh = mi.TINY
    alpha = 8.0
    layers = []
    for li in range(sh.layers):
        prm = mi.block_params(0, 89, li, sh, mi.LoraSpec(4, alpha, p_drop), w_std=0.2)
        for proj in block.PROJS:
            prm[proj]["B"] = (prm[proj]["B"] * 30).astype(np.float32)
        layers.append(block.quantize_params(prm))
    glob = mi.stack_globals(0, 89, sh, 8)
    glob = {k: (v * 10 if k in ("emb", "lm") else v) for k, v in glob.items()}
    return sh, alpha, layers, glob


def test_accumulated_gradient_is_gradient_of_mean_loss():
    """Finite differences of the mean loss over 2 micro-batches with dropout (each
    micro-batch its own masks) against the accumulated gradient."""
    sh, alpha, layers, glob = _fd_stack(0.1)
    toks = [mi.tokens(0, 89, m, 8, sh.vocab) for m in range(2)]
    loss, grads = step.accumulated(layers, glob, toks, sh, alpha, 0.1, 5, 2)
    h = 1e-6
    rng = np.random.default_rng(4)
    for li, proj, name in [(0, "k", "A"), (1, "up", "B"), (1, "o", "A")]:
        g = grads[li][proj][0 if name == "A" else 1]
        idx = tuple(int(rng.integers(0, s)) for s in g.shape)

        def with_delta(dlt):
            ls = [dict(l) for l in layers]
            ls[li] = {k: (dict(v) if isinstance(v, dict) else v) for k, v in layers[li].items()}
            arr = layers[li][proj][name].astype(np.float64).copy()
            arr[idx] += dlt
            ls[li][proj][name] = arr
            return step.accumulated(ls, glob, toks, sh, alpha, 0.1, 5, 2)[0]

        fd = (with_delta(h) - with_delta(-h)) / (2 * h)
        assert abs(fd - g[idx]) <= 1e-6 * max(1e-3, abs(fd)) + 1e-9, (li, proj, name, fd, g[idx])


def test_accumulation_special_cases():
    """Without dropout, M copies of one micro-batch give that micro-batch's loss and
    gradient; with dropout the copies differ (micro keys the masks), and the result is the
    mean of the separately computed micro-batch results."""
    sh, alpha, layers, glob = _fd_stack(0.0)
    t0 = mi.tokens(0, 89, 0, 8, sh.vocab)
    l1, g1 = step.forward_backward(layers, glob, t0, sh, alpha, 0.0, 5, 0)
    l4, g4 = step.accumulated(layers, glob, [t0] * 4, sh, alpha, 0.0, 5, 0)
    assert abs(l4 - l1) <= 1e-14 * abs(l1)
    for a, b in zip(g1, g4):
        for proj in block.PROJS:
            for i in range(2):
                assert np.allclose(a[proj][i], b[proj][i], rtol=1e-13, atol=1e-18)
    sh, alpha, layers, glob = _fd_stack(0.1)
    la, ga = step.forward_backward(layers, glob, t0, sh, alpha, 0.1, 5, 0, micro=0)
    lb, gb = step.forward_backward(layers, glob, t0, sh, alpha, 0.1, 5, 0, micro=1)
    assert la != lb
    l2, g2 = step.accumulated(layers, glob, [t0, t0], sh, alpha, 0.1, 5, 0)
    assert abs(l2 - (la + lb) / 2) <= 1e-14 * abs(l2)
    assert np.allclose(g2[1]["gate"][0], (ga[1]["gate"][0] + gb[1]["gate"][0]) / 2, rtol=1e-13, atol=1e-18)


def test_bf16_base_step():
    """The bf16-base stack (frozen base kept in bf16): with W set to the dequantized NF4
    matrices it reproduces the NF4 stack exactly, and with its own bf16 W its gradient
    matches central differences of its loss."""
    from oracle import nf4
    sh, alpha, layers, glob = _fd_stack(0.1)
    toks = mi.tokens(0, 89, 0, 8, sh.vocab)
    as_bf16 = []
    for qp in layers:
        d = {proj: {"W": nf4.dequantize(qp[proj]["codes"], qp[proj]["absmax"]), "bias": qp[proj]["bias"],
                    "A": qp[proj]["A"], "B": qp[proj]["B"]} for proj in block.PROJS}
        d["ln1"], d["ln2"] = qp["ln1"], qp["ln2"]
        as_bf16.append(d)
    la, ga = step.forward_backward(layers, glob, toks, sh, alpha, 0.1, 5, 0)
    lb, gb = step.forward_backward(as_bf16, glob, toks, sh, alpha, 0.1, 5, 0)
    assert la == lb
    for x, y in zip(ga, gb):
        for proj in block.PROJS:
            assert np.array_equal(x[proj][0], y[proj][0]) and np.array_equal(x[proj][1], y[proj][1])

    bl = [block.bf16_params(mi.block_params(0, 90, li, sh, mi.LoraSpec(4, alpha, 0.1), w_std=0.2))
          for li in range(sh.layers)]
    for d in bl:
        for proj in block.PROJS:
            d[proj]["B"] = (d[proj]["B"] * 30).astype(np.float32)
    loss, grads = step.forward_backward(bl, glob, toks, sh, alpha, 0.1, 5, 0)
    h = 1e-6
    for li, proj, name, idx in [(0, "v", "A", (1, 3)), (1, "down", "B", (5, 2))]:
        def with_delta(dlt):
            ls = [{k: (dict(v) if isinstance(v, dict) else v) for k, v in d.items()} for d in bl]
            arr = bl[li][proj][name].astype(np.float64).copy()
            arr[idx] += dlt
            ls[li][proj][name] = arr
            return step.forward_backward(ls, glob, toks, sh, alpha, 0.1, 5, 0)[0]
        g = grads[li][proj][0 if name == "A" else 1][idx]
        fd = (with_delta(h) - with_delta(-h)) / (2 * h)
        assert abs(fd - g) <= 1e-6 * max(1e-3, abs(fd)) + 1e-9, (li, proj, name, fd, g)
