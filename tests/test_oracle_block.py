"""Pins for the oracle's Qwen2.5-shaped block (CPU only): library routines for
sub-steps, closed-form special cases, finite differences."""
import numpy as np
import torch

import msq_inputs as mi
from oracle import block, lora, nf4

SH = mi.BlockShape(hidden=64, heads=2, kv_heads=1, head_dim=32, inter=128)


def _params(w_std=0.2, seed=0, r=4):
    p = mi.block_params(seed, 77, 0, SH, mi.LoraSpec(r, 8.0, 0.2), w_std=w_std)
    for proj in block.PROJS:
        p[proj]["B"] = (p[proj]["B"] * 30).astype(np.float32)  # make the LoRA branch visible
    return block.quantize_params(p)


def test_rmsnorm_matches_torch():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5, 64))
    w = 1 + 0.1 * rng.standard_normal(64)
    y, _ = block.rmsnorm(x, w)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (64,), torch.from_numpy(w), eps=1e-6)
    assert np.allclose(y, ref.numpy(), rtol=1e-13, atol=1e-13)


def test_attention_matches_torch_sdpa():
    rng = np.random.default_rng(1)
    T, H, KV, D = 7, 4, 2, 16
    q = rng.standard_normal((T, H, D))
    k = rng.standard_normal((T, KV, D))
    v = rng.standard_normal((T, KV, D))
    out, _ = block.attention(q, k, v, H, KV)
    tq = torch.from_numpy(q).permute(1, 0, 2)
    tk = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(H // KV, dim=0)
    tv = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(H // KV, dim=0)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True)
    assert np.allclose(out, ref.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-12)


def test_single_token_attention_returns_v():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((1, 4, 8))
    k = rng.standard_normal((1, 2, 8))
    v = rng.standard_normal((1, 2, 8))
    out, _ = block.attention(q, k, v, 4, 2)
    assert np.allclose(out[0, :2], v[0, 0]) and np.allclose(out[0, 2:], v[0, 1])


def test_rope_position_zero_is_identity_and_preserves_pair_norms():
    cos, sin = block.rope_tables(6, 16)
    rng = np.random.default_rng(3)
    x = rng.standard_normal((6, 2, 16))
    y = block.rope(x, cos, sin)
    assert np.array_equal(y[0], x[0])
    n_in = x[..., :8] ** 2 + x[..., 8:] ** 2
    n_out = y[..., :8] ** 2 + y[..., 8:] ** 2
    assert np.allclose(n_in, n_out, rtol=1e-12)
    # angle of pair i at position t is t * theta^(-2i/D)
    t, i = 5, 3
    ang = t * 1e6 ** (-2 * i / 16)
    assert np.isclose(cos[t, i], np.cos(ang)) and np.isclose(sin[t, 8 + i], np.sin(ang))


def test_block_finite_differences():
    qp = _params()
    io = mi.block_io(0, 77, SH, 8)
    x = io["x"].astype(np.float64)
    dy = io["dy"].astype(np.float64)
    alpha, p = 8.0, 0.2
    rk = lora.RngKey(seed=5, step=3)
    out, cache = block.forward(x, qp, SH, 1, alpha, p, rk)
    dx, grads = block.backward(dy, cache, qp, SH, 1, alpha, p, rk)

    def loss(xx, q2):
        o, _ = block.forward(xx, q2, SH, 1, alpha, p, rk)
        return float(np.sum(o * dy))

    h = 1e-6
    rng = np.random.default_rng(4)
    for _ in range(6):
        idx = (int(rng.integers(0, 8)), int(rng.integers(0, 64)))
        xp, xm = x.copy(), x.copy()
        xp[idx] += h
        xm[idx] -= h
        fd = (loss(xp, qp) - loss(xm, qp)) / (2 * h)
        assert abs(fd - dx[idx]) <= 1e-6 * max(1.0, abs(fd)), ("x", idx, fd, dx[idx])
    for proj in block.PROJS:
        for which in (0, 1):
            name = "A" if which == 0 else "B"
            g = grads[proj][which]
            for _ in range(3):
                idx = tuple(int(rng.integers(0, s)) for s in g.shape)
                qpp = {k: (dict(v) if isinstance(v, dict) else v) for k, v in qp.items()}
                qpm = {k: (dict(v) if isinstance(v, dict) else v) for k, v in qp.items()}
                ap = qp[proj][name].astype(np.float64).copy()
                am = ap.copy()
                ap[idx] += h
                am[idx] -= h
                qpp[proj][name] = ap
                qpm[proj][name] = am
                fd = (loss(x, qpp) - loss(x, qpm)) / (2 * h)
                assert abs(fd - g[idx]) <= 1e-6 * max(1.0, abs(fd)), (proj, name, idx, fd, g[idx])


def test_block_dropout_replay_and_zero_dropout():
    qp = _params()
    io = mi.block_io(1, 77, SH, 8)
    rk = lora.RngKey(seed=5, step=3)
    o1, _ = block.forward(io["x"], qp, SH, 2, 8.0, 0.2, rk)
    o2, _ = block.forward(io["x"], qp, SH, 2, 8.0, 0.2, rk)
    assert np.array_equal(o1, o2)
    o3, _ = block.forward(io["x"], qp, SH, 2, 8.0, 0.2, lora.RngKey(seed=5, step=4))
    assert not np.array_equal(o1, o3)
    z1, _ = block.forward(io["x"], qp, SH, 2, 8.0, 0.0, rk)
    z2, _ = block.forward(io["x"], qp, SH, 2, 8.0, 0.0, lora.RngKey(seed=6, step=4))
    assert np.array_equal(z1, z2)
