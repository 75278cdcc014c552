"""GPU parity of the optimizer step (msq_adamw_step) against the oracle's AdamW (float64)."""
import numpy as np
import pytest
import torch

from oracle import step as ostep

pytestmark = pytest.mark.gpu
msq = pytest.importorskip("memory_streamed_qlora_amd")

LR, BETAS, EPS, WD = ostep.LR, (ostep.BETA1, ostep.BETA2), ostep.ADAM_EPS, ostep.WD
U = 2.0 ** -24  # fp32 unit roundoff


def _tensors(seed, sizes):
    rng = np.random.default_rng(seed)
    p = [rng.uniform(-0.05, 0.05, n).astype(np.float32) for n in sizes]
    return p, rng


def test_adamw_steps_match_the_oracle():
    """Five steps over 19 tensors (more than one launch's 16; sizes ragged, below and above a
    workgroup's 8192 elements, one empty), gradients spanning 1e-8 .. 1 with exact zeros:
    parameters within a few fp32 roundings of the float64 update, moments to 1e-6
    relative, and the partial sums of g^2 summing to the float64 squared norm."""
    sizes = [1, 3, 4, 5, 63, 64, 8191, 8192, 8193, 20000, 0, 81920, 16 * 5120 + 7, 16, 100, 4097, 12345, 2, 8]
    p_np, rng = _tensors(0, sizes)
    dev = [torch.from_numpy(x.copy()).cuda() for x in p_np]
    m_d = [torch.zeros_like(x) for x in dev]
    v_d = [torch.zeros_like(x) for x in dev]
    p64 = [x.astype(np.float64) for x in p_np]
    m64 = [np.zeros(n) for n in sizes]
    v64 = [np.zeros(n) for n in sizes]
    n_part = msq.adamw_partials(dev)
    assert n_part == sum(-(-n // 8192) for n in sizes)
    for t in range(1, 6):
        g_np = []
        for n in sizes:
            g = (rng.standard_normal(n) * 10.0 ** rng.uniform(-8, 0, n)).astype(np.float32)
            g[rng.random(n) < 0.05] = 0.0
            g_np.append(g)
        g_d = [torch.from_numpy(g).cuda() for g in g_np]
        gsq = torch.full((n_part,), float("nan"), device="cuda")
        msq.adamw_step(dev, g_d, m_d, v_d, t, LR, BETAS, EPS, WD, gsq=gsq)
        torch.cuda.synchronize()
        for i in range(len(sizes)):
            # the oracle steps from the GPU's own previous state (fp32 values, exact in f64)
            p_prev, m_prev, v_prev = p64[i], m64[i], v64[i]
            rp, rm, rv = ostep.adamw(p_prev, g_np[i].astype(np.float64), m_prev, v_prev, t)
            gp = dev[i].cpu().numpy().astype(np.float64)
            gm = m_d[i].cpu().numpy().astype(np.float64)
            gv = v_d[i].cpu().numpy().astype(np.float64)
            if sizes[i]:
                g64 = np.abs(g_np[i].astype(np.float64))
                # a few fp32 roundings of the terms (the sums may cancel, so the bound is on
                # the terms, not on the result)
                tol_m = 4 * U * (BETAS[0] * np.abs(m_prev) + (1 - BETAS[0]) * g64) + 1e-45
                assert np.all(np.abs(gm - rm) <= tol_m), f"tensor {i} step {t}: m"
                assert np.all(np.abs(gv - rv) <= 6 * U * np.abs(rv) + 1e-45), f"tensor {i} step {t}: v"
                tol_p = 4 * U * (np.abs(p_prev) + np.abs(rp)) + 1e-5 * LR
                assert np.all(np.abs(gp - rp) <= tol_p), f"tensor {i} step {t}: p off by {np.max(np.abs(gp - rp))}"
            p64[i], m64[i], v64[i] = gp, gm, gv
        want = sum(float(np.sum(g.astype(np.float64) ** 2)) for g in g_np)
        got = float(gsq.double().sum())
        assert not torch.isnan(gsq).any()
        assert abs(got - want) <= 1e-5 * want


def test_adamw_is_deterministic_and_tracks_torch():
    """Two runs give the same bits; over 20 steps the parameters stay within 1e-6 of
    torch.optim.AdamW's (same hyperparameters)."""
    n = 3 * 8192 + 77
    rng = np.random.default_rng(3)
    p0 = rng.uniform(-0.05, 0.05, n).astype(np.float32)
    gs = [(rng.standard_normal(n) * 1e-3).astype(np.float32) for _ in range(20)]

    def run():
        p = torch.from_numpy(p0.copy()).cuda()
        m, v = torch.zeros_like(p), torch.zeros_like(p)
        gsq = torch.zeros(msq.adamw_partials([p]), device="cuda")
        for t, g in enumerate(gs, 1):
            msq.adamw_step([p], [torch.from_numpy(g).cuda()], [m], [v], t, LR, BETAS, EPS, WD, gsq=gsq)
        torch.cuda.synchronize()
        return p, m, v, gsq

    a, b = run(), run()
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    tp = torch.nn.Parameter(torch.from_numpy(p0.copy()).cuda())
    opt = torch.optim.AdamW([tp], lr=LR, betas=BETAS, eps=EPS, weight_decay=WD)
    for g in gs:
        tp.grad = torch.from_numpy(g).cuda()
        opt.step()
    torch.cuda.synchronize()
    assert torch.max(torch.abs(tp.detach() - a[0])).item() <= 1e-6
