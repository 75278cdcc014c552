"""GPU parity against the oracle where the earlier tests did not reach:

  * every projection launch of the Qwen2.5-7B and -72B shapes (grouped q+k+v, o, grouped
    gate+up, down) at 512 tokens with dropout 0.1, forward and backward, in the launch
    configuration the stack uses.  The oracle evaluates sampled output columns (y) and
    input columns (dx) one by one, and u, dA, dB whole (they are small);
  * 1000 tokens (a second, partial 512-row tile), single and grouped, forward and
    backward, dropout 0.1;
  * the exact-integer case on split plans (K = N = 5120: the reduction is split over
    several workgroups and summed by the split reduction) and on grouped launches: every
    product and sum is exact in fp32, so the GPU must equal the oracle after the one final
    rounding, bit for bit;
  * the dropout masks bit for bit: with A = I (r = K = 64) and B = 0, u = drop(x) exactly,
    so u must equal fp32(x * sigma) where the oracle keeps and 0 where it drops; with W = 0,
    B = I and alpha = r the backward's dx is sigma * keep (.) dy, which checks the mask the
    backward GEMM replays.  Single and grouped, p in {0.1, 0.5}.
Bar: max |gpu - ref| <= 2e-2 * RMS(ref) per tensor (on the sampled columns where sampled)."""
import numpy as np
import pytest
import torch

import msq_inputs as mi
from oracle import lora as olora
from oracle import nf4 as onf4
from oracle import philox as ophilox

from gpu_util import assert_parity, bf16_bits, dev_bf16, dev_f32, host_f64

pytestmark = pytest.mark.gpu
msq = pytest.importorskip("memory_streamed_qlora_amd")

PID = msq.ops.PROJ_ID


def _host_bf16(t: torch.Tensor) -> np.ndarray:
    """Device bf16 tensor -> float32 values on the host (exact)."""
    return t.float().cpu().numpy()


def _deq_rows(W_dev: torch.Tensor, rows: np.ndarray) -> np.ndarray:
    """The oracle's dequantized rows of W (its own quantization of those rows)."""
    w = _host_bf16(W_dev[torch.from_numpy(rows).cuda()])
    c, a = onf4.quantize(w)
    return onf4.dequantize(c, a)


def _deq_cols(W_dev: torch.Tensor, cols: np.ndarray) -> np.ndarray:
    """The oracle's dequantized columns of W: each column's 64-element quantization block
    (whole, as in the full matrix: blocks never straddle a row) quantized and dequantized."""
    blocks = np.unique(cols // 64)
    idx = (blocks[:, None] * 64 + np.arange(64)[None, :]).reshape(-1)
    w = _host_bf16(W_dev[:, torch.from_numpy(idx).cuda()])
    c, a = onf4.quantize(w)
    deq = onf4.dequantize(c, a)
    pos = {b: i for i, b in enumerate(blocks)}
    return deq[:, [pos[c_ // 64] * 64 + c_ % 64 for c_ in cols]]


def _sample(n: int, count: int, rng) -> np.ndarray:
    pick = rng.choice(n, size=min(count, n), replace=False)
    return np.unique(np.concatenate([pick, [0, n - 1]])).astype(np.int64)


def _launch_case(shape, names, seed, T=512, p=0.1, samples=32):
    """One launch of the stack's: projections `names` of one input (a group when more than
    one), forward then backward, against the oracle on sampled columns."""
    K = shape.proj_shape(names[0])[0]
    lo = mi.LoraSpec(16, 32.0, p)
    rng = np.random.default_rng(seed)
    x = mi.normal_bf16(mi.rng_for(seed, 5, 0, 900), (T, K), 1.0)
    projs, host = [], []
    for nm in names:
        N = shape.proj_shape(nm)[1]
        pid = PID[nm]
        W = mi.device_normal_bf16(seed, 5, 0, 16 * pid + mi.T_W, (N, K), 0.02, "cuda")
        A = mi.uniform_f32(mi.rng_for(seed, 5, 0, 16 * pid + mi.T_A), (16, K), 1.0 / np.sqrt(K))
        B = mi.normal_f32(mi.rng_for(seed, 5, 0, 16 * pid + mi.T_B), (N, 16), 0.01)
        bias = mi.normal_bf16(mi.rng_for(seed, 5, 0, 16 * pid + mi.T_BIAS), (N,), 0.02) if nm in ("q", "k", "v") else None
        dy = mi.normal_bf16(mi.rng_for(seed, 5, 0, 16 * pid + mi.T_DY), (T, N), 1.0)
        key = olora.RngKey(seed=seed, step=2, layer=7, proj=pid)
        projs.append({"base": msq.nf4_quantize(W), "bias": dev_bf16(bias) if bias is not None else None,
                      "A": dev_f32(A), "B": dev_f32(B), "key": msq.rng_key(seed, 2, 0, 7, pid)})
        host.append(dict(W=W, A=A, B=B, bias=bias, dy=dy, key=key, N=N))
    cfg = msq.Lora(16, 32.0, p)
    xd = dev_bf16(x)
    if len(names) > 1:
        outs = msq.lora_fwd_group(xd, projs, cfg)
        gp = [{"base": pr["base"], "A": pr["A"], "B": pr["B"], "key": pr["key"], "dy": dev_bf16(h["dy"]), "u": u}
              for pr, h, (_, u) in zip(projs, host, outs)]
        dx, dAB = msq.lora_bwd_group(xd, gp, cfg)
    else:
        pr, h = projs[0], host[0]
        y, u = msq.nf4_lora_fwd(xd, pr["base"][0], pr["base"][1], pr["bias"], pr["A"], pr["B"], cfg, pr["key"],
                                path="tiled")
        outs = [(y, u)]
        dx, dA, dB = msq.nf4_lora_bwd(dev_bf16(h["dy"]), xd, pr["base"][0], pr["base"][1], pr["A"], pr["B"], cfg,
                                      pr["key"], u=u, path="tiled")
        dAB = [(dA, dB)]
    torch.cuda.synchronize()
    kcols = _sample(K, samples, rng)
    rdx = np.zeros((T, kcols.size))
    ratios = {}
    for nm, h, (y, u), (dA, dB) in zip(names, host, outs, dAB):
        ncols = _sample(h["N"], samples, rng)
        Wr = _deq_rows(h["W"], ncols)
        ry, ru = olora.fwd_dense(x, Wr, h["bias"][ncols] if h["bias"] is not None else None, h["A"],
                                 h["B"][ncols], 32.0, p, h["key"])
        ratios[nm + ".y"] = assert_parity(host_f64(y)[:, ncols], ry, name=f"{nm} y (sampled)")
        ratios[nm + ".u"] = assert_parity(host_f64(u), ru, name=f"{nm} u")
        Wc = _deq_cols(h["W"], kcols)
        rdx_p, rdA, rdB = olora.bwd_dense(h["dy"], x, Wc, h["A"], h["B"], 32.0, p, h["key"], dx_cols=kcols)
        rdx += rdx_p
        ratios[nm + ".dA"] = assert_parity(host_f64(dA), rdA, name=f"{nm} dA")
        ratios[nm + ".dB"] = assert_parity(host_f64(dB), rdB, name=f"{nm} dB")
        del h["W"]
    ratios["dx"] = assert_parity(host_f64(dx)[:, kcols], rdx, name="+".join(names) + " dx (sampled)")
    print("+".join(names), {k: f"{v:.2e}" for k, v in ratios.items()}, flush=True)


LAUNCHES = [("q", "k", "v"), ("o",), ("gate", "up"), ("down",)]


@pytest.mark.parametrize("names", LAUNCHES, ids=["qkv", "o", "gate_up", "down"])
def test_qwen7b_launch_shapes_dropout(names):
    print(f"7B {names}", flush=True)
    _launch_case(mi.QWEN25_7B, names, seed=7)


@pytest.mark.parametrize("names", LAUNCHES, ids=["qkv", "o", "gate_up", "down"])
def test_qwen72b_launch_shapes_dropout(names):
    print(f"72B {names}", flush=True)
    _launch_case(mi.QWEN25_72B, names, seed=72)


@pytest.mark.parametrize("names", LAUNCHES, ids=["qkv", "o", "gate_up", "down"])
def test_qwen32b_launch_shapes_dropout(names):
    print(f"32B {names}", flush=True)
    _launch_case(mi.QWEN25_32B, names, seed=32)


# ---- 1000 tokens: a second, partial row tile ----------------------------------------------

SMALL = mi.BlockShape(hidden=1024, heads=8, kv_heads=2, head_dim=128, inter=1536)


@pytest.mark.parametrize("names", LAUNCHES, ids=["qkv", "o", "gate_up", "down"])
def test_thousand_tokens(names):
    print(f"T=1000 {names}", flush=True)
    _launch_case(SMALL, names, seed=1000, T=1000, samples=4096)   # every column at these sizes


# ---- exact-integer case on split plans and grouped launches --------------------------------

def _int_weights(rng, N, K):
    e = rng.integers(-2, 2, size=(N, K // 64))
    sgn = rng.integers(-1, 2, size=(N, K)).astype(np.float32)
    sgn[:, ::64] = 1.0
    return (sgn * np.repeat(2.0 ** e, 64, axis=1)).astype(np.float32)


@pytest.mark.parametrize("ns", [(5120,), (5120, 1024, 1024)], ids=["single_split", "grouped_qkv"])
def test_exact_integer_split_and_grouped_bitwise(ns):
    """T 512, K 5120: x in [-2, 2], W in {-1, 0, 1} * 2^e (e in [-2, 1]), A, B, dy in
    {-1, 0, 1}.  Every partial sum stays below 2^24 in units of 2^-2, so fp32 sums are exact
    in any order; the outputs are the exact values after the final rounding (bf16 y and dx)
    or exactly (u, dA, dB)."""
    rng = np.random.default_rng(51)
    T, K, r = 512, 5120, 16
    x = rng.integers(-2, 3, size=(T, K)).astype(np.float32)
    projs, host = [], []
    for i, N in enumerate(ns):
        W = _int_weights(rng, N, K)
        A = rng.integers(-1, 2, size=(r, K)).astype(np.float32)
        B = rng.integers(-1, 2, size=(N, r)).astype(np.float32)
        dy = rng.integers(-1, 2, size=(T, N)).astype(np.float32)
        codes, a = onf4.quantize(W)
        assert np.array_equal(onf4.dequantize(codes, a), W)
        projs.append({"base": (torch.from_numpy(codes).cuda(), dev_f32(a)), "bias": None, "A": dev_f32(A),
                      "B": dev_f32(B), "key": msq.rng_key(0, 0, 0, 0, i)})
        host.append((codes, a, A, B, dy))
    cfg = msq.Lora(r, 32.0, 0.0)
    xd = dev_bf16(x)
    if len(ns) == 1:
        pr = projs[0]
        y, u = msq.nf4_lora_fwd(xd, pr["base"][0], pr["base"][1], None, pr["A"], pr["B"], cfg, pr["key"],
                                path="tiled")
        outs = [(y, u)]
        dx, dA, dB = msq.nf4_lora_bwd(dev_bf16(host[0][4]), xd, pr["base"][0], pr["base"][1], pr["A"], pr["B"],
                                      cfg, pr["key"], u=u, path="tiled")
        dAB = [(dA, dB)]
    else:
        outs = msq.lora_fwd_group(xd, projs, cfg)
        gp = [{"base": pr["base"], "A": pr["A"], "B": pr["B"], "key": pr["key"], "dy": dev_bf16(h[4]), "u": u}
              for pr, h, (_, u) in zip(projs, host, outs)]
        dx, dAB = msq.lora_bwd_group(xd, gp, cfg)
    torch.cuda.synchronize()
    rdx = 0.0
    for (codes, a, A, B, dy), (y, u), (dA, dB) in zip(host, outs, dAB):
        ry, ru = olora.fwd(x, codes, a, None, A, B, 32.0, 0.0, olora.RngKey())
        rdx_i, rdA, rdB = olora.bwd(dy, x, codes, a, A, B, 32.0, 0.0, olora.RngKey())
        rdx = rdx + rdx_i
        assert np.array_equal(bf16_bits(y), onf4.bf16_to_bits(onf4.bf16_round(ry.astype(np.float32))))
        assert np.array_equal(u.cpu().numpy().astype(np.float64), ru)
        assert np.array_equal(dA.cpu().numpy().astype(np.float64), rdA)
        assert np.array_equal(dB.cpu().numpy().astype(np.float64), rdB)
    assert np.max(np.abs(rdx)) < 2 ** 22
    assert np.array_equal(bf16_bits(dx), onf4.bf16_to_bits(onf4.bf16_round(np.asarray(rdx, np.float32))))


# ---- the dropout masks, bit for bit --------------------------------------------------------

def _expected_drop(x: np.ndarray, p: float, key: olora.RngKey) -> np.ndarray:
    """fp32(x * sigma) where the oracle's mask keeps, 0 where it drops (one fp32 rounding of
    the exact product, which is what a single fp32 multiply gives)."""
    keep = ophilox.keep_mask(x.shape[0], x.shape[1], p, key.seed, key.layer, key.proj, key.step, key.micro)
    sigma = float(ophilox.drop_scale(p))
    return np.where(keep, (x.astype(np.float64) * sigma).astype(np.float32), np.float32(0.0))


@pytest.mark.parametrize("p", [0.1, 0.5])
@pytest.mark.parametrize("n_proj", [1, 3])
def test_dropout_masks_bit_exact(p, n_proj):
    T, K, r = 300, 64, 64
    rng = np.random.default_rng(int(p * 10) + n_proj)
    x = mi.normal_bf16(rng, (T, K), 1.0)
    eye = dev_f32(np.eye(64, dtype=np.float32))
    zero_w = msq.nf4_quantize(torch.zeros(64, K, dtype=torch.bfloat16, device="cuda"))
    keys = [olora.RngKey(seed=123 + 7 * i, step=9, micro=1, layer=41, proj=(i + 4) % 7) for i in range(n_proj)]
    dkeys = [msq.rng_key(k.seed, k.step, k.micro, k.layer, k.proj) for k in keys]
    cfg = msq.Lora(r, float(r), p)                                   # alpha = r: s = 1
    zeros_B = torch.zeros(64, r, device="cuda")
    xd = dev_bf16(x)
    # forward: u = drop(x) A^T with A = I
    if n_proj == 1:
        _, u = msq.nf4_lora_fwd(xd, zero_w[0], zero_w[1], None, eye, zeros_B, cfg, dkeys[0])
        us = [u]
    else:
        outs = msq.lora_fwd_group(xd, [{"base": zero_w, "bias": None, "A": eye, "B": zeros_B, "key": k}
                                       for k in dkeys], cfg)
        us = [u for _, u in outs]
    torch.cuda.synchronize()
    for i, (u, k) in enumerate(zip(us, keys)):
        want = _expected_drop(x, p, k)
        got = u.cpu().numpy()
        # value equality: every kept value bit for bit, every dropped one zero (of either sign)
        assert np.array_equal(got, want), f"projection {i}: u != drop(x)"
        kept = np.mean(want != 0)
        assert abs(kept - (1 - p)) < 5 * np.sqrt(p * (1 - p) / want.size) + 0.01
    # backward: W = 0, B = I, A = I, alpha = r: dx = sigma * keep (.) dy (fp32 output); in a
    # group only projection j's dy is non-zero, so dx is its term alone
    dy = mi.normal_bf16(rng, (T, 64), 1.0)
    for j in range(n_proj):
        if n_proj == 1:
            dx, _, _ = msq.nf4_lora_bwd(dev_bf16(dy), xd, zero_w[0], zero_w[1], eye, eye, cfg, dkeys[0],
                                        out_dtype=torch.float32)
        else:
            gp = [{"base": zero_w, "A": eye, "B": eye, "key": k,
                   "dy": dev_bf16(dy if i == j else np.zeros_like(dy))} for i, k in enumerate(dkeys)]
            dx, _ = msq.lora_bwd_group(xd, gp, cfg, out_dtype=torch.float32)
        torch.cuda.synchronize()
        want = _expected_drop(dy, p, keys[j])
        got = dx.cpu().numpy()
        assert np.array_equal(got, want), f"projection {j}: dx != sigma keep dy"
