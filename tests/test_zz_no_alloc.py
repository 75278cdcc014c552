"""nf4_lora_fwd_noalloc: the forward with the library's static per-GPU scratch in place of
a caller workspace (for callers that cannot allocate).  Called through the C ABI and
compared with nf4_lora_fwd on the same inputs: two calls in a row, the second smaller,
so the second runs on scratch the first left behind.  Both run the same kernels with
the same plan, so the outputs must agree bit for bit (stronger than the 2e-2*RMS bar,
which is checked too, against the oracle, on the small call)."""
import ctypes

import numpy as np
import pytest
import torch

import msq_inputs as mi
from oracle import lora as olora
from oracle import nf4 as onf4

from gpu_util import assert_parity, dev_bf16, host_f64

abi = pytest.importorskip("memory_streamed_qlora_amd._abi")
msq = pytest.importorskip("memory_streamed_qlora_amd")


def _p(t):
    return None if t is None else t.data_ptr()


def test_noalloc_rejects_shapes_beyond_the_scratch_on_the_host():
    """No GPU needed: the size check comes before any HIP call."""
    L = abi.lib()
    FAKE = 0x10000
    need = L.nf4_lora_workspace_size(65535, 29568, 29568, 16)
    assert need > (128 << 20)
    rc = L.nf4_lora_fwd_noalloc(FAKE, 65535, 29568, 29568, FAKE, FAKE, None, None, FAKE, FAKE,
                                abi.LoraCfg(16, 32.0, 0.0, 0), abi.RngKey(0, 0, 0, 0, 0), FAKE, None, None)
    assert rc == abi.MSQ_E_WORKSPACE
    assert "static" in L.msq_last_error().decode()
    # an invalid shape is reported as nf4_lora_fwd reports it
    rc = L.nf4_lora_fwd_noalloc(FAKE, 8, 96, 64, FAKE, FAKE, None, None, FAKE, FAKE,
                                abi.LoraCfg(16, 32.0, 0.0, 0), abi.RngKey(0, 0, 0, 0, 0), FAKE, None, None)
    assert rc == abi.MSQ_E_SHAPE


def _case(T, K, N, p, act_f32, seed):
    lo = mi.LoraSpec(16, 32.0, p)
    inp = mi.linear_inputs(seed, 97, 0, "q", K, N, T, lo, with_bias=True)
    codes, absmax = msq.nf4_quantize(dev_bf16(inp["W"]))
    x = dev_bf16(inp["x"])
    res = dev_bf16(inp["dy"])  # any [T, N] tensor in y's type serves as the residual
    if act_f32:
        x, res = x.float(), res.float()
    A = torch.from_numpy(inp["A"]).cuda()
    B = torch.from_numpy(inp["B"]).cuda()
    bias = dev_bf16(inp["bias"])
    flags = (abi.MSQ_ACT_F32 | abi.MSQ_OUT_F32) if act_f32 else 0
    cfg = abi.LoraCfg(16, 32.0, p, flags)
    key = abi.RngKey(11, 3, 0, 5, 4)
    return inp, codes, absmax, x, res, A, B, bias, cfg, key


@pytest.mark.gpu
def test_noalloc_forward_equals_workspace_forward_two_calls():
    L = abi.lib()
    stream = torch.cuda.current_stream().cuda_stream
    # call 1: a split plan (q/o of the 32B shape) with dropout, bias and residual; call 2:
    # a smaller single-pass shape with fp32 activations, on the scratch call 1 left behind
    for T, K, N, p, f32 in ((512, 5120, 5120, 0.1, False), (200, 896, 896, 0.2, True)):
        print(f"noalloc case T={T} K={K} N={N} p={p} fp32={f32}", flush=True)
        inp, codes, absmax, x, res, A, B, bias, cfg, key = _case(T, K, N, p, f32, seed=T)
        dt = x.dtype
        y_ref = torch.empty(T, N, dtype=dt, device="cuda")
        u_ref = torch.empty(T, 16, dtype=torch.float32, device="cuda")
        need = L.nf4_lora_workspace_size(T, K, N, 16)
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        assert L.nf4_lora_fwd(_p(x), T, K, N, _p(codes), _p(absmax), _p(bias), _p(res), _p(A), _p(B), cfg, key,
                              _p(y_ref), _p(u_ref), _p(ws), need, stream) == 0
        y = torch.full((T, N), 7.0, dtype=dt, device="cuda")
        u = torch.full((T, 16), 7.0, dtype=torch.float32, device="cuda")
        rc = L.nf4_lora_fwd_noalloc(_p(x), T, K, N, _p(codes), _p(absmax), _p(bias), _p(res), _p(A), _p(B), cfg,
                                    key, _p(y), _p(u), stream)
        assert rc == 0, L.msq_last_error().decode()
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref), "y differs from nf4_lora_fwd"
        assert torch.equal(u, u_ref), "u differs from nf4_lora_fwd"
        assert_parity(host_f64(y), host_f64(y_ref), name="y")
        if T == 200:  # small enough for the oracle
            oc, oa = onf4.quantize(inp["W"])
            rk = olora.RngKey(seed=11, step=3, micro=0, layer=5, proj=4)
            ry, ru = olora.fwd(inp["x"], oc, oa, inp["bias"], inp["A"], inp["B"], 32.0, p, rk)
            assert_parity(host_f64(y) - host_f64(res), ry, name="y vs oracle")
            assert_parity(host_f64(u), ru, name="u vs oracle")
