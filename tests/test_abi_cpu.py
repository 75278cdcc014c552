"""C-ABI checks that need no GPU: the library loads, exports every symbol the header
declares, its host-computed codebook equals the oracle's, and invalid arguments are
rejected on the host before any HIP call (fake, never-dereferenced addresses)."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "msq.h")

abi = pytest.importorskip("memory_streamed_qlora_amd._abi")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(",
                       src, flags=re.M)
    return sorted(set(names))


def test_library_exports_every_declared_symbol():
    lib = abi.lib()
    declared = _declared_functions()
    assert len(declared) >= 17
    for name in declared:
        assert hasattr(lib, name), name
    assert set(declared) == set(abi.EXPORTED)
    header = open(os.path.join(ROOT, "include", "msq.h")).read()
    assert lib.msq_abi_version() == int(re.search(r"#define MSQ_ABI_VERSION (\d+)", header).group(1))
    assert lib.msq_abi_version() == abi.ABI_VERSION


def test_host_codebook_equals_oracle():
    from oracle import nf4
    out = (ctypes.c_float * 16)()
    assert abi.lib().msq_nf4_codebook(out) == 0
    got = np.frombuffer(out, dtype=np.float32)
    assert np.array_equal(got.view(np.uint32), nf4.codebook().view(np.uint32))


FAKE = 0x10000  # 256-byte aligned, never dereferenced: every call below fails validation first


def _err():
    return abi.lib().msq_last_error().decode()


def test_quantize_rejects_bad_arguments():
    L = abi.lib()
    assert L.nf4_quantize(FAKE, 4, 96, FAKE, FAKE, None) == abi.MSQ_E_SHAPE
    assert "multiple of 64" in _err()
    assert L.nf4_quantize(None, 4, 64, FAKE, FAKE, None) == abi.MSQ_E_INVAL
    assert L.nf4_quantize(FAKE, -1, 64, FAKE, FAKE, None) == abi.MSQ_E_INVAL
    assert L.nf4_quantize(FAKE + 2, 4, 64, FAKE, FAKE, None) == abi.MSQ_E_INVAL
    assert L.nf4_quantize(FAKE, 0, 64, FAKE, FAKE, None) == 0            # empty: no-op
    assert L.nf4_dequantize(FAKE, FAKE, 4, 32, FAKE, None) == abi.MSQ_E_SHAPE


def _fwd(t=8, k=128, n=128, r=16, alpha=32.0, p=0.0, ws=None, x=FAKE, proj=0, layer=0, bias=None):
    L = abi.lib()
    need = L.nf4_lora_workspace_size(t, k, n, r)
    return L.nf4_lora_fwd(x, t, k, n, FAKE, FAKE, bias, None, FAKE, FAKE, abi.LoraCfg(r, alpha, p),
                          abi.RngKey(0, 0, 0, layer, proj), FAKE, None, FAKE,
                          need if ws is None else ws, None)


def test_linear_rejects_bad_arguments():
    assert _fwd(k=96) == abi.MSQ_E_SHAPE
    assert _fwd(n=100) == abi.MSQ_E_SHAPE
    assert _fwd(r=65) == abi.MSQ_E_SHAPE
    assert _fwd(r=-1) == abi.MSQ_E_SHAPE
    assert _fwd(p=1.0) == abi.MSQ_E_DROPOUT
    assert _fwd(p=-0.1) == abi.MSQ_E_DROPOUT
    assert _fwd(p=float("nan")) == abi.MSQ_E_DROPOUT
    assert _fwd(alpha=float("inf")) == abi.MSQ_E_DROPOUT
    assert _fwd(ws=1024) == abi.MSQ_E_WORKSPACE
    assert _fwd(x=FAKE + 8) == abi.MSQ_E_INVAL
    assert _fwd(bias=FAKE + 2) == abi.MSQ_E_INVAL
    assert _fwd(proj=16) == abi.MSQ_E_INVAL
    assert _fwd(t=70000) == abi.MSQ_E_SHAPE
    assert _fwd(t=0) == 0                                                 # empty: no-op
    L = abi.lib()
    need = L.nf4_lora_workspace_size(8, 128, 128, 16)
    rc = L.nf4_lora_bwd(FAKE, FAKE, 8, 128, 128, FAKE, FAKE, FAKE, FAKE, abi.LoraCfg(16, 32.0, 0.0),
                        abi.RngKey(), None, FAKE, 2, FAKE, FAKE, 0, FAKE, need, None)
    assert rc == abi.MSQ_E_INVAL and "accumulate" in _err()
    rc = L.nf4_lora_bwd(FAKE, FAKE, 8, 128, 128, FAKE, FAKE, FAKE, FAKE, abi.LoraCfg(16, 32.0, 0.0),
                        abi.RngKey(), None, FAKE, 0, None, FAKE, 0, FAKE, need, None)
    assert rc == abi.MSQ_E_INVAL


def test_linear_rejects_bad_residual():
    L = abi.lib()
    need = L.nf4_lora_workspace_size(8, 128, 128, 16)
    args = lambda res, flags: (FAKE, 8, 128, 128, FAKE, FAKE, None, res, FAKE, FAKE,  # noqa: E731
                               abi.LoraCfg(16, 32.0, 0.0, flags), abi.RngKey(0, 0, 0, 0, 0), FAKE, FAKE,
                               FAKE, need, None)
    assert L.nf4_lora_fwd(*args(FAKE + 8, 0)) == abi.MSQ_E_INVAL
    assert "misaligned" in _err()
    assert L.nf4_lora_fwd(*args(FAKE, abi.MSQ_U_ONLY)) == abi.MSQ_E_INVAL
    assert "residual" in _err()


def test_path_flags():
    L = abi.lib()
    need = L.nf4_lora_workspace_size(8, 128, 128, 33)
    args = lambda r, flags: (FAKE, 8, 128, 128, FAKE, FAKE, None, None, FAKE, FAKE,  # noqa: E731
                             abi.LoraCfg(r, 32.0, 0.0, flags), abi.RngKey(0, 0, 0, 0, 0), FAKE, FAKE,
                             FAKE, need, None)
    assert L.nf4_lora_fwd(*args(16, abi.MSQ_PATH_TILED | abi.MSQ_PATH_SMALL)) == abi.MSQ_E_INVAL
    assert "together" in _err()
    assert L.nf4_lora_fwd(*args(33, abi.MSQ_PATH_SMALL)) == abi.MSQ_E_SHAPE
    assert "r <= 32" in _err()
    assert L.nf4_lora_fwd(*args(6, abi.MSQ_PATH_SMALL)) == abi.MSQ_E_SHAPE
    assert L.nf4_lora_fwd(*args(16, 64)) == abi.MSQ_E_INVAL                 # an unknown bit
    assert "unknown flags" in _err()
    key = abi.RngKey(0, 0, 0, 0, 0)
    one = (abi.LoraProj * 1)(abi.LoraProj(128, FAKE, FAKE, None, None, None, FAKE, FAKE, key, FAKE, None))
    gneed = L.lora_group_workspace_size(8, 128, one, 1, 16)
    assert L.lora_fwd_group(FAKE, 8, 128, one, 1, abi.LoraCfg(16, 32.0, 0.0, abi.MSQ_PATH_SMALL), FAKE, gneed,
                            None) == abi.MSQ_E_INVAL
    assert "tiled path" in _err()


def test_glue_rejects_bad_arguments():
    """The pointwise glue entries validate on the host; n == 0 / t == 0 is a no-op that
    touches no pointer."""
    L = abi.lib()
    assert L.msq_swiglu_fwd(None, None, 0, None, None) == 0
    assert L.msq_swiglu_bwd(None, None, None, 0, None, None, None) == 0
    assert L.msq_swiglu_fwd(FAKE, FAKE, -1, FAKE, None) == abi.MSQ_E_SHAPE
    assert L.msq_swiglu_fwd(FAKE, FAKE, (1 << 40) + 1, FAKE, None) == abi.MSQ_E_SHAPE
    assert L.msq_swiglu_fwd(FAKE, None, 8, FAKE, None) == abi.MSQ_E_INVAL
    assert L.msq_swiglu_fwd(FAKE, FAKE + 4, 8, FAKE, None) == abi.MSQ_E_INVAL
    assert "misaligned" in _err()
    assert L.msq_swiglu_bwd(FAKE, FAKE, FAKE, 8, FAKE, None, None) == abi.MSQ_E_INVAL
    for fn in (L.msq_rope_fwd, L.msq_rope_bwd):
        assert fn(None, None, None, 0, 1, 64, None, None) == 0
        assert fn(FAKE, FAKE, FAKE, 4, 2, 63, FAKE, None) == abi.MSQ_E_SHAPE
        assert fn(FAKE, FAKE, FAKE, 4, 0, 64, FAKE, None) == abi.MSQ_E_SHAPE
        assert fn(FAKE, FAKE, FAKE, -1, 2, 64, FAKE, None) == abi.MSQ_E_SHAPE
        assert fn(FAKE, FAKE, FAKE, 1 << 30, 1 << 10, 1 << 10, FAKE, None) == abi.MSQ_E_SHAPE
        assert fn(FAKE, None, FAKE, 4, 2, 64, FAKE, None) == abi.MSQ_E_INVAL
        assert fn(FAKE, FAKE, FAKE + 8, 4, 2, 64, FAKE, None) == abi.MSQ_E_INVAL
    assert L.msq_rmsnorm_apply_fwd(None, None, None, 0, 64, None, None) == 0
    assert L.msq_rmsnorm_apply_fwd(FAKE, FAKE, FAKE, 4, 6, FAKE, None) == abi.MSQ_E_SHAPE
    assert L.msq_rmsnorm_apply_fwd(FAKE, FAKE, FAKE, -1, 64, FAKE, None) == abi.MSQ_E_SHAPE
    assert L.msq_rmsnorm_apply_fwd(FAKE, FAKE + 2, FAKE, 4, 64, FAKE, None) == abi.MSQ_E_INVAL
    assert L.msq_rmsnorm_apply_bwd(FAKE, FAKE, FAKE, FAKE, 4, 64, FAKE, None, None) == abi.MSQ_E_INVAL
    assert L.msq_rmsnorm_apply_bwd(FAKE + 4, FAKE, FAKE, FAKE, 4, 64, FAKE, FAKE, None) == abi.MSQ_E_INVAL


def _adam_tensors(*specs):
    arr = (abi.AdamwTensor * len(specs))()
    for i, (p, g, m, v, n) in enumerate(specs):
        arr[i] = abi.AdamwTensor(p, g, m, v, n)
    return arr


def test_adamw_rejects_bad_arguments_and_counts_partials():
    """msq_adamw_step validates everything on the host (nothing below reaches a launch);
    msq_adamw_partials counts one partial per 8192 elements of each tensor."""
    L = abi.lib()
    cfg = abi.AdamwCfg(2e-4, 0.9, 0.999, 1e-8, 0.01)
    ok = _adam_tensors((FAKE, FAKE + 256, FAKE + 512, FAKE + 768, 8))
    assert L.msq_adamw_partials(_adam_tensors((0, 0, 0, 0, 8192), (0, 0, 0, 0, 8193), (0, 0, 0, 0, 0),
                                              (0, 0, 0, 0, 1)), 4) == 1 + 2 + 0 + 1
    assert L.msq_adamw_partials(_adam_tensors((0, 0, 0, 0, -1)), 1) == -1
    assert L.msq_adamw_partials(None, 0) == 0
    assert L.msq_adamw_step(None, 0, cfg, 1, None, None) == 0                   # nothing to do
    assert L.msq_adamw_step(_adam_tensors((None, None, None, None, 0)), 1, cfg, 1, None, None) == 0
    assert L.msq_adamw_step(ok, -1, cfg, 1, None, None) == abi.MSQ_E_INVAL
    assert L.msq_adamw_step(ok, 1, cfg, 0, None, None) == abi.MSQ_E_INVAL
    assert "step" in _err()
    for bad in (abi.AdamwCfg(-1.0, 0.9, 0.999, 1e-8, 0.01), abi.AdamwCfg(2e-4, 1.0, 0.999, 1e-8, 0.01),
                abi.AdamwCfg(2e-4, 0.9, -0.1, 1e-8, 0.01), abi.AdamwCfg(2e-4, 0.9, 0.999, 0.0, 0.01),
                abi.AdamwCfg(2e-4, 0.9, 0.999, 1e-8, -0.01), abi.AdamwCfg(float("nan"), 0.9, 0.999, 1e-8, 0.0)):
        assert L.msq_adamw_step(ok, 1, bad, 1, None, None) == abi.MSQ_E_INVAL
    assert L.msq_adamw_step(_adam_tensors((FAKE, FAKE, FAKE, FAKE, -4)), 1, cfg, 1, None, None) == abi.MSQ_E_INVAL
    assert L.msq_adamw_step(_adam_tensors((FAKE, None, FAKE, FAKE, 4)), 1, cfg, 1, None, None) == abi.MSQ_E_INVAL
    assert "null" in _err()
    assert L.msq_adamw_step(_adam_tensors((FAKE, FAKE, FAKE + 4, FAKE, 4)), 1, cfg, 1, None, None) == abi.MSQ_E_INVAL
    assert "misaligned" in _err()


def test_kernel_copy_rejects_bad_arguments():
    """Size, null, alignment and overlap are checked before any pointer is looked at."""
    L = abi.lib()
    assert L.msq_kernel_copy(None, None, 0, None) == 0
    assert L.msq_kernel_copy(None, FAKE, 16, None) == abi.MSQ_E_INVAL
    assert L.msq_kernel_copy(FAKE, FAKE + 4096, 24, None) == abi.MSQ_E_INVAL
    assert L.msq_kernel_copy(FAKE + 8, FAKE + 4096, 32, None) == abi.MSQ_E_INVAL
    assert "aligned" in _err()
    assert L.msq_kernel_copy(FAKE, FAKE + 16, 64, None) == abi.MSQ_E_INVAL
    assert "overlap" in _err()


def test_stream_load_rejects_bad_arguments():
    """The loader validates jobs and staging on the host before any HIP call."""
    L = abi.lib()
    assert L.nf4_stream_load_device_bytes(96, 4) == 0
    assert L.nf4_stream_load_device_bytes(128, 0) == 0
    dev_need = L.nf4_stream_load_device_bytes(128, 8)
    host_need = L.nf4_stream_load_host_bytes(128, 8)
    assert dev_need >= 2 * (8 * 128 * 2 + 8 * 64 + 8 * 2) and host_need >= 2 * 8 * 128 * 2
    jobs = (abi.QuantJob * 2)(abi.QuantJob(FAKE, 4, 128, FAKE, FAKE), abi.QuantJob(FAKE, 4, 96, FAKE, FAKE))
    assert L.nf4_stream_load(jobs, 2, 8, FAKE, dev_need, FAKE, host_need, 4, None) == abi.MSQ_E_SHAPE
    jobs[1] = abi.QuantJob(None, 4, 64, FAKE, FAKE)
    assert L.nf4_stream_load(jobs, 2, 8, FAKE, dev_need, FAKE, host_need, 4, None) == abi.MSQ_E_INVAL
    jobs[1] = abi.QuantJob(FAKE, 4, 64, FAKE, FAKE)
    assert L.nf4_stream_load(jobs, 2, 8, FAKE, dev_need - 1, FAKE, host_need, 4, None) == abi.MSQ_E_WORKSPACE
    assert L.nf4_stream_load(jobs, 2, 8, FAKE + 16, dev_need, FAKE, host_need, 4, None) == abi.MSQ_E_INVAL
    assert L.nf4_stream_load(jobs, 2, 8, FAKE, dev_need, FAKE, host_need, 0, None) == abi.MSQ_E_INVAL
    assert L.nf4_stream_load(jobs, 2, 0, FAKE, dev_need, FAKE, host_need, 4, None) == abi.MSQ_E_INVAL
    empty = (abi.QuantJob * 1)(abi.QuantJob(None, 0, 64, None, None))
    assert L.nf4_stream_load(empty, 1, 8, None, 0, None, 0, 4, None) == abi.MSQ_E_INVAL
    assert L.nf4_stream_load(None, 0, 8, None, 0, None, 0, 4, None) == 0


def test_group_rejects_bad_arguments():
    L = abi.lib()
    key = abi.RngKey(0, 0, 0, 0, 0)

    def proj(n=128, w=None, codes=FAKE, y=FAKE):
        return abi.LoraProj(n, codes, FAKE if codes else None, w, None, None, FAKE, FAKE, key, y, None)

    two = (abi.LoraProj * 2)(proj(), proj(n=64))
    need = L.lora_group_workspace_size(8, 128, two, 2, 16)
    assert need > 0
    cfg = abi.LoraCfg(16, 32.0, 0.0)
    assert L.lora_fwd_group(FAKE, 8, 128, two, 0, cfg, FAKE, need, None) == abi.MSQ_E_INVAL
    assert L.lora_fwd_group(FAKE, 8, 128, two, 4, cfg, FAKE, need, None) == abi.MSQ_E_INVAL
    assert L.lora_fwd_group(FAKE, 8, 128, two, 2, cfg, FAKE, need - 1, None) == abi.MSQ_E_WORKSPACE
    assert L.lora_fwd_group(FAKE, 8, 128, two, 2, abi.LoraCfg(16, 32.0, 0.0, abi.MSQ_U_ONLY), FAKE, need,
                            None) == abi.MSQ_E_INVAL
    mixed = (abi.LoraProj * 2)(proj(), proj(codes=None, w=FAKE))
    assert L.lora_fwd_group(FAKE, 8, 128, mixed, 2, cfg, FAKE, need, None) == abi.MSQ_E_INVAL
    assert "mixed" in _err()
    bad_n = (abi.LoraProj * 2)(proj(), proj(n=100))
    assert L.lora_group_workspace_size(8, 128, bad_n, 2, 16) == 0
    assert L.lora_fwd_group(FAKE, 8, 128, bad_n, 2, cfg, FAKE, need, None) == abi.MSQ_E_SHAPE
    no_y = (abi.LoraProj * 1)(proj(y=None))
    assert L.lora_fwd_group(FAKE, 8, 128, no_y, 1, cfg, FAKE, need, None) == abi.MSQ_E_INVAL


def test_group_bwd_rejects_bad_arguments():
    L = abi.lib()
    key = abi.RngKey(0, 0, 0, 0, 0)

    def proj(n=128, w=None, codes=FAKE, dy=FAKE, dA=FAKE):
        return abi.LoraProjGrad(n, codes, FAKE if codes else None, w, FAKE, FAKE, key, dy, None, dA, FAKE)

    two = (abi.LoraProjGrad * 2)(proj(), proj(n=64))
    need = L.lora_group_bwd_workspace_size(8, 128, two, 2, 16)
    assert need > 0
    cfg = abi.LoraCfg(16, 32.0, 0.0)

    def call(arr, n, c=cfg, ws=need, dx=FAKE, acc=0):
        return L.lora_bwd_group(FAKE, 8, 128, arr, n, c, dx, acc, 0, FAKE, ws, None)

    assert call(two, 0) == abi.MSQ_E_INVAL
    assert call(two, 4) == abi.MSQ_E_INVAL
    assert call(two, 2, ws=need - 1) == abi.MSQ_E_WORKSPACE
    assert call(two, 2, c=abi.LoraCfg(16, 32.0, 0.0, abi.MSQ_U_ONLY)) == abi.MSQ_E_INVAL
    assert call(two, 2, acc=2) == abi.MSQ_E_INVAL
    assert call(two, 2, dx=None) == abi.MSQ_E_INVAL
    assert call(two, 2, dx=FAKE + 8) == abi.MSQ_E_INVAL
    mixed = (abi.LoraProjGrad * 2)(proj(), proj(codes=None, w=FAKE))
    assert call(mixed, 2) == abi.MSQ_E_INVAL
    assert "mixed" in _err()
    bad_n = (abi.LoraProjGrad * 2)(proj(), proj(n=100))
    assert L.lora_group_bwd_workspace_size(8, 128, bad_n, 2, 16) == 0
    assert call(bad_n, 2) == abi.MSQ_E_SHAPE
    assert call((abi.LoraProjGrad * 1)(proj(dy=None)), 1) == abi.MSQ_E_INVAL
    assert call((abi.LoraProjGrad * 1)(proj(dA=None)), 1) == abi.MSQ_E_INVAL
    assert "dA" in _err()
    # r == 0 needs no adapters or gradient outputs
    bare = (abi.LoraProjGrad * 1)(abi.LoraProjGrad(128, FAKE, FAKE, None, None, None, key, FAKE, None, None, None))
    assert L.lora_group_bwd_workspace_size(8, 128, bare, 1, 0) > 0


def test_group_bwd_plan_has_a_split_per_projection():
    """Split i of a backward group adds projection i's LoRA term, so even a reduction of
    three k-steps (which a single projection would not split) is cut in three: the
    workspace holds three fp32 partial copies of dx."""
    L = abi.lib()
    key = abi.RngKey(0, 0, 0, 0, 0)
    t, k = 8, 128
    arr = (abi.LoraProjGrad * 3)(*[abi.LoraProjGrad(64, FAKE, FAKE, None, FAKE, FAKE, key, FAKE, None, FAKE, FAKE)
                                   for _ in range(3)])
    assert L.lora_group_bwd_workspace_size(t, k, arr, 3, 16) >= 3 * t * k * 4


def test_workspace_size_depends_on_shape_only():
    L = abi.lib()
    a = L.nf4_lora_workspace_size(512, 5120, 27648, 16)
    b = L.nf4_lora_workspace_size(512, 5120, 27648, 16)
    assert a == b > 512 * 27648 * 4
    assert L.nf4_lora_workspace_size(512, 100, 64, 16) == 0
    assert L.nf4_lora_workspace_size(0, 64, 64, 16) > 0


def test_window_rejects_small_arena_and_names_what_fits():
    L = abi.lib()
    n = 8
    ptrs = (ctypes.c_void_p * n)(*([FAKE] * n))
    sizes = (ctypes.c_size_t * n)(*([1000 * 256] * n))
    need = L.block_stream_arena_bytes(sizes, n, 4, 2)
    assert need == 2 * 4 * 1000 * 256
    assert L.block_stream_arena_bytes(sizes, n, 1, 8) == need          # ring of 8 single layers
    assert L.block_stream_arena_bytes(sizes, n, 2, 3) == 3 * 2 * 1000 * 256
    assert L.block_stream_arena_bytes(sizes, n, 4, 1) == 0
    h = ctypes.c_void_p()
    cs = (ctypes.c_void_p * 2)(None, None)  # default streams: nothing here reaches a HIP call
    rc = L.block_stream_create(ctypes.byref(h), ptrs, sizes, n, 4, 2, FAKE, need - 1, cs, 2)
    assert rc == abi.MSQ_E_WINDOW
    assert "window_blocks=3" in _err()
    rc = L.block_stream_create(ctypes.byref(h), ptrs, sizes, n, 4, 2, FAKE, 1000, cs, 1)
    assert rc == abi.MSQ_E_WINDOW and "not even one layer" in _err()
    assert L.block_stream_create(ctypes.byref(h), ptrs, sizes, n, 9, 2, FAKE, need, cs, 2) == abi.MSQ_E_INVAL
    assert L.block_stream_create(ctypes.byref(h), ptrs, sizes, n, 4, 1, FAKE, need, cs, 2) == abi.MSQ_E_INVAL
    assert L.block_stream_create(ctypes.byref(h), ptrs, sizes, n, 4, 2, FAKE + 16, need, cs, 2) == abi.MSQ_E_INVAL
    # the copy streams: an array of 1 .. MSQ_MAX_COPY_STREAMS
    assert L.block_stream_create(ctypes.byref(h), ptrs, sizes, n, 4, 2, FAKE, need, None, 1) == abi.MSQ_E_INVAL
    assert L.block_stream_create(ctypes.byref(h), ptrs, sizes, n, 4, 2, FAKE, need, cs, 0) == abi.MSQ_E_INVAL
    assert L.block_stream_create(ctypes.byref(h), ptrs, sizes, n, 4, 2, FAKE, need, cs, 5) == abi.MSQ_E_INVAL
    assert "n_copy_streams=5" in _err()
    assert L.block_stream_prefetch(None, 0) == abi.MSQ_E_INVAL


def test_window_positions_have_fixed_ranges():
    """Position q of a slot is as large as the largest layer any window puts at position q,
    so the ranges of different positions never overlap whatever the sizes: with layers of
    4096 + 256 i bytes in windows of 3, a slot is 4096+256*6 + 4096+256*7 + 4096+256*8
    (the last window's layers, the largest at each position)."""
    L = abi.lib()
    n = 9
    sizes = (ctypes.c_size_t * n)(*[4096 + 256 * i for i in range(n)])
    assert L.block_stream_arena_bytes(sizes, n, 3, 2) == 2 * sum(4096 + 256 * i for i in (6, 7, 8))
    # a short last window: 7 layers in windows of 3 -> positions sized by layers 6, 4, 5
    assert L.block_stream_arena_bytes(sizes, 7, 3, 2) == 2 * sum(4096 + 256 * i for i in (6, 4, 5))
    # sizes are rounded up to 256 bytes per position
    odd = (ctypes.c_size_t * 4)(1000, 10, 300, 1)
    assert L.block_stream_arena_bytes(odd, 4, 2, 3) == 3 * (1024 + 256)   # max(1000, 300), max(10, 1)
    # one byte short of the fixed layout is too small, and the message names what fits
    need = L.block_stream_arena_bytes(sizes, n, 3, 2)
    h = ctypes.c_void_p()
    cs = (ctypes.c_void_p * 1)(None)
    ptrs = (ctypes.c_void_p * n)(*([FAKE] * n))
    assert L.block_stream_create(ctypes.byref(h), ptrs, sizes, n, 3, 2, FAKE, need - 1, cs, 1) == abi.MSQ_E_WINDOW
    assert "window_blocks=2" in _err()


def test_window_checks_blobs_are_pinned():
    """A blob in ordinary (pageable) host memory is refused once every other argument has
    passed: MSQ_E_INVAL where the HIP runtime can tell, MSQ_E_HIP where it cannot (no GPU
    here); either way no window is created."""
    L = abi.lib()
    n = 2
    bufs = [ctypes.create_string_buffer(4096) for _ in range(n)]
    ptrs = (ctypes.c_void_p * n)(*[ctypes.addressof(b) for b in bufs])
    sizes = (ctypes.c_size_t * n)(4096, 4096)
    need = L.block_stream_arena_bytes(sizes, n, 1, 2)
    h = ctypes.c_void_p(12345)
    cs = (ctypes.c_void_p * 1)(None)
    rc = L.block_stream_create(ctypes.byref(h), ptrs, sizes, n, 1, 2, FAKE, need, cs, 1)
    assert rc in (abi.MSQ_E_INVAL, abi.MSQ_E_HIP)
    assert "pinned" in _err() and h.value is None


def test_host_alloc_rejects_bad_sizes():
    L = abi.lib()
    p = ctypes.c_void_p()
    assert L.msq_host_alloc(0, ctypes.byref(p)) == abi.MSQ_E_INVAL
    assert L.msq_host_alloc(1 << 47, ctypes.byref(p)) == abi.MSQ_E_INVAL
    assert L.msq_host_alloc(4096, None) == abi.MSQ_E_INVAL
    assert L.msq_host_free(None) == abi.MSQ_OK


def test_timing_collect_without_records():
    L = abi.lib()
    n = ctypes.c_int(-1)
    assert L.msq_timing_collect(None, 0, ctypes.byref(n)) == 0
    assert n.value == 0


def test_strerror_covers_every_code():
    L = abi.lib()
    for code in (0, -1, -2, -3, -4, -5, -6, -7):
        assert L.msq_strerror(code) and L.msq_strerror(code) != b"unknown error"


def test_missing_library_raises_on_use(tmp_path):
    """Without libmsq.so the package still imports (so the build module can run), and
    the first call into the library raises: nothing falls back to the CPU."""
    import shutil
    import subprocess
    import sys

    pkg = tmp_path / "memory_streamed_qlora_amd"
    pkg.mkdir()
    for f in os.listdir(os.path.join(ROOT, "memory_streamed_qlora_amd")):
        if f.endswith(".py"):
            shutil.copy(os.path.join(ROOT, "memory_streamed_qlora_amd", f), pkg / f)
    code = ("import sys; sys.path.insert(0, %r); import memory_streamed_qlora_amd as m; "
            "import memory_streamed_qlora_amd.build; m.nf4_codebook()" % str(tmp_path))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "libmsq.so not found" in r.stderr


def test_u_given_flag():
    """MSQ_U_GIVEN: a forward flag that needs r > 0 and the given u, and excludes
    MSQ_U_ONLY; a group needs every projection's u."""
    L = abi.lib()
    need = L.nf4_lora_workspace_size(8, 128, 128, 16)
    G = abi.MSQ_U_GIVEN
    args = lambda r, flags, u: (FAKE, 8, 128, 128, FAKE, FAKE, None, None, FAKE, FAKE,  # noqa: E731
                                abi.LoraCfg(r, 32.0, 0.0, flags), abi.RngKey(0, 0, 0, 0, 0), FAKE, u,
                                FAKE, need, None)
    assert L.nf4_lora_fwd(*args(16, G | abi.MSQ_U_ONLY, FAKE)) == abi.MSQ_E_INVAL
    assert "nothing to compute" in _err()
    assert L.nf4_lora_fwd(*args(0, G, FAKE)) == abi.MSQ_E_INVAL
    assert "r > 0" in _err()
    assert L.nf4_lora_fwd(*args(16, G, None)) == abi.MSQ_E_INVAL
    assert "u_out" in _err()
    bneed = L.nf4_lora_workspace_size(8, 128, 128, 16)
    assert L.nf4_lora_bwd(FAKE, FAKE, 8, 128, 128, FAKE, FAKE, FAKE, FAKE, abi.LoraCfg(16, 32.0, 0.0, G),
                          abi.RngKey(0, 0, 0, 0, 0), FAKE, FAKE, 0, FAKE, FAKE, 0, FAKE, bneed, None) == abi.MSQ_E_INVAL
    assert "forward flags" in _err()
    key = abi.RngKey(0, 0, 0, 0, 0)
    two = (abi.LoraProj * 2)(abi.LoraProj(128, FAKE, FAKE, None, None, None, FAKE, FAKE, key, FAKE, FAKE),
                             abi.LoraProj(64, FAKE, FAKE, None, None, None, FAKE, FAKE, key, FAKE, None))
    gneed = L.lora_group_workspace_size(8, 128, two, 2, 16)
    assert L.lora_fwd_group(FAKE, 8, 128, two, 2, abi.LoraCfg(16, 32.0, 0.0, G), FAKE, gneed, None) == abi.MSQ_E_INVAL
    assert "every projection's u_out" in _err()
