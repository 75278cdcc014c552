"""The streamed quantizing loader (nf4_stream_load, Stack.load).

The pages' default loader stages one tensor at a time, quantizes it and evicts it; its
device peak stays far below a standard load's, its output is byte-identical to the
standard load's (sha256 manifests) and training re-gates at 0.00e+00 on the loaded base
("Poros" research post, streamed-loader paragraph).  Checked here on a synthetic
Qwen2.5-0.5B-shaped checkpoint in safetensors format (random bf16 weights, read through
a memory map) and on 32B-shaped layers from host memory:
  * per-layer sha256 of the streamed-loaded blobs == the standard load's;
  * the codes and absmax equal the oracle's quantization of the same bf16 matrices;
  * the chunk size does not change a byte (one-row chunks against the default);
  * the device peak of the streamed load is its two staging slots, the standard load's
    the whole bf16 base;
  * training after a streamed load is bitwise the training after a standard load, and
    streamed == resident on the loaded base."""
import hashlib

import numpy as np
import pytest
import torch

from oracle import nf4 as onf4

pytestmark = pytest.mark.gpu
msq = pytest.importorskip("memory_streamed_qlora_amd")
from memory_streamed_qlora_amd import stack as S  # noqa: E402

SHAPE05 = S.Shape(896, 14, 2, 64, 4864, 24, vocab=1024)


def _synthetic_checkpoint(shape: S.Shape, seed: int) -> dict:
    """Qwen2-named host bf16 tensors with the family's shapes (random weights)."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    t = {}
    for l in range(shape.layers):
        for proj in S.PROJS:
            K, N = shape.proj_shape(proj)
            t[S.Stack.tensor_name(l, proj)] = (torch.randn(N, K, generator=g) * 0.02).to(torch.bfloat16)
            if proj in ("q", "k", "v"):
                t[S.Stack.tensor_name(l, proj, "bias")] = (torch.randn(N, generator=g) * 0.02).to(torch.bfloat16)
        for nm in ("input_layernorm", "post_attention_layernorm"):
            t[f"model.layers.{l}.{nm}.weight"] = (1 + 0.02 * torch.randn(shape.hidden, generator=g)).to(torch.bfloat16)
    t["model.embed_tokens.weight"] = (torch.randn(shape.vocab, shape.hidden, generator=g) * 0.02).to(torch.bfloat16)
    t["lm_head.weight"] = (torch.randn(shape.vocab, shape.hidden, generator=g) * 0.02).to(torch.bfloat16)
    t["model.norm.weight"] = (1 + 0.02 * torch.randn(shape.hidden, generator=g)).to(torch.bfloat16)
    return t


@pytest.fixture(scope="module")
def checkpoint(tmp_path_factory):
    from safetensors import safe_open
    from safetensors.torch import save_file
    path = tmp_path_factory.mktemp("ckpt") / "qwen25_05b_synthetic.safetensors"
    t = _synthetic_checkpoint(SHAPE05, 11)
    save_file(t, str(path))
    del t
    f = safe_open(str(path), framework="pt", device="cpu")
    return lambda name: f.get_tensor(name).contiguous()


def _digests(blobs):
    return [hashlib.sha256(b.numpy().tobytes()).hexdigest() for b in blobs]


def _load(shape, source, loader, **kw):
    """(blobs, device peak of the load above what was allocated before)."""
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    before = torch.cuda.memory_allocated()
    blobs = S.Stack.load_base(shape, source, loader, **kw)
    torch.cuda.synchronize()
    return blobs, torch.cuda.max_memory_allocated() - before


def _base_bytes(shape: S.Shape) -> int:
    return sum(2 * shape.proj_shape(p)[0] * shape.proj_shape(p)[1] for p in S.PROJS) * shape.layers


def test_streamed_load_is_byte_identical_to_standard_load(checkpoint):
    peaks, digests = {}, {}
    for loader in ("standard", "streamed"):
        print(f"[loader] {loader}", flush=True)
        blobs, peaks[loader] = _load(SHAPE05, checkpoint, loader)
        digests[loader] = _digests(blobs)
        if loader == "streamed":
            # codes and absmax of two projections against the oracle's quantization
            v = S.LayerLayout(SHAPE05).views(blobs[3])
            for proj in ("q", "k"):
                w = checkpoint(S.Stack.tensor_name(3, proj)).view(torch.int16).numpy().view(np.uint16)
                w32 = (w.astype(np.uint32) << 16).view(np.float32)
                codes, absmax = onf4.quantize(w32)
                assert np.array_equal(v[(proj, "codes")].numpy(), codes), proj
                assert np.array_equal(v[(proj, "absmax")].numpy().view(np.uint32), absmax.view(np.uint32)), proj
        del blobs
    assert digests["streamed"] == digests["standard"], "streamed load differs from the standard load"
    total = _base_bytes(SHAPE05)
    print(f"[loader] device peak: standard {peaks['standard'] / 1e6:.1f} MB, streamed "
          f"{peaks['streamed'] / 1e6:.1f} MB (bf16 base {total / 1e6:.1f} MB)", flush=True)
    assert peaks["standard"] >= total
    assert peaks["streamed"] <= 100e6  # the two 32 MB staging slots and their NF4 outputs


def test_chunk_size_does_not_change_a_byte(checkpoint):
    lay = S.LayerLayout(SHAPE05)
    blobs = []
    for chunk in (4096, 1 << 20, 32 << 20):
        blob = torch.zeros(lay.nbytes, dtype=torch.uint8, pin_memory=True)
        v = lay.views(blob)
        info = msq.nf4_stream_load([(checkpoint(S.Stack.tensor_name(5, p)), v[(p, "codes")], v[(p, "absmax")])
                                    for p in S.PROJS], chunk_bytes=chunk, host_threads=4)
        print(f"[loader] chunk {chunk}: {info}", flush=True)
        blobs.append(blob)
    assert torch.equal(blobs[0], blobs[1]) and torch.equal(blobs[1], blobs[2])


def test_training_on_loaded_base_is_bitwise(checkpoint):
    """Streamed-loaded vs standard-loaded base, and streamed vs resident on the streamed
    load: 2 optimizer steps with dropout, every surface equal."""
    shape = S.Shape(896, 14, 2, 64, 4864, 4, vocab=1024)
    outs = []
    for loader, mode in (("standard", "streamed"), ("streamed", "streamed"), ("streamed", "resident")):
        st = S.Stack.load(shape, 128, checkpoint, loader=loader, seed=2, mode=mode, window_blocks=1, p_drop=0.1)
        res = []
        for s in range(2):
            loss, gn = st.train_step(S.random_tokens(2, s, 128, shape.vocab, st.dev))
            res.append((loss.item(), gn.item()))
        torch.cuda.synchronize()
        outs.append((res, {k: v.clone() for k, v in st.state_tensors().items()}))
        st.close()
    for other in outs[1:]:
        assert other[0] == outs[0][0]
        for k in outs[0][1]:
            assert torch.equal(outs[0][1][k], other[1][k]), k


@pytest.mark.slow
def test_qwen32b_layers_streamed_load():
    """Four Qwen2.5-32B-shaped layers (3.9 GB of bf16) from pageable host memory:
    byte-identical to the standard load; reports the loader's rate and device peak."""
    import time
    shape = S.Shape(5120, 40, 8, 128, 27648, 4, vocab=1024)
    src = {}
    g = torch.Generator(device="cuda").manual_seed(5)
    for l in range(shape.layers):
        for proj in S.PROJS:
            K, N = shape.proj_shape(proj)
            src[S.Stack.tensor_name(l, proj)] = (torch.randn(N, K, generator=g, device="cuda") * 0.02).to(
                torch.bfloat16).cpu()
            if proj in ("q", "k", "v"):
                src[S.Stack.tensor_name(l, proj, "bias")] = torch.zeros(N, dtype=torch.bfloat16)
        for nm in ("input_layernorm", "post_attention_layernorm"):
            src[f"model.layers.{l}.{nm}.weight"] = torch.ones(shape.hidden)
    src["model.embed_tokens.weight"] = torch.zeros(shape.vocab, shape.hidden, dtype=torch.bfloat16)
    src["lm_head.weight"] = torch.zeros(shape.vocab, shape.hidden, dtype=torch.bfloat16)
    src["model.norm.weight"] = torch.ones(shape.hidden)
    digests, peaks = {}, {}
    for loader in ("standard", "streamed"):
        t0 = time.perf_counter()
        blobs, peaks[loader] = _load(shape, src.__getitem__, loader)
        dt = time.perf_counter() - t0
        digests[loader] = _digests(blobs)
        print(f"[loader 32B] {loader}: {dt:.2f}s for {_base_bytes(shape) / 1e9:.2f} GB bf16 "
              f"({_base_bytes(shape) / dt / 1e9:.1f} GB/s), device peak {peaks[loader] / 1e9:.3f} GB", flush=True)
        del blobs
    assert digests["streamed"] == digests["standard"]
    assert peaks["standard"] >= _base_bytes(shape)
    assert peaks["streamed"] <= 100e6
