"""MI355X (gfx950) streamed NF4 + LoRA training hot path.

The compute lives in libmsq.so (C ABI: include/msq.h, HIP kernels under csrc/);
``ops`` is its thin Python binding and ``stack`` the Qwen2.5-shaped training step
that drives it.  Importing the package loads the library; if it is missing or was
built for another ABI version, the import still succeeds (so that the build module can
run) but every call into the library raises -- there is no CPU fallback.
"""
from ._abi import MsqError, lib as _load_library  # noqa: F401
from .ops import (BlockStreamWindow, Lora, Workspace, abi_version, adamw_partials, adamw_step,  # noqa: F401
                  bf16_lora_bwd, bf16_lora_fwd, kernel_copy,
                  lora_bwd_group, lora_fwd_group, nf4_codebook,
                  nf4_dequantize, nf4_lora_bwd, nf4_lora_fwd, nf4_lora_workspace_size,
                  nf4_quantize, nf4_stream_load, rmsnorm_apply_bwd, rmsnorm_apply_fwd, rng_key, rope_bwd, rope_fwd,
                  swiglu_bwd, swiglu_fwd,
                  timing_collect, timing_enable)

try:
    _load_library()
except ImportError:  # not built yet, or stale: every call into the library raises the same error
    pass
