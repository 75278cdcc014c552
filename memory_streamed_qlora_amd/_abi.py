"""ctypes declarations of libmsq (include/msq.h).  Loading fails loudly: there is no
CPU or PyTorch fallback for any operation of the library."""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmsq.so")

MSQ_OK = 0
MSQ_E_INVAL = -1
MSQ_E_SHAPE = -2
MSQ_E_DROPOUT = -3
MSQ_E_WORKSPACE = -4
MSQ_E_WINDOW = -5
MSQ_E_ORDER = -6
MSQ_E_HIP = -7

ERROR_NAMES = {
    MSQ_E_INVAL: "MSQ_E_INVAL", MSQ_E_SHAPE: "MSQ_E_SHAPE", MSQ_E_DROPOUT: "MSQ_E_DROPOUT",
    MSQ_E_WORKSPACE: "MSQ_E_WORKSPACE", MSQ_E_WINDOW: "MSQ_E_WINDOW", MSQ_E_ORDER: "MSQ_E_ORDER",
    MSQ_E_HIP: "MSQ_E_HIP",
}


class RngKey(ctypes.Structure):
    _fields_ = [("seed", ctypes.c_uint64), ("step", ctypes.c_uint32), ("micro", ctypes.c_uint32),
                ("layer", ctypes.c_uint32), ("proj", ctypes.c_uint32)]


MSQ_ACT_F32 = 1
MSQ_OUT_F32 = 2
MSQ_U_ONLY = 4
MSQ_U_GIVEN = 32
MSQ_PATH_TILED = 8
MSQ_PATH_SMALL = 16
MSQ_MAX_COPY_STREAMS = 4


class LoraCfg(ctypes.Structure):
    _fields_ = [("r", ctypes.c_int32), ("alpha", ctypes.c_float), ("p_drop", ctypes.c_float),
                ("flags", ctypes.c_uint32)]


class WindowStats(ctypes.Structure):
    _fields_ = [("bytes_copied", ctypes.c_uint64), ("windows_copied", ctypes.c_uint64),
                ("windows_reused", ctypes.c_uint64), ("copy_ms", ctypes.c_double),
                ("copies_timed", ctypes.c_uint64), ("busy_ms", ctypes.c_double)]


class QuantJob(ctypes.Structure):
    _fields_ = [("src", ctypes.c_void_p), ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("codes", ctypes.c_void_p), ("absmax", ctypes.c_void_p)]


class LoraProj(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int64), ("codes", ctypes.c_void_p), ("absmax", ctypes.c_void_p),
                ("w", ctypes.c_void_p), ("bias", ctypes.c_void_p), ("residual", ctypes.c_void_p),
                ("A", ctypes.c_void_p), ("B", ctypes.c_void_p), ("key", RngKey), ("y", ctypes.c_void_p),
                ("u_out", ctypes.c_void_p)]


class LoraProjGrad(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int64), ("codes", ctypes.c_void_p), ("absmax", ctypes.c_void_p),
                ("w", ctypes.c_void_p), ("A", ctypes.c_void_p), ("B", ctypes.c_void_p), ("key", RngKey),
                ("dy", ctypes.c_void_p), ("u", ctypes.c_void_p), ("dA", ctypes.c_void_p), ("dB", ctypes.c_void_p)]


class AdamwCfg(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_double), ("beta1", ctypes.c_double), ("beta2", ctypes.c_double),
                ("eps", ctypes.c_double), ("weight_decay", ctypes.c_double)]


class AdamwTensor(ctypes.Structure):
    _fields_ = [("p", ctypes.c_void_p), ("g", ctypes.c_void_p), ("m", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("n", ctypes.c_int64)]


class KernelTiming(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 48), ("launches", ctypes.c_uint64),
                ("total_ms", ctypes.c_double), ("total_flops", ctypes.c_double),
                ("total_bytes", ctypes.c_double)]


class MsqError(RuntimeError):
    def __init__(self, fn: str, code: int, detail: str):
        self.code = code
        self.fn = fn
        super().__init__(f"{fn} failed: {ERROR_NAMES.get(code, code)}: {detail}")


_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_SIG = {
    "msq_abi_version": (ctypes.c_int, []),
    "msq_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "msq_last_error": (ctypes.c_char_p, []),
    "msq_nf4_codebook": (ctypes.c_int, [_P]),
    "nf4_quantize": (ctypes.c_int, [_P, _I64, _I64, _P, _P, _P]),
    "nf4_dequantize": (ctypes.c_int, [_P, _P, _I64, _I64, _P, _P]),
    "nf4_lora_workspace_size": (ctypes.c_size_t, [_I64, _I64, _I64, ctypes.c_int32]),
    "nf4_lora_fwd": (ctypes.c_int, [_P, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P, LoraCfg, RngKey,
                                    _P, _P, _P, ctypes.c_size_t, _P]),
    "nf4_lora_fwd_noalloc": (ctypes.c_int, [_P, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P, LoraCfg, RngKey,
                                            _P, _P, _P]),
    "nf4_lora_bwd": (ctypes.c_int, [_P, _P, _I64, _I64, _I64, _P, _P, _P, _P, LoraCfg, RngKey, _P,
                                    _P, ctypes.c_int, _P, _P, ctypes.c_int, _P, ctypes.c_size_t,
                                    _P]),
    "msq_swiglu_fwd": (ctypes.c_int, [_P, _P, _I64, _P, _P]),
    "msq_swiglu_bwd": (ctypes.c_int, [_P, _P, _P, _I64, _P, _P, _P]),
    "msq_rope_fwd": (ctypes.c_int, [_P, _P, _P, _I64, ctypes.c_int32, ctypes.c_int32, _P, _P]),
    "msq_rope_bwd": (ctypes.c_int, [_P, _P, _P, _I64, ctypes.c_int32, ctypes.c_int32, _P, _P]),
    "msq_rmsnorm_apply_fwd": (ctypes.c_int, [_P, _P, _P, _I64, _I64, _P, _P]),
    "msq_rmsnorm_apply_bwd": (ctypes.c_int, [_P, _P, _P, _P, _I64, _I64, _P, _P, _P]),
    "bf16_lora_fwd": (ctypes.c_int, [_P, _I64, _I64, _I64, _P, _P, _P, _P, _P, LoraCfg, RngKey,
                                     _P, _P, _P, ctypes.c_size_t, _P]),
    "bf16_lora_bwd": (ctypes.c_int, [_P, _P, _I64, _I64, _I64, _P, _P, _P, LoraCfg, RngKey, _P,
                                     _P, ctypes.c_int, _P, _P, ctypes.c_int, _P, ctypes.c_size_t,
                                     _P]),
    "lora_group_workspace_size": (ctypes.c_size_t, [_I64, _I64, _P, ctypes.c_int, ctypes.c_int32]),
    "lora_fwd_group": (ctypes.c_int, [_P, _I64, _I64, _P, ctypes.c_int, LoraCfg, _P, ctypes.c_size_t, _P]),
    "lora_group_bwd_workspace_size": (ctypes.c_size_t, [_I64, _I64, _P, ctypes.c_int, ctypes.c_int32]),
    "lora_bwd_group": (ctypes.c_int, [_P, _I64, _I64, _P, ctypes.c_int, LoraCfg, _P, ctypes.c_int, ctypes.c_int, _P,
                                      ctypes.c_size_t, _P]),
    "msq_kernel_copy": (ctypes.c_int, [_P, _P, ctypes.c_size_t, _P]),
    "msq_adamw_partials": (_I64, [_P, ctypes.c_int]),
    "msq_adamw_step": (ctypes.c_int, [_P, ctypes.c_int, AdamwCfg, _I64, _P, _P]),
    "msq_host_alloc": (ctypes.c_int, [ctypes.c_size_t, _P]),
    "msq_host_free": (ctypes.c_int, [_P]),
    "nf4_stream_load_device_bytes": (ctypes.c_size_t, [_I64, _I64]),
    "nf4_stream_load_host_bytes": (ctypes.c_size_t, [_I64, _I64]),
    "nf4_stream_load": (ctypes.c_int, [_P, ctypes.c_int, _I64, _P, ctypes.c_size_t, _P, ctypes.c_size_t,
                                       ctypes.c_int, _P]),
    "block_stream_arena_bytes": (ctypes.c_size_t, [_P, ctypes.c_int, ctypes.c_int, ctypes.c_int]),
    "block_stream_create": (ctypes.c_int, [_P, _P, _P, ctypes.c_int, ctypes.c_int, ctypes.c_int, _P,
                                           ctypes.c_size_t, _P, ctypes.c_int]),
    "block_stream_prefetch": (ctypes.c_int, [_P, ctypes.c_int]),
    "block_stream_acquire": (ctypes.c_int, [_P, ctypes.c_int, _P, _P]),
    "block_stream_release": (ctypes.c_int, [_P, ctypes.c_int, _P]),
    "block_stream_release_layer": (ctypes.c_int, [_P, ctypes.c_int, _P]),
    "block_stream_stats": (ctypes.c_int, [_P, _P]),
    "block_stream_destroy": (ctypes.c_int, [_P]),
    "msq_timing_enable": (ctypes.c_int, [ctypes.c_int]),
    "msq_timing_collect": (ctypes.c_int, [_P, ctypes.c_int, _P]),
    "msq_timing_reserve": (ctypes.c_int, [ctypes.c_int]),
}
EXPORTED = tuple(_SIG)

ABI_VERSION = 15  # MSQ_ABI_VERSION of include/msq.h
_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"libmsq.so not found at {LIB_PATH}: build it with "
                "`python -m memory_streamed_qlora_amd.build` (there is no CPU fallback)")
        h = ctypes.CDLL(LIB_PATH)
        h.msq_abi_version.restype = ctypes.c_int
        h.msq_abi_version.argtypes = []
        if h.msq_abi_version() != ABI_VERSION:
            raise ImportError(f"{LIB_PATH} has ABI version {h.msq_abi_version()}, this binding expects "
                              f"{ABI_VERSION}: rebuild it with `python -m memory_streamed_qlora_amd.build`")
        for name, (res, args) in _SIG.items():
            try:
                f = getattr(h, name)
            except AttributeError as e:
                raise ImportError(f"{LIB_PATH} lacks {name}: rebuild it with "
                                  "`python -m memory_streamed_qlora_amd.build`") from e
            f.restype = res
            f.argtypes = args
        _lib = h
    return _lib


def check(fn: str, rc: int) -> None:
    if rc != MSQ_OK:
        detail = lib().msq_last_error().decode(errors="replace")
        raise MsqError(fn, rc, detail)
