"""Python binding of libmsq with the C-ABI's names.

Argument marshalling only: tensors are checked for device, dtype and layout, their
addresses and sizes are passed to the library, and any error code is raised as
MsqError.  Every computation happens in the library's HIP kernels; PyTorch only
provides device memory and streams.  Outputs not supplied by the caller are
allocated with torch on the input's device.
"""
from __future__ import annotations

import ctypes
import functools
import sys
from dataclasses import dataclass
from typing import Optional, Sequence, Tuple

import torch

from . import _abi
from ._abi import LoraCfg, RngKey, check, lib

PROJS = ("q", "k", "v", "o", "gate", "up", "down")
PROJ_ID = {p: i for i, p in enumerate(PROJS)}


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _req(t: torch.Tensor, name: str, dtype: torch.dtype, shape: Tuple[int, ...]) -> None:
    # one combined test on the common path (a call checks ~10 tensors); the messages below
    # name what is wrong
    if type(t) is torch.Tensor and t.is_cuda and t.dtype is dtype and t.shape == shape and t.is_contiguous():
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor (got {t.device})")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def abi_version() -> int:
    return lib().msq_abi_version()


def nf4_codebook() -> torch.Tensor:
    """The library's 16 NF4 levels (host, float32)."""
    out = torch.empty(16, dtype=torch.float32)
    check("msq_nf4_codebook", lib().msq_nf4_codebook(out.data_ptr()))
    return out


def nf4_quantize(w: torch.Tensor, codes: Optional[torch.Tensor] = None,
                 absmax: Optional[torch.Tensor] = None, stream=None):
    """w bf16 [n, k] -> (codes uint8 [n, k/2], absmax fp32 [n, k/64])."""
    n, k = w.shape
    _req(w, "w", torch.bfloat16, (n, k))
    if codes is None:
        codes = torch.empty((n, k // 2), dtype=torch.uint8, device=w.device)
    if absmax is None:
        absmax = torch.empty((n, k // 64), dtype=torch.float32, device=w.device)
    _req(codes, "codes", torch.uint8, (n, k // 2))
    _req(absmax, "absmax", torch.float32, (n, k // 64))
    check("nf4_quantize", lib().nf4_quantize(_ptr(w), n, k, _ptr(codes), _ptr(absmax), _stream(stream)))
    return codes, absmax


def nf4_dequantize(codes: torch.Tensor, absmax: torch.Tensor, out: Optional[torch.Tensor] = None,
                   stream=None) -> torch.Tensor:
    n, kh = codes.shape
    k = 2 * kh
    _req(codes, "codes", torch.uint8, (n, kh))
    _req(absmax, "absmax", torch.float32, (n, k // 64))
    if out is None:
        out = torch.empty((n, k), dtype=torch.bfloat16, device=codes.device)
    _req(out, "out", torch.bfloat16, (n, k))
    check("nf4_dequantize", lib().nf4_dequantize(_ptr(codes), _ptr(absmax), n, k, _ptr(out), _stream(stream)))
    return out


@functools.lru_cache(maxsize=1024)
def nf4_lora_workspace_size(t: int, k: int, n: int, r: int) -> int:
    # a function of the shape alone (cached: the fused calls ask for it every time)
    return int(lib().nf4_lora_workspace_size(t, k, n, r))


class Workspace:
    """A growable device scratch buffer for the fused linear calls (one per stream)."""

    def __init__(self, device=None):
        self.device = torch.device(device or "cuda")
        self.buf: Optional[torch.Tensor] = None

    def get(self, nbytes: int) -> torch.Tensor:
        nbytes = max(int(nbytes), 256)
        if self.buf is None or self.buf.numel() < nbytes:
            self.buf = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        return self.buf


_default_ws = {}


def _workspace(device: torch.device, nbytes: int, ws: Optional[Workspace], stream_handle: Optional[int] = None
               ) -> torch.Tensor:
    if ws is None:
        key = (device.index, stream_handle if stream_handle is not None
               else torch.cuda.current_stream(device).cuda_stream)
        ws = _default_ws.get(key)
        if ws is None:
            ws = _default_ws.setdefault(key, Workspace(device))
    return ws.get(nbytes)


@dataclass(frozen=True)
class Lora:
    r: int = 16
    alpha: float = 32.0
    p_drop: float = 0.0

    def c(self, flags: int = 0) -> LoraCfg:
        return LoraCfg(self.r, self.alpha, self.p_drop, flags)


_ACT_DTYPES = (torch.bfloat16, torch.float32)


def _flags(act_dtype: torch.dtype, out_dtype: torch.dtype) -> int:
    if act_dtype not in _ACT_DTYPES or out_dtype not in _ACT_DTYPES:
        raise TypeError("activations and outputs must be bfloat16 or float32")
    return (_abi.MSQ_ACT_F32 if act_dtype == torch.float32 else 0) | \
           (_abi.MSQ_OUT_F32 if out_dtype == torch.float32 else 0)


_PATHS = {"auto": 0, "tiled": _abi.MSQ_PATH_TILED, "small": _abi.MSQ_PATH_SMALL}


def _path_flags(path: str) -> int:
    """Path flags of a single fused call: "auto" (the library picks by shape), "tiled" or
    "small" (see MSQ_PATH_TILED / MSQ_PATH_SMALL)."""
    if path not in _PATHS:
        raise ValueError(f"path must be one of {sorted(_PATHS)}, not {path!r}")
    return _PATHS[path]


def rng_key(seed: int = 0, step: int = 0, micro: int = 0, layer: int = 0, proj: int = 0) -> RngKey:
    return RngKey(seed, step, micro, layer, proj)


def _base_args(base: Tuple[torch.Tensor, ...], k: int) -> Tuple[str, int, list]:
    """(entry-point prefix, n, pointer arguments) for an NF4 (codes, absmax) or bf16 (w,) base."""
    if len(base) == 2:
        codes, absmax = base
        n = codes.shape[0]
        _req(codes, "codes", torch.uint8, (n, k // 2))
        _req(absmax, "absmax", torch.float32, (n, k // 64))
        return "nf4", n, [_ptr(codes), _ptr(absmax)]
    (w,) = base
    n = w.shape[0]
    _req(w, "w", torch.bfloat16, (n, k))
    return "bf16", n, [_ptr(w)]


def _lora_fwd(base, x, bias, A, B, cfg, key, y, u_out, want_u, workspace, stream, out_dtype, u_only, residual,
              noalloc=False, path="auto", u_given=False):
    t, k = x.shape
    _req(x, "x", x.dtype, (t, k))
    fmt, n, bptr = _base_args(base, k)
    out_dtype = out_dtype or (y.dtype if y is not None else x.dtype)
    flags = _flags(x.dtype, out_dtype) | _path_flags(path)
    if bias is not None:
        _req(bias, "bias", torch.bfloat16, (n,))
    r = cfg.r
    if r > 0:
        _req(A, "A", torch.float32, (r, k))
        _req(B, "B", torch.float32, (n, r))
    if u_given:
        if u_only or r == 0 or u_out is None:
            raise ValueError("u_given needs r > 0 and the given u as u_out, and excludes u_only")
        flags |= _abi.MSQ_U_GIVEN
    if u_only:
        if r == 0:
            raise ValueError("u_only needs r > 0")
        flags |= _abi.MSQ_U_ONLY
        want_u = True
        y = None
    else:
        if y is None:
            y = torch.empty((t, n), dtype=out_dtype, device=x.device)
        _req(y, "y", out_dtype, (t, n))
    if residual is not None:
        if u_only:
            raise ValueError("u_only computes no y to add a residual to")
        _req(residual, "residual", out_dtype, (t, n))
    if want_u and r > 0 and u_out is None:
        u_out = torch.empty((t, r), dtype=torch.float32, device=x.device)
    if u_out is not None:
        _req(u_out, "u_out", torch.float32, (t, r))
    args = (_ptr(x), t, k, n, *bptr, _ptr(bias), _ptr(residual), _ptr(A) if r > 0 else None,
            _ptr(B) if r > 0 else None, cfg.c(flags), key, _ptr(y), _ptr(u_out))
    if noalloc:  # the library's static scratch, no workspace
        check("nf4_lora_fwd_noalloc", lib().nf4_lora_fwd_noalloc(*args, _stream(stream)))
        return y, u_out
    need = nf4_lora_workspace_size(t, k, n, r)
    sh = _stream(stream)
    ws = _workspace(x.device, need, workspace, sh if stream is None else None)
    fn = f"{fmt}_lora_fwd"
    check(fn, getattr(lib(), fn)(
        _ptr(x), t, k, n, *bptr, _ptr(bias), _ptr(residual), _ptr(A) if r > 0 else None,
        _ptr(B) if r > 0 else None, cfg.c(flags), key, _ptr(y), _ptr(u_out), _ptr(ws), ws.numel(), sh))
    return y, u_out


def _lora_bwd(base, dy, x, A, B, cfg, key, u, dx, dx_accumulate, dA, dB, dAB_accumulate, workspace, stream,
              out_dtype, path="auto"):
    t, k = x.shape
    _req(x, "x", x.dtype, (t, k))
    fmt, n, bptr = _base_args(base, k)
    _req(dy, "dy", x.dtype, (t, n))
    out_dtype = out_dtype or (dx.dtype if dx is not None else x.dtype)
    flags = _flags(x.dtype, out_dtype) | _path_flags(path)
    r = cfg.r
    if r > 0:
        _req(A, "A", torch.float32, (r, k))
        _req(B, "B", torch.float32, (n, r))
        if dA is None:
            dA = torch.empty((r, k), dtype=torch.float32, device=x.device)
        if dB is None:
            dB = torch.empty((n, r), dtype=torch.float32, device=x.device)
        _req(dA, "dA", torch.float32, (r, k))
        _req(dB, "dB", torch.float32, (n, r))
        if u is not None:
            _req(u, "u", torch.float32, (t, r))
    if dx is None:
        dx = torch.empty((t, k), dtype=out_dtype, device=x.device)
    _req(dx, "dx", out_dtype, (t, k))
    need = nf4_lora_workspace_size(t, k, n, r)
    sh = _stream(stream)
    ws = _workspace(x.device, need, workspace, sh if stream is None else None)
    fn = f"{fmt}_lora_bwd"
    check(fn, getattr(lib(), fn)(
        _ptr(dy), _ptr(x), t, k, n, *bptr, _ptr(A) if r > 0 else None,
        _ptr(B) if r > 0 else None, cfg.c(flags), key, _ptr(u) if r > 0 else None, _ptr(dx),
        int(dx_accumulate), _ptr(dA) if r > 0 else None, _ptr(dB) if r > 0 else None,
        int(dAB_accumulate), _ptr(ws), ws.numel(), sh))
    return dx, (dA if r > 0 else None), (dB if r > 0 else None)


def lora_fwd_group(x: torch.Tensor, projs: Sequence[dict], cfg: Lora, want_u: bool = True,
                   workspace: Optional[Workspace] = None, stream=None,
                   out_dtype: Optional[torch.dtype] = None, u_given: bool = False):
    """Up to three projections of the same x in one pass (lora_fwd_group): each dict has
    base ((codes, absmax) or (w,)), bias, A, B, key and optionally residual; with u_given,
    also "u": the projection's u from an earlier call, used instead of forming it.  Returns
    a list of (y, u)."""
    t, k = x.shape
    _req(x, "x", x.dtype, (t, k))
    out_dtype = out_dtype or x.dtype
    flags = _flags(x.dtype, out_dtype)
    if u_given:
        if cfg.r == 0:
            raise ValueError("u_given needs r > 0")
        flags |= _abi.MSQ_U_GIVEN
    if not 1 <= len(projs) <= 3:
        raise ValueError("a group has 1 to 3 projections")
    arr = (_abi.LoraProj * len(projs))()
    outs = []
    r = cfg.r
    for i, pr in enumerate(projs):
        fmt, n, bptr = _base_args(pr["base"], k)
        bias, res = pr.get("bias"), pr.get("residual")
        if bias is not None:
            _req(bias, "bias", torch.bfloat16, (n,))
        if res is not None:
            _req(res, "residual", out_dtype, (t, n))
        if r > 0:
            _req(pr["A"], "A", torch.float32, (r, k))
            _req(pr["B"], "B", torch.float32, (n, r))
        y = torch.empty((t, n), dtype=out_dtype, device=x.device)
        if u_given:
            u = pr["u"]
            _req(u, "u", torch.float32, (t, r))
        else:
            u = torch.empty((t, r), dtype=torch.float32, device=x.device) if (want_u and r > 0) else None
        codes, absmax, w = (bptr + [None])[:3] if fmt == "nf4" else (None, None, bptr[0])
        arr[i] = _abi.LoraProj(n, codes, absmax, w, _ptr(bias), _ptr(res), _ptr(pr["A"]) if r > 0 else None,
                               _ptr(pr["B"]) if r > 0 else None, pr["key"], _ptr(y), _ptr(u))
        outs.append((y, u))
    need = int(lib().lora_group_workspace_size(t, k, arr, len(projs), r))
    if need == 0:
        raise ValueError(f"invalid group: {lib().msq_last_error().decode(errors='replace')}")
    ws = _workspace(x.device, need, workspace)
    check("lora_fwd_group", lib().lora_fwd_group(_ptr(x), t, k, arr, len(projs), cfg.c(flags), _ptr(ws), ws.numel(),
                                                 _stream(stream)))
    return outs


def lora_bwd_group(x: torch.Tensor, projs: Sequence[dict], cfg: Lora, dx: Optional[torch.Tensor] = None,
                   dx_accumulate: bool = False, dAB_accumulate: bool = False,
                   workspace: Optional[Workspace] = None, stream=None,
                   out_dtype: Optional[torch.dtype] = None):
    """Backward of up to three projections of the same x (lora_bwd_group): each dict has
    base ((codes, absmax) or (w,)), A, B, key, dy, and optionally u (the forward's) and dA,
    dB outputs.  Returns (dx, [(dA, dB), ...]) with dx the sum of the projections' input
    gradients."""
    t, k = x.shape
    _req(x, "x", x.dtype, (t, k))
    out_dtype = out_dtype or (dx.dtype if dx is not None else x.dtype)
    flags = _flags(x.dtype, out_dtype)
    if not 1 <= len(projs) <= 3:
        raise ValueError("a group has 1 to 3 projections")
    arr = (_abi.LoraProjGrad * len(projs))()
    grads = []
    r = cfg.r
    for i, pr in enumerate(projs):
        fmt, n, bptr = _base_args(pr["base"], k)
        dy = pr["dy"]
        _req(dy, "dy", x.dtype, (t, n))
        dA = dB = None
        u = pr.get("u")
        if r > 0:
            _req(pr["A"], "A", torch.float32, (r, k))
            _req(pr["B"], "B", torch.float32, (n, r))
            dA = pr.get("dA")
            dB = pr.get("dB")
            dA = torch.empty((r, k), dtype=torch.float32, device=x.device) if dA is None else dA
            dB = torch.empty((n, r), dtype=torch.float32, device=x.device) if dB is None else dB
            _req(dA, "dA", torch.float32, (r, k))
            _req(dB, "dB", torch.float32, (n, r))
            if u is not None:
                _req(u, "u", torch.float32, (t, r))
        codes, absmax, w = (bptr + [None])[:3] if fmt == "nf4" else (None, None, bptr[0])
        arr[i] = _abi.LoraProjGrad(n, codes, absmax, w, _ptr(pr["A"]) if r > 0 else None,
                                   _ptr(pr["B"]) if r > 0 else None, pr["key"], _ptr(dy),
                                   _ptr(u) if r > 0 else None, _ptr(dA), _ptr(dB))
        grads.append((dA, dB))
    if dx is None:
        dx = torch.empty((t, k), dtype=out_dtype, device=x.device)
    _req(dx, "dx", out_dtype, (t, k))
    need = int(lib().lora_group_bwd_workspace_size(t, k, arr, len(projs), r))
    if need == 0:
        raise ValueError(f"invalid group: {lib().msq_last_error().decode(errors='replace')}")
    ws = _workspace(x.device, need, workspace)
    check("lora_bwd_group", lib().lora_bwd_group(_ptr(x), t, k, arr, len(projs), cfg.c(flags), _ptr(dx),
                                                 int(dx_accumulate), int(dAB_accumulate), _ptr(ws), ws.numel(),
                                                 _stream(stream)))
    return dx, grads


def nf4_lora_fwd(x: torch.Tensor, codes: torch.Tensor, absmax: torch.Tensor,
                 bias: Optional[torch.Tensor], A: Optional[torch.Tensor], B: Optional[torch.Tensor],
                 cfg: Lora, key: RngKey, y: Optional[torch.Tensor] = None,
                 u_out: Optional[torch.Tensor] = None, want_u: bool = True,
                 workspace: Optional[Workspace] = None, stream=None,
                 out_dtype: Optional[torch.dtype] = None, u_only: bool = False,
                 residual: Optional[torch.Tensor] = None, path: str = "auto", u_given: bool = False):
    """y = [residual +] (x W^T + bias + (alpha/r) drop(x) A^T B^T), W the NF4 base.  Returns
    (y, u) (u None if not wanted).

    x may be bf16 or fp32; y is out_dtype (default: x's dtype, or y's if given).
    residual ([t, n], y's dtype) is added in the output pass, rounded as a separate add.
    u_only: compute only u (y is None).  u_given: u_out holds u from an earlier call with the
    same x, A and key, used instead of forming it.  path: "auto" (by shape), "tiled" or
    "small"."""
    return _lora_fwd((codes, absmax), x, bias, A, B, cfg, key, y, u_out, want_u, workspace, stream, out_dtype,
                     u_only, residual, path=path, u_given=u_given)


def nf4_lora_fwd_noalloc(x: torch.Tensor, codes: torch.Tensor, absmax: torch.Tensor,
                         bias: Optional[torch.Tensor], A: Optional[torch.Tensor], B: Optional[torch.Tensor],
                         cfg: Lora, key: RngKey, y: Optional[torch.Tensor] = None,
                         u_out: Optional[torch.Tensor] = None, want_u: bool = True, stream=None,
                         out_dtype: Optional[torch.dtype] = None, u_only: bool = False,
                         residual: Optional[torch.Tensor] = None, path: str = "auto", u_given: bool = False):
    """nf4_lora_fwd with the library's static per-GPU scratch in place of a workspace (the
    entry point for callers that cannot allocate).  Pass y (and u_out) to allocate nothing
    here either."""
    return _lora_fwd((codes, absmax), x, bias, A, B, cfg, key, y, u_out, want_u, None, stream, out_dtype,
                     u_only, residual, noalloc=True, path=path, u_given=u_given)


def bf16_lora_fwd(x: torch.Tensor, w: torch.Tensor, bias: Optional[torch.Tensor], A: Optional[torch.Tensor],
                  B: Optional[torch.Tensor], cfg: Lora, key: RngKey, y: Optional[torch.Tensor] = None,
                  u_out: Optional[torch.Tensor] = None, want_u: bool = True,
                  workspace: Optional[Workspace] = None, stream=None,
                  out_dtype: Optional[torch.dtype] = None, u_only: bool = False,
                  residual: Optional[torch.Tensor] = None, path: str = "auto", u_given: bool = False):
    """nf4_lora_fwd over a frozen base kept in bf16, w [n, k]."""
    return _lora_fwd((w,), x, bias, A, B, cfg, key, y, u_out, want_u, workspace, stream, out_dtype, u_only,
                     residual, path=path, u_given=u_given)


def nf4_lora_bwd(dy: torch.Tensor, x: torch.Tensor, codes: torch.Tensor, absmax: torch.Tensor,
                 A: Optional[torch.Tensor], B: Optional[torch.Tensor], cfg: Lora, key: RngKey,
                 u: Optional[torch.Tensor] = None, dx: Optional[torch.Tensor] = None,
                 dx_accumulate: bool = False, dA: Optional[torch.Tensor] = None,
                 dB: Optional[torch.Tensor] = None, dAB_accumulate: bool = False,
                 workspace: Optional[Workspace] = None, stream=None,
                 out_dtype: Optional[torch.dtype] = None, path: str = "auto"):
    """Returns (dx, dA, dB); dA/dB are None when r == 0.  dy and x share one dtype (bf16
    or fp32); dx is out_dtype (default: dx's dtype if given, else the activations').
    path: "auto" (by shape), "tiled" or "small"."""
    return _lora_bwd((codes, absmax), dy, x, A, B, cfg, key, u, dx, dx_accumulate, dA, dB, dAB_accumulate,
                     workspace, stream, out_dtype, path=path)


def bf16_lora_bwd(dy: torch.Tensor, x: torch.Tensor, w: torch.Tensor, A: Optional[torch.Tensor],
                  B: Optional[torch.Tensor], cfg: Lora, key: RngKey, u: Optional[torch.Tensor] = None,
                  dx: Optional[torch.Tensor] = None, dx_accumulate: bool = False,
                  dA: Optional[torch.Tensor] = None, dB: Optional[torch.Tensor] = None,
                  dAB_accumulate: bool = False, workspace: Optional[Workspace] = None, stream=None,
                  out_dtype: Optional[torch.dtype] = None, path: str = "auto"):
    """nf4_lora_bwd over a frozen base kept in bf16, w [n, k]."""
    return _lora_bwd((w,), dy, x, A, B, cfg, key, u, dx, dx_accumulate, dA, dB, dAB_accumulate, workspace,
                     stream, out_dtype, path=path)


# ---------------------------------------------------------------------------------
# pointwise block glue (fp32, contiguous)

def swiglu_fwd(g: torch.Tensor, u: torch.Tensor, out: Optional[torch.Tensor] = None, stream=None):
    """a = silu(g) * u, element for element the value of the unfused two-step chain."""
    _req(g, "g", torch.float32, tuple(g.shape))
    _req(u, "u", torch.float32, tuple(g.shape))
    a = torch.empty_like(g) if out is None else out
    _req(a, "a", torch.float32, tuple(g.shape))
    check("msq_swiglu_fwd", lib().msq_swiglu_fwd(_ptr(g), _ptr(u), g.numel(), _ptr(a), _stream(stream)))
    return a


def swiglu_bwd(da: torch.Tensor, g: torch.Tensor, u: torch.Tensor, in_place: bool = False, stream=None):
    """(dg, du) of a = silu(g) * u; in_place writes dg over g and du over u."""
    for nm, t in (("da", da), ("g", g), ("u", u)):
        _req(t, nm, torch.float32, tuple(g.shape))
    dg, du = (g, u) if in_place else (torch.empty_like(g), torch.empty_like(g))
    check("msq_swiglu_bwd", lib().msq_swiglu_bwd(_ptr(da), _ptr(g), _ptr(u), g.numel(), _ptr(dg), _ptr(du),
                                                 _stream(stream)))
    return dg, du


def _rope(fn: str, x: torch.Tensor, cos: torch.Tensor, sin: torch.Tensor, stream) -> torch.Tensor:
    if x.dim() != 3:
        raise ValueError(f"{fn}: x must be [t, heads, d], got {tuple(x.shape)}")
    t, h, d = x.shape
    _req(x, "x", torch.float32, (t, h, d))
    _req(cos, "cos", torch.float32, (t, d))
    _req(sin, "sin", torch.float32, (t, d))
    y = torch.empty_like(x)
    check(fn, getattr(lib(), fn)(_ptr(x), _ptr(cos), _ptr(sin), t, h, d, _ptr(y), _stream(stream)))
    return y


def rope_fwd(x: torch.Tensor, cos: torch.Tensor, sin: torch.Tensor, stream=None) -> torch.Tensor:
    """Rotary embedding of x [t, heads, d] (rotate-half pairs) with tables cos, sin [t, d]."""
    return _rope("msq_rope_fwd", x, cos, sin, stream)


def rope_bwd(dy: torch.Tensor, cos: torch.Tensor, sin: torch.Tensor, stream=None) -> torch.Tensor:
    """Gradient of rope_fwd with respect to x."""
    return _rope("msq_rope_bwd", dy, cos, sin, stream)



def rmsnorm_apply_fwd(h: torch.Tensor, r: torch.Tensor, w: torch.Tensor, stream=None) -> torch.Tensor:
    """y = (h * r) * w for h [t, d], r [t, 1] (the row's reciprocal RMS), w [d]."""
    t, d = h.shape
    _req(h, "h", torch.float32, (t, d))
    _req(r, "r", torch.float32, (t, 1))
    _req(w, "w", torch.float32, (d,))
    y = torch.empty_like(h)
    check("msq_rmsnorm_apply_fwd", lib().msq_rmsnorm_apply_fwd(_ptr(h), _ptr(r), _ptr(w), t, d, _ptr(y),
                                                               _stream(stream)))
    return y


def rmsnorm_apply_bwd(dy: torch.Tensor, h: torch.Tensor, r: torch.Tensor, w: torch.Tensor, stream=None):
    """(dh, hdot): dh = (dy * w) * r, hdot = (dy * w) * h; the caller sums hdot per row for dr."""
    t, d = h.shape
    _req(dy, "dy", torch.float32, (t, d))
    _req(h, "h", torch.float32, (t, d))
    _req(r, "r", torch.float32, (t, 1))
    _req(w, "w", torch.float32, (d,))
    dh, hdot = torch.empty_like(h), torch.empty_like(h)
    check("msq_rmsnorm_apply_bwd", lib().msq_rmsnorm_apply_bwd(_ptr(dy), _ptr(h), _ptr(r), _ptr(w), t, d,
                                                               _ptr(dh), _ptr(hdot), _stream(stream)))
    return dh, hdot


def kernel_copy(src: torch.Tensor, dst: torch.Tensor, stream=None) -> torch.Tensor:
    """dst <- src by a kernel (msq_kernel_copy): each side a device tensor or pinned host
    memory (pinned_empty); same dtype and number of elements, contiguous."""
    for nm, t in (("src", src), ("dst", dst)):
        if not isinstance(t, torch.Tensor) or not t.is_contiguous():
            raise ValueError(f"{nm} must be a contiguous tensor")
    if src.dtype != dst.dtype or src.numel() != dst.numel():
        raise ValueError(f"src {src.dtype}[{src.numel()}] and dst {dst.dtype}[{dst.numel()}] differ")
    check("msq_kernel_copy", lib().msq_kernel_copy(_ptr(src), _ptr(dst), src.numel() * src.element_size(),
                                                   _stream(stream)))
    return dst


# ---------------------------------------------------------------------------------
# optimizer step

def _adamw_tensors(params, grads, ms, vs):
    arr = (_abi.AdamwTensor * len(params))()
    for i, (p, g, m, v) in enumerate(zip(params, grads, ms, vs)):
        n = p.numel()
        for nm, t in (("p", p), ("g", g), ("m", m), ("v", v)):
            _req(t, nm, torch.float32, tuple(p.shape))
        arr[i] = _abi.AdamwTensor(_ptr(p), _ptr(g), _ptr(m), _ptr(v), n)
    return arr


def adamw_partials(params: Sequence[torch.Tensor]) -> int:
    """Number of g^2 partial sums adamw_step writes for these tensors."""
    arr = (_abi.AdamwTensor * len(params))()
    for i, p in enumerate(params):
        arr[i].n = p.numel()
    return int(lib().msq_adamw_partials(arr, len(params)))


def adamw_step(params: Sequence[torch.Tensor], grads: Sequence[torch.Tensor], ms: Sequence[torch.Tensor],
               vs: Sequence[torch.Tensor], step: int, lr: float, betas: Tuple[float, float], eps: float,
               weight_decay: float, gsq: Optional[torch.Tensor] = None, stream=None) -> None:
    """AdamW (msq_adamw_step) in place on fp32 params and moments; gsq, if given, receives
    adamw_partials(params) partial sums of the gradients' squares."""
    arr = _adamw_tensors(params, grads, ms, vs)
    if gsq is not None:
        _req(gsq, "gsq", torch.float32, (adamw_partials(params),))
    cfg = _abi.AdamwCfg(lr, betas[0], betas[1], eps, weight_decay)
    check("msq_adamw_step", lib().msq_adamw_step(arr, len(params), cfg, step, _ptr(gsq), _stream(stream)))


def nf4_stream_load(jobs: Sequence[Tuple[torch.Tensor, torch.Tensor, torch.Tensor]], chunk_bytes: int = 32 << 20,
                    host_threads: int = 8, stream=None, device=None) -> dict:
    """Streamed quantizing load: jobs of (w bf16 host [rows, cols], codes uint8 host
    [rows, cols/2], absmax fp32 host [rows, cols/64]); each w is quantized on the device
    chunk by chunk into its codes and absmax.  chunk_bytes bounds the bf16 bytes of one
    chunk (two chunks are staged at a time).  Returns the staging sizes used."""
    if not jobs:
        return {"device_bytes": 0, "host_bytes": 0, "chunk_rows": 0}
    arr = (_abi.QuantJob * len(jobs))()
    max_cols = 0
    for i, (w, codes, absmax) in enumerate(jobs):
        if w.dim() != 2:
            raise ValueError(f"job {i}: w must be 2-D")
        rows, cols = w.shape
        for nm, t, dt, shp in (("w", w, torch.bfloat16, (rows, cols)), ("codes", codes, torch.uint8, (rows, cols // 2)),
                               ("absmax", absmax, torch.float32, (rows, cols // 64))):
            if t.device.type != "cpu" or t.dtype != dt or tuple(t.shape) != shp or not t.is_contiguous():
                raise ValueError(f"job {i}: {nm} must be a contiguous host {dt} tensor of shape {shp}")
        arr[i] = _abi.QuantJob(w.data_ptr(), rows, cols, codes.data_ptr(), absmax.data_ptr())
        max_cols = max(max_cols, cols)
    chunk_rows = max(1, chunk_bytes // (2 * max_cols))
    dev_need = int(lib().nf4_stream_load_device_bytes(max_cols, chunk_rows))
    host_need = int(lib().nf4_stream_load_host_bytes(max_cols, chunk_rows))
    if dev_need == 0:
        raise ValueError(f"cols must be a multiple of 64 (widest job has {max_cols})")
    dev = torch.device(device or "cuda")
    staging = torch.empty(dev_need, dtype=torch.uint8, device=dev)
    bounce = torch.empty(host_need, dtype=torch.uint8, pin_memory=True)
    check("nf4_stream_load", lib().nf4_stream_load(arr, len(jobs), chunk_rows, _ptr(staging), dev_need,
                                                   _ptr(bounce), host_need, host_threads, _stream(stream)))
    del staging, bounce
    return {"device_bytes": dev_need, "host_bytes": host_need, "chunk_rows": chunk_rows}

def pinned_empty(nbytes: int) -> torch.Tensor:
    """A uint8 CPU tensor of nbytes in pinned host memory from msq_host_alloc: exactly that
    size (torch's pinned allocator rounds each block up to a power of two).  The memory is
    released with msq_host_free when the last view of the tensor is gone."""
    nbytes = int(nbytes)
    p = ctypes.c_void_p()
    check("msq_host_alloc", lib().msq_host_alloc(nbytes, ctypes.byref(p)))
    addr = int(p.value)

    def _release(_self, addr=addr, finalizing=sys.is_finalizing, free=lib().msq_host_free):
        # at interpreter exit module globals may already be gone: everything this needs is
        # bound here, and the process's pinned memory goes with the process anyway
        if not finalizing():
            free(addr)

    owner = type("PinnedHostBytes", (ctypes.c_uint8 * nbytes,), {"__del__": _release}).from_address(addr)
    return torch.frombuffer(owner, dtype=torch.uint8)


class BlockStreamWindow:
    """block_stream_* over pinned host blobs and a caller-owned device arena; layer l is
    copied on copy_streams[l % len(copy_streams)]."""

    def __init__(self, host_blobs: Sequence[torch.Tensor], window_blocks: int, n_slots: int = 2,
                 arena: Optional[torch.Tensor] = None, copy_stream: Optional[torch.cuda.Stream] = None,
                 device=None, copy_streams: Optional[Sequence[torch.cuda.Stream]] = None):
        self.n_layers = len(host_blobs)
        self.window_blocks = int(window_blocks)
        self.n_slots = int(n_slots)
        for i, b in enumerate(host_blobs):
            if b.device.type != "cpu" or b.dtype != torch.uint8 or not b.is_contiguous():
                raise ValueError(f"host blob {i} must be a contiguous uint8 CPU tensor (in pinned memory)")
        self.host_blobs = list(host_blobs)
        self._ptrs = (ctypes.c_void_p * self.n_layers)(*[b.data_ptr() for b in host_blobs])
        self._sizes = (ctypes.c_size_t * self.n_layers)(*[b.numel() for b in host_blobs])
        self.arena_bytes_needed = int(lib().block_stream_arena_bytes(self._sizes, self.n_layers,
                                                                     self.window_blocks, self.n_slots))
        if self.arena_bytes_needed == 0:
            raise ValueError(f"invalid window: {self.n_layers} layers, {self.window_blocks} per window, "
                             f"{self.n_slots} slots (at least 2 slots, 1 <= window_blocks <= layers)")
        dev = torch.device(device or "cuda")
        if arena is None:
            arena = torch.empty(self.arena_bytes_needed, dtype=torch.uint8, device=dev)
        if arena.device.type != "cuda" or arena.dtype != torch.uint8:
            raise ValueError("arena must be a device uint8 tensor")
        self.arena = arena
        if copy_streams is None:
            copy_streams = [copy_stream or torch.cuda.Stream(device=arena.device)]
        self.copy_streams = list(copy_streams)
        self.copy_stream = self.copy_streams[0]
        self._streams = (ctypes.c_void_p * len(self.copy_streams))(*[cs.cuda_stream for cs in self.copy_streams])
        h = ctypes.c_void_p()
        check("block_stream_create", lib().block_stream_create(
            ctypes.byref(h), self._ptrs, self._sizes, self.n_layers, self.window_blocks, self.n_slots,
            arena.data_ptr(), arena.numel(), self._streams, len(self.copy_streams)))
        self._h = h

    def prefetch(self, first_layer: int) -> None:
        check("block_stream_prefetch", lib().block_stream_prefetch(self._h, first_layer))

    def acquire(self, layer: int, stream=None) -> int:
        p = ctypes.c_void_p()
        check("block_stream_acquire", lib().block_stream_acquire(self._h, layer, _stream(stream),
                                                                 ctypes.byref(p)))
        return int(p.value)

    def acquire_view(self, layer: int, stream=None) -> torch.Tensor:
        """The layer's bytes inside the arena as a uint8 tensor view."""
        addr = self.acquire(layer, stream)
        off = addr - self.arena.data_ptr()
        return self.arena[off: off + self.host_blobs[layer].numel()]

    def release(self, first_layer: int, stream=None) -> None:
        check("block_stream_release", lib().block_stream_release(self._h, first_layer, _stream(stream)))

    def release_layer(self, layer: int, stream=None) -> None:
        check("block_stream_release_layer", lib().block_stream_release_layer(self._h, layer, _stream(stream)))

    def stats(self) -> dict:
        s = _abi.WindowStats()
        check("block_stream_stats", lib().block_stream_stats(self._h, ctypes.byref(s)))
        return {"bytes_copied": s.bytes_copied, "windows_copied": s.windows_copied,
                "windows_reused": s.windows_reused, "copy_ms": s.copy_ms, "copies_timed": s.copies_timed,
                "busy_ms": s.busy_ms}

    def close(self) -> None:
        if getattr(self, "_h", None):
            h, self._h = self._h, None
            check("block_stream_destroy", lib().block_stream_destroy(h))
            self.host_blobs = []
            self.arena = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def timing_enable(on=True) -> None:
    """True/1: time every launch; 2: only the dense GEMM launches; False/0: off."""
    check("msq_timing_enable", lib().msq_timing_enable(int(on)))


def timing_reserve(events: int) -> None:
    """Pool at least `events` timing events ahead of a timed region (two per launch)."""
    check("msq_timing_reserve", lib().msq_timing_reserve(int(events)))


def timing_collect() -> dict:
    """Per label "<kernel> <shape>": launches, total_ms, total_flops, total_bytes (then reset)."""
    cap = 256
    arr = (_abi.KernelTiming * cap)()
    n = ctypes.c_int()
    check("msq_timing_collect", lib().msq_timing_collect(arr, cap, ctypes.byref(n)))
    out = {}
    for i in range(min(n.value, cap)):
        e = arr[i]
        out[e.name.decode()] = {"launches": int(e.launches), "total_ms": e.total_ms,
                                "total_flops": e.total_flops, "total_bytes": e.total_bytes}
    return out
