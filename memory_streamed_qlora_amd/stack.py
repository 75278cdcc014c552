"""Streamed (and resident) training step of a Qwen2.5-shaped NF4 + LoRA stack.

The step the pages describe ("Poros" research post, the training-step paragraph;
package README, "How it works"):
  forward   blocks run in order while their frozen NF4 weights stream through a
            device window of n_slots slots (block_stream_prefetch on a side stream); only
            block-boundary activations are kept; each window is released (a pointer
            release -- the base is read-only) as soon as its blocks have run
  loss      frozen bf16 lm_head + mean next-token cross-entropy
  backward  windows in reverse: reload, recompute each block's forward with the same
            dropout keys (the counter-based masks replay exactly), then differentiate
            the adapters and the block input only
  update    one AdamW step on the fp32 adapters (the library's msq_adamw_step), identical
            to the resident run's; each layer's step runs as soon as its gradients are
            final, inside the backward, and also yields the partial sums of the squared
            gradients for the step's gradient norm.
Resident mode runs the same code with every layer's blob already in device memory.
Gradient accumulation over M micro-batches runs micro-batch by micro-batch or
block-major (every micro-batch through a window before the next window), with the
same bits either way; dropout masks are keyed by the micro-batch index.

Every projection goes through the library (nf4_lora_fwd / nf4_lora_bwd) with fp32
activations in and out; the library rounds them to bf16 only as the MFMA operand of
the frozen-base product.  The pointwise glue -- the SwiGLU product, rotary embedding
from precomputed tables, RMSNorm's scaling by the row's reciprocal RMS and the weights,
and the two residual adds per block (fused into the output pass of the o and down
projections) -- runs in the library too (glue="native"); each
fused chain reproduces the unfused PyTorch chain element for element (the pages allow
only such fusions, "Poros" README, Roadmap, "The Poros kernel"), and glue="torch" runs
that unfused chain.  The rest -- RMSNorm's mean, causal GQA attention, embedding
gather, lm_head and cross-entropy -- holds reductions, so it stays unfused fp32 PyTorch,
deterministic.  Block constants (eps 1e-6, RoPE base 1e6) and optimizer settings are
readings of the Qwen2 family and of textbook AdamW; the pages name neither.
"""
from __future__ import annotations

import math
import time
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np
import torch

from . import ops

PROJS = ops.PROJS
PROJ_ID = ops.PROJ_ID
EPS = 1e-6
ROPE_THETA = 1.0e6
LR, BETAS, ADAM_EPS, WD = 2e-4, (0.9, 0.999), 1e-8, 0.01


@dataclass(frozen=True)
class Shape:
    """Qwen2.5-family geometry."""

    hidden: int
    heads: int
    kv_heads: int
    head_dim: int
    inter: int
    layers: int
    vocab: int = 152064

    def proj_shape(self, proj: str) -> Tuple[int, int]:
        """(K = in_features, N = out_features)"""
        h, q, kv = self.hidden, self.heads * self.head_dim, self.kv_heads * self.head_dim
        return {"q": (h, q), "k": (h, kv), "v": (h, kv), "o": (q, h), "gate": (h, self.inter),
                "up": (h, self.inter), "down": (self.inter, h)}[proj]


QWEN25_05B = Shape(896, 14, 2, 64, 4864, 24)
QWEN25_7B = Shape(3584, 28, 4, 128, 18944, 28)
QWEN25_32B = Shape(5120, 40, 8, 128, 27648, 64)
QWEN25_72B = Shape(8192, 64, 8, 128, 29568, 80)


def _align(x: int, a: int = 256) -> int:
    return (x + a - 1) // a * a


class LayerLayout:
    """One layer's frozen base as a single contiguous blob (the unit the window
    streams): for q, k, v, o, gate, up, down in order, packed NF4 codes [N, K/2] then
    fp32 absmax [N, K/64] (base "nf4"), or the bf16 matrix [N, K] (base "bf16"); then the
    bf16 q/k/v biases.  Every segment starts on a 256-byte boundary."""

    def __init__(self, shape: Shape, base: str = "nf4"):
        assert base in ("nf4", "bf16")
        self.base = base
        self.segs: Dict[Tuple[str, str], Tuple[int, int, torch.dtype, Tuple[int, ...]]] = {}
        off = 0
        for proj in PROJS:
            K, N = shape.proj_shape(proj)
            if base == "bf16":
                self.segs[(proj, "w")] = (off, 2 * N * K, torch.bfloat16, (N, K))
                off = _align(off + 2 * N * K)
                continue
            self.segs[(proj, "codes")] = (off, N * K // 2, torch.uint8, (N, K // 2))
            off = _align(off + N * K // 2)
            self.segs[(proj, "absmax")] = (off, N * K // 16, torch.float32, (N, K // 64))
            off = _align(off + N * K // 16)
        for proj in ("q", "k", "v"):
            N = shape.proj_shape(proj)[1]
            self.segs[(proj, "bias")] = (off, 2 * N, torch.bfloat16, (N,))
            off = _align(off + 2 * N)
        self.nbytes = off

    def views(self, blob: torch.Tensor) -> Dict[Tuple[str, str], torch.Tensor]:
        out = {}
        for key, (off, nb, dt, shp) in self.segs.items():
            out[key] = blob[off: off + nb].view(dt).view(shp)
        return out


# ---------------------------------------------------------------------------------
# autograd bridge to the library

def _fwd(base, x, bias, A, B, cfg, key, **kw):
    """The library's forward for an NF4 (codes, absmax) or bf16 (w,) base."""
    if len(base) == 2:
        return ops.nf4_lora_fwd(x, base[0], base[1], bias, A, B, cfg, key, **kw)
    return ops.bf16_lora_fwd(x, base[0], bias, A, B, cfg, key, **kw)


def _bwd(base, dy, x, A, B, cfg, key, **kw):
    if len(base) == 2:
        return ops.nf4_lora_bwd(dy, x, base[0], base[1], A, B, cfg, key, **kw)
    return ops.bf16_lora_bwd(dy, x, base[0], A, B, cfg, key, **kw)


class _LoraLinear(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, A, B, base, bias, residual, cfg, key, value_unused, u_given):
        if value_unused:
            # selective recompute: the backward reads only x and u, never y, so the
            # frozen-base product is skipped and y is a zero placeholder (with u kept
            # from the first forward, nothing runs at all)
            u = u_given if u_given is not None else _fwd(base, x, bias, A, B, cfg, key, u_only=True)[1]
            y = x.new_zeros(()).expand(x.shape[0], base[0].shape[0])
        elif u_given is not None:
            # u kept from the first forward (the same bits the product would give again)
            y, u = _fwd(base, x, bias, A, B, cfg, key, u_out=u_given, u_given=True, residual=residual)
        else:
            y, u = _fwd(base, x, bias, A, B, cfg, key, want_u=True, residual=residual)
        ctx.save_for_backward(x, A, B, u)
        ctx.base, ctx.cfg, ctx.key = base, cfg, key
        return y

    @staticmethod
    def backward(ctx, dy):
        x, A, B, u = ctx.saved_tensors
        dy = dy.contiguous()
        dx, dA, dB = _bwd(ctx.base, dy, x, A, B, ctx.cfg, ctx.key, u=u)
        # y = residual + (...): the residual's gradient is dy itself
        dres = dy if ctx.needs_input_grad[5] else None
        return dx, dA, dB, None, None, dres, None, None, None, None


def lora_linear(x, A, B, base: Tuple[torch.Tensor, ...], bias, cfg: ops.Lora, key,
                value_unused: bool = False, residual: Optional[torch.Tensor] = None,
                u_keep: Optional[list] = None, u_given: Optional[torch.Tensor] = None) -> torch.Tensor:
    """[residual +] the projection over an NF4 (codes, absmax) or bf16 (w,) frozen base;
    with a residual the add happens in the library's output pass.  u_keep (a list, outside
    autograd): u is appended to it; u_given: u from an earlier forward of the same x, used
    instead of forming it."""
    if torch.is_grad_enabled() and (x.requires_grad or A.requires_grad or B.requires_grad or
                                    (residual is not None and residual.requires_grad)):
        return _LoraLinear.apply(x, A, B, base, bias, residual, cfg, key, value_unused and cfg.r > 0,
                                 u_given if cfg.r > 0 else None)
    want = u_keep is not None and cfg.r > 0
    y, u = _fwd(base, x, bias, A, B, cfg, key, want_u=want, residual=residual)
    if want:
        u_keep.append(u)
    return y


class _Spec:
    """One projection of a group: its base, bias and dropout key."""

    __slots__ = ("base", "bias", "key")

    def __init__(self, base, bias, key):
        self.base, self.bias, self.key = base, bias, key


class _LoraLinearGroup(torch.autograd.Function):
    """Projections of one input (q/k/v, gate/up): the forward is one grouped library pass,
    and so is the backward (lora_bwd_group: the projections' input gradients summed by one
    GEMM over their concatenated rows, each projection's dA / dB as in a single call)."""

    @staticmethod
    def forward(ctx, x, specs, cfg, us_given, *AB):
        projs = [{"base": sp.base, "bias": sp.bias, "key": sp.key, "A": AB[2 * i], "B": AB[2 * i + 1]}
                 for i, sp in enumerate(specs)]
        if us_given is not None:
            for pr, u in zip(projs, us_given):
                pr["u"] = u
            outs = ops.lora_fwd_group(x, projs, cfg, u_given=True)
        else:
            outs = ops.lora_fwd_group(x, projs, cfg, want_u=True)
        ctx.save_for_backward(x, *AB, *[u for _, u in outs])
        ctx.specs, ctx.cfg = specs, cfg
        return tuple(y for y, _ in outs)

    @staticmethod
    def backward(ctx, *dys):
        P = len(ctx.specs)
        saved = ctx.saved_tensors
        x, AB, us = saved[0], saved[1:1 + 2 * P], saved[1 + 2 * P:]
        projs = [{"base": sp.base, "A": AB[2 * i], "B": AB[2 * i + 1], "key": sp.key, "dy": dys[i].contiguous(),
                  "u": us[i]} for i, sp in enumerate(ctx.specs)]
        dx, dAB = ops.lora_bwd_group(x, projs, ctx.cfg)
        return (dx, None, None, None, *[g for pair in dAB for g in pair])


def lora_linear_group(x, specs, As, Bs, cfg: ops.Lora, u_keep: Optional[list] = None,
                      us_given: Optional[Sequence[torch.Tensor]] = None):
    """The projections of one input x, grouped: a tuple of outputs.  u_keep / us_given as
    in lora_linear, one u per projection."""
    if torch.is_grad_enabled() and (x.requires_grad or any(a.requires_grad or b.requires_grad
                                                           for a, b in zip(As, Bs))):
        AB = [t for pair in zip(As, Bs) for t in pair]
        return _LoraLinearGroup.apply(x, specs, cfg, tuple(us_given) if (us_given and cfg.r > 0) else None, *AB)
    projs = [{"base": sp.base, "bias": sp.bias, "key": sp.key, "A": a, "B": b} for sp, a, b in zip(specs, As, Bs)]
    want = u_keep is not None and cfg.r > 0
    outs = ops.lora_fwd_group(x, projs, cfg, want_u=want)
    if want:
        u_keep.extend(u for _, u in outs)
    return tuple(y for y, _ in outs)


class _SwiGLU(torch.autograd.Function):
    """a = silu(g) * u.  in_place: the backward writes dg over g and du over u, for callers
    whose g and u feed nothing else (the layer's gate and up outputs), which keeps two
    [T, intermediate] fp32 buffers out of the backward's peak."""

    @staticmethod
    def forward(ctx, g, u, in_place=False):
        ctx.save_for_backward(g, u)
        ctx.in_place = in_place
        return ops.swiglu_fwd(g, u)

    @staticmethod
    def backward(ctx, da):
        g, u = ctx.saved_tensors
        dg, du = ops.swiglu_bwd(da.contiguous(), g, u, in_place=ctx.in_place)
        return dg, du, None


class _RMSNormApply(torch.autograd.Function):
    """y = (h * r) * w with r = the row's reciprocal RMS, computed outside by PyTorch."""

    @staticmethod
    def forward(ctx, h, r, w):
        ctx.save_for_backward(h, r, w)
        return ops.rmsnorm_apply_fwd(h, r, w)

    @staticmethod
    def backward(ctx, dy):
        h, r, w = ctx.saved_tensors
        dh, hdot = ops.rmsnorm_apply_bwd(dy.contiguous(), h, r, w)
        # r's gradient: the row sum the product's own gradient takes (a reduction, in PyTorch)
        dr = hdot.sum(-1, keepdim=True) if ctx.needs_input_grad[1] else None
        return dh, dr, None


class _RoPE(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, cos, sin):
        ctx.save_for_backward(cos, sin)
        return ops.rope_fwd(x, cos, sin)

    @staticmethod
    def backward(ctx, dy):
        cos, sin = ctx.saved_tensors
        return ops.rope_bwd(dy.contiguous(), cos, sin), None, None


# ---------------------------------------------------------------------------------
# block glue (fp32 except where it feeds the library in bf16)

def rmsnorm(h: torch.Tensor, w: torch.Tensor) -> torch.Tensor:
    """The unfused PyTorch chain."""
    return h * torch.rsqrt(torch.mean(h * h, dim=-1, keepdim=True) + EPS) * w


def rmsnorm_native(h: torch.Tensor, w: torch.Tensor) -> torch.Tensor:
    """The same chain with its pointwise tail fused in the library; the mean and rsqrt
    (over [T, 1]) stay in PyTorch."""
    r = torch.rsqrt(torch.mean(h * h, dim=-1, keepdim=True) + EPS)
    return _RMSNormApply.apply(h, r, w)


def rope_tables(T: int, D: int, device) -> Tuple[torch.Tensor, torch.Tensor]:
    inv = ROPE_THETA ** (-np.arange(0, D, 2, dtype=np.float64) / D)
    ang = np.arange(T, dtype=np.float64)[:, None] * inv[None, :]
    cos = np.concatenate([np.cos(ang), np.cos(ang)], 1).astype(np.float32)
    sin = np.concatenate([np.sin(ang), np.sin(ang)], 1).astype(np.float32)
    return torch.from_numpy(cos).to(device), torch.from_numpy(sin).to(device)


def rope(x: torch.Tensor, cos: torch.Tensor, sin: torch.Tensor) -> torch.Tensor:
    """x [T, H, D] with rotate-half pairs (i, i + D/2); the unfused PyTorch chain."""
    h = x.shape[-1] // 2
    rot = torch.cat([-x[..., h:], x[..., :h]], dim=-1)
    return x * cos[:, None, :] + rot * sin[:, None, :]


def causal_gqa_attention(q, k, v, mask_rep):
    """q [T,H,D], k/v [T,KV,D] fp32 -> [T, H*D] fp32; key/value head j serves query heads
    j*g .. j*g+g-1 (g = H/KV).  The g query heads that share a key/value head are stacked
    along the rows of one operand, so each product is a batch of KV GEMMs over g*T rows
    (no expanded copies of k and v), and the scale and the causal mask (mask_rep: the
    additive [T, T] mask repeated for the g heads, [g*T, T]) are applied by the score
    product itself (baddbmm)."""
    T, H, D = q.shape
    KV = k.shape[1]
    g = H // KV
    qh = q.permute(1, 0, 2).reshape(KV, g * T, D)
    kt = k.permute(1, 2, 0).contiguous()
    vh = v.permute(1, 0, 2).contiguous()
    s = torch.baddbmm(mask_rep, qh, kt, alpha=1.0 / math.sqrt(D))
    p = torch.softmax(s, dim=-1)
    o = torch.bmm(p, vh)
    return o.view(H, T, D).permute(1, 0, 2).reshape(T, H * D)


_COPY_STREAMS: Dict[Tuple[int, int], torch.cuda.Stream] = {}


def copy_streams(device, n: int) -> List[torch.cuda.Stream]:
    """n copy streams of a device, shared by every stack of the process: a stream keeps the
    hardware queue it was first given, so fresh streams per stack could end up sharing the
    compute stream's queue once earlier stacks hold the others."""
    dev = torch.device(device)
    idx = dev.index if dev.index is not None else torch.cuda.current_device()
    out = []
    for i in range(n):
        if (idx, i) not in _COPY_STREAMS:
            _COPY_STREAMS[(idx, i)] = torch.cuda.Stream(device=torch.device("cuda", idx))
        out.append(_COPY_STREAMS[(idx, i)])
    return out


class _HostBound:
    """A block-boundary activation parked in pinned host memory during the forward."""

    __slots__ = ("host",)

    def __init__(self, host: torch.Tensor):
        self.host = host


@dataclass
class StepResult:
    loss: float
    grad_norm: float
    seconds: float
    window_stats: Optional[dict] = None


class Stack:
    """A Qwen2.5-shaped NF4 + LoRA stack with streamed or resident frozen base."""

    def __init__(self, shape: Shape, seq: int, r: int = 16, alpha: float = 32.0, p_drop: float = 0.0,
                 window_blocks: int = 4, mode: str = "streamed", seed: int = 0, device=None,
                 n_slots: int = 2, glue: str = "native", base: str = "nf4", group: bool = True,
                 layer_release: bool = True, lm_stream: Optional[bool] = None, n_copy_streams: int = 2,
                 keep_grads: bool = True, checkpoint_every: int = 1, offload_bounds: bool = False,
                 device_bounds: int = 4, keep_u: bool = True):
        assert mode in ("streamed", "resident")
        assert glue in ("native", "torch")
        self.shape, self.seq, self.mode, self.seed = shape, seq, mode, seed
        self.glue = glue
        self.group = group
        # keep each projection's u from the step's first forward for the recompute (T x r
        # fp32 per projection: 7 x 32 KB per layer at 512 tokens), which then skips the
        # rank-r products
        self.keep_u = keep_u
        self._u_kept: Dict[Tuple[int, int], Dict[str, torch.Tensor]] = {}
        self.layer_release = layer_release
        # the frozen lm_head in pinned host memory, streamed by the loss (streamed stacks by
        # default); False keeps it on the device
        self.lm_stream = (mode == "streamed") if lm_stream is None else lm_stream
        self.cfg = ops.Lora(r, alpha, p_drop)
        self.window_blocks = window_blocks
        self.n_slots = n_slots
        self.n_copy_streams = n_copy_streams
        # False: a layer's gradients are dropped once its AdamW step (inside the backward)
        # has used them, so only one layer's gradients are ever held
        self.keep_grads = keep_grads
        # the forward keeps the input of every checkpoint_every-th layer (layers l with
        # l % checkpoint_every == 0); the backward recomputes the others from the checkpoint
        # below them, in no-grad forwards, when it enters their group.  Groups never
        # straddle a window, so a group's layers are all in the window being processed.
        if checkpoint_every < 1 or window_blocks % checkpoint_every:
            raise ValueError(f"checkpoint_every={checkpoint_every} must be >= 1 and divide "
                             f"window_blocks={window_blocks}")
        self.checkpoint_every = checkpoint_every
        # offload_bounds: the forward parks every kept block-boundary activation except the
        # top device_bounds layers' in pinned host memory, and the backward brings each back
        # when it reaches it, both by kernel copies on the compute stream (msq_kernel_copy:
        # the GPU's own loads and stores over the link, not queued behind the window's
        # engine copies).  The bits do not change; the device then holds a few boundaries
        # instead of all of them at the turnaround, the step's peak.
        self.offload_bounds = offload_bounds
        self.device_bounds = device_bounds
        self._host_bounds: Optional[torch.Tensor] = None
        self.dev = torch.device(device or "cuda")
        self.layout = LayerLayout(shape, base)
        self.host_blobs: List[torch.Tensor] = []
        self.dev_blobs: List[torch.Tensor] = []
        self.window: Optional[ops.BlockStreamWindow] = None
        self.ln1: List[torch.Tensor] = []
        self.ln2: List[torch.Tensor] = []
        self.A: List[Dict[str, torch.nn.Parameter]] = []
        self.B: List[Dict[str, torch.nn.Parameter]] = []
        self.emb = self.lm = self.lnf = None
        self.lm_host: Optional[torch.Tensor] = None
        self._lm_ring = None
        self.lm_copy_timing = False  # time each lm_head chunk copy (events on the copy stream)
        self._lm_copy_log: List[Tuple[torch.cuda.Event, torch.cuda.Event, int]] = []
        self.cos, self.sin = rope_tables(seq, shape.head_dim, self.dev)
        self.mask_add = torch.triu(torch.full((seq, seq), float("-inf"), device=self.dev), 1)
        self._mask_reps: Dict[int, torch.Tensor] = {}
        # AdamW state per layer: the moments (created at the layer's first update, zeros) and
        # the partial sums of g^2 its last update wrote
        self._m: List[Optional[List[torch.Tensor]]] = []
        self._v: List[Optional[List[torch.Tensor]]] = []
        self._gsq: List[torch.Tensor] = []
        self.step_index = 0

    # -- construction ------------------------------------------------------------
    def _store_layer(self, blob_dev: torch.Tensor) -> None:
        if self.mode == "resident":
            self.dev_blobs.append(blob_dev)
        else:
            host = ops.pinned_empty(blob_dev.numel())
            host.copy_(blob_dev)
            self.host_blobs.append(host)

    def add_layer(self, W: Dict[str, torch.Tensor], bias: Dict[str, torch.Tensor], A, B, ln1, ln2):
        """W[proj] bf16 [N, K] on the device -> NF4 into a fresh blob (nf4_quantize), or
        copied as it is for a bf16 base."""
        blob = torch.zeros(self.layout.nbytes, dtype=torch.uint8, device=self.dev)
        v = self.layout.views(blob)
        for proj in PROJS:
            if self.layout.base == "bf16":
                v[(proj, "w")].copy_(W[proj])
            else:
                ops.nf4_quantize(W[proj], v[(proj, "codes")], v[(proj, "absmax")])
        for proj in ("q", "k", "v"):
            v[(proj, "bias")].copy_(bias[proj])
        self._store_layer(blob)
        self.A.append({p: torch.nn.Parameter(A[p].to(self.dev, torch.float32).contiguous()) for p in PROJS})
        self.B.append({p: torch.nn.Parameter(B[p].to(self.dev, torch.float32).contiguous()) for p in PROJS})
        self.ln1.append(ln1.to(self.dev, torch.float32))
        self.ln2.append(ln2.to(self.dev, torch.float32))

    def set_globals(self, emb: torch.Tensor, lm: torch.Tensor, lnf: torch.Tensor) -> None:
        """The frozen token embedding stays in host memory (a step gathers only its T rows
        and copies them over).  The frozen lm_head lives on the device in resident mode; in
        streamed mode it stays in pinned host memory and the loss streams it chunk by chunk
        through a two-chunk device ring, like the base (lm_stream).  The final norm is on the
        device."""
        self.emb = emb.detach().to("cpu", torch.bfloat16).contiguous()
        if self.lm_stream:
            self.lm_host = ops.pinned_empty(lm.numel() * 2).view(torch.bfloat16).view(lm.shape)
            self.lm_host.copy_(lm)
            self.lm = None
        else:
            self.lm = lm.to(self.dev, torch.bfloat16).contiguous()
        self.lnf = lnf.to(self.dev, torch.float32)

    def _mask_rep(self, T: int) -> torch.Tensor:
        """The causal mask of T tokens repeated for the query heads of one key/value head."""
        if T not in self._mask_reps:
            g = self.shape.heads // self.shape.kv_heads
            self._mask_reps[T] = self.mask_add[:T, :T].repeat(g, 1).contiguous()
        return self._mask_reps[T]

    def _embed(self, tokens: torch.Tensor) -> torch.Tensor:
        """Rows of the host embedding for `tokens` (host or device), as fp32 on the device."""
        idx = tokens if tokens.device.type == "cpu" else tokens.cpu()
        rows = self.emb.index_select(0, idx).pin_memory()
        return rows.to(self.dev, non_blocking=True).float()

    def finalize(self) -> None:
        # one AdamW launch per layer: a layer's update runs as soon as its gradients are
        # final (inside the backward, overlapping the window's copies)
        L = len(self.A)
        self._m, self._v = [None] * L, [None] * L
        self._gsq = [torch.zeros(ops.adamw_partials(self._layer_params(l)), dtype=torch.float32, device=self.dev)
                     for l in range(L)]
        if self.mode == "streamed" or self.lm_stream:
            self.copy_streams = copy_streams(self.dev, self.n_copy_streams)
            self.copy_stream = self.copy_streams[0]

        if self.mode == "streamed":
            self.window = ops.BlockStreamWindow(self.host_blobs, self.window_blocks, self.n_slots,
                                                copy_streams=self.copy_streams, device=self.dev)

    @classmethod
    def random(cls, shape: Shape, seq: int, seed: int = 0, cfg_id: int = 0, w_std: float = 0.02,
               **kw) -> "Stack":
        """Random-weight stack generated layer by layer on the device (the base is
        drawn, quantized with nf4_quantize (or kept in bf16) and, when streamed, moved to
        pinned host memory one layer at a time, so the device never holds more than one
        layer)."""
        st = cls(shape, seq, seed=seed, **kw)
        dev = st.dev
        gen = st._generators(cfg_id)

        for l in range(shape.layers):
            W, bias = {}, {}
            A, B = st._draw_adapters(l, gen)
            for i, proj in enumerate(PROJS):
                K, N = shape.proj_shape(proj)
                W[proj] = (torch.randn(N, K, generator=gen(l, 16 * i), device=dev) * w_std).to(torch.bfloat16)
                if proj in ("q", "k", "v"):
                    bias[proj] = (torch.randn(N, generator=gen(l, 16 * i + 1), device=dev) * 0.02).to(torch.bfloat16)
            ln1 = 1 + 0.02 * torch.randn(shape.hidden, generator=gen(l, 200), device=dev)
            ln2 = 1 + 0.02 * torch.randn(shape.hidden, generator=gen(l, 201), device=dev)
            st.add_layer(W, bias, A, B, ln1, ln2)
            del W
        ge = gen(10000, 0)
        emb = (torch.randn(shape.vocab, shape.hidden, generator=ge, device=dev) * 0.02).to(torch.bfloat16)
        lm = (torch.randn(shape.vocab, shape.hidden, generator=gen(10000, 1), device=dev) * 0.02).to(torch.bfloat16)
        lnf = 1 + 0.02 * torch.randn(shape.hidden, generator=gen(10000, 2), device=dev)
        st.set_globals(emb, lm, lnf)
        st.finalize()
        return st

    def _generators(self, cfg_id: int):
        """gen(layer, tensor_id): the device generator every drawn tensor comes from."""
        def gen(layer, tid):
            g = torch.Generator(device=self.dev)
            g.manual_seed((self.seed * 1000003 + cfg_id * 10007 + layer * 101 + tid) & 0x7FFFFFFFFFFFFFFF)
            return g
        return gen

    def _draw_adapters(self, l: int, gen):
        """Layer l's LoRA adapters: A ~ U(+-1/sqrt(K)), B ~ N(0, 0.01)."""
        r = self.cfg.r
        A, B = {}, {}
        for i, proj in enumerate(PROJS):
            K, N = self.shape.proj_shape(proj)
            A[proj] = (torch.rand(r, K, generator=gen(l, 16 * i + 2), device=self.dev) * 2 - 1) / math.sqrt(K)
            B[proj] = torch.randn(N, r, generator=gen(l, 16 * i + 3), device=self.dev) * 0.01
        return A, B

    @staticmethod
    def tensor_name(layer: int, proj: str, kind: str = "weight") -> str:
        """A projection's name in a Qwen2-style checkpoint (the loader's source naming)."""
        mod = "mlp" if proj in ("gate", "up", "down") else "self_attn"
        return f"model.layers.{layer}.{mod}.{proj}_proj.{kind}"

    @classmethod
    def load_base(cls, shape: Shape, source, loader: str = "streamed", device=None, chunk_bytes: int = 32 << 20,
                  host_threads: int = 8) -> List[torch.Tensor]:
        """Every layer's NF4 base (LayerLayout, with the q/k/v biases) as a pinned host
        blob, quantized from a host bf16 source: source(name) returns a contiguous host
        tensor under the Qwen2 checkpoint names (tensor_name).

        loader "streamed" (the pages' default): nf4_stream_load quantizes each layer's
        projections chunk by chunk straight into the layer's pinned blob; the device holds
        only the two staging slots.  "standard": every base matrix is first moved to the
        device (the whole bf16 base materialised there), then quantized with nf4_quantize
        and the blobs copied back.  Both give the same bytes."""
        if loader not in ("streamed", "standard"):
            raise ValueError(f"loader must be 'streamed' or 'standard', got {loader!r}")
        dev = torch.device(device or "cuda")
        layout = LayerLayout(shape)
        L = shape.layers
        W_dev = None
        if loader == "standard":
            W_dev = {(l, p): source(cls.tensor_name(l, p)).to(dev) for l in range(L) for p in PROJS}
        blobs = []
        for l in range(L):
            if loader == "streamed":
                blob = ops.pinned_empty(layout.nbytes).zero_()
                v = layout.views(blob)
                ops.nf4_stream_load([(source(cls.tensor_name(l, p)), v[(p, "codes")], v[(p, "absmax")])
                                     for p in PROJS], chunk_bytes=chunk_bytes, host_threads=host_threads,
                                    device=dev)
            else:
                blob_dev = torch.zeros(layout.nbytes, dtype=torch.uint8, device=dev)
                vd = layout.views(blob_dev)
                for p in PROJS:
                    ops.nf4_quantize(W_dev.pop((l, p)), vd[(p, "codes")], vd[(p, "absmax")])
                blob = ops.pinned_empty(layout.nbytes)
                blob.copy_(blob_dev)
                del blob_dev
                v = layout.views(blob)
            for p in ("q", "k", "v"):
                v[(p, "bias")].copy_(source(cls.tensor_name(l, p, "bias")))
            blobs.append(blob)
        return blobs

    @classmethod
    def load(cls, shape: Shape, seq: int, source, loader: str = "streamed", seed: int = 0, cfg_id: int = 0,
             chunk_bytes: int = 32 << 20, host_threads: int = 8, **kw) -> "Stack":
        """A stack whose frozen NF4 base comes from load_base (same source and loaders);
        the norms and the frozen embedding / lm_head come from the source
        (model.layers.{l}.input_layernorm.weight / post_attention_layernorm.weight,
        model.embed_tokens.weight, lm_head.weight, model.norm.weight), the adapters are
        drawn as in random()."""
        st = cls(shape, seq, seed=seed, **kw)
        if st.layout.base != "nf4":
            raise ValueError("the quantizing loader builds an NF4 base")
        dev = st.dev
        blobs = cls.load_base(shape, source, loader, dev, chunk_bytes, host_threads)
        gen = st._generators(cfg_id)
        for l, blob in enumerate(blobs):
            if st.mode == "resident":
                st.dev_blobs.append(blob.to(dev))
            else:
                st.host_blobs.append(blob)
            A, B = st._draw_adapters(l, gen)
            st.A.append({p: torch.nn.Parameter(A[p].contiguous()) for p in PROJS})
            st.B.append({p: torch.nn.Parameter(B[p].contiguous()) for p in PROJS})
            st.ln1.append(source(f"model.layers.{l}.input_layernorm.weight").to(dev, torch.float32))
            st.ln2.append(source(f"model.layers.{l}.post_attention_layernorm.weight").to(dev, torch.float32))
        del blobs
        st.set_globals(source("model.embed_tokens.weight"), source("lm_head.weight"), source("model.norm.weight"))
        st.finalize()
        return st

    # -- one layer -----------------------------------------------------------------
    def _base(self, views, proj):
        return ((views[(proj, "w")],) if self.layout.base == "bf16" else
                (views[(proj, "codes")], views[(proj, "absmax")]))

    def _lin_group(self, x, l, views, projs, step, micro, keep=None, given=None):
        """Projections of one input: one grouped pass (group=True) or one call each.  keep:
        a dict that receives each projection's u; given: such a dict from the first forward."""
        if not self.group:
            return tuple(self._lin(x, l, views, p, step, micro, keep=keep, given=given) for p in projs)
        specs = [_Spec(self._base(views, p), views.get((p, "bias")), ops.rng_key(self.seed, step, micro, l, PROJ_ID[p]))
                 for p in projs]
        uk = [] if keep is not None else None
        ys = lora_linear_group(x, specs, [self.A[l][p] for p in projs], [self.B[l][p] for p in projs], self.cfg,
                               u_keep=uk, us_given=[given[p] for p in projs] if given else None)
        if uk:
            keep.update(zip(projs, uk))
        return ys

    def _lin(self, x, l, views, proj, step, micro, value_unused=False, residual=None, keep=None, given=None):
        key = ops.rng_key(self.seed, step, micro, l, PROJ_ID[proj])
        bias = views.get((proj, "bias"))
        base = self._base(views, proj)
        uk = [] if keep is not None else None
        ug = given[proj] if given else None
        if residual is not None and self.glue == "torch":
            y = residual + lora_linear(x, self.A[l][proj], self.B[l][proj], base, bias, self.cfg, key,
                                       value_unused, u_keep=uk, u_given=ug)
        else:
            y = lora_linear(x, self.A[l][proj], self.B[l][proj], base, bias, self.cfg, key, value_unused, residual,
                            u_keep=uk, u_given=ug)
        if uk:
            keep[proj] = uk[0]
        return y

    def layer_forward(self, h: torch.Tensor, l: int, views, step: int, micro: int = 0,
                      recompute: bool = False, keep_u: bool = False) -> torch.Tensor:
        """Activations stay fp32; the library rounds them to bf16 only as MFMA operands.

        recompute=True (the backward's rerun, with autograd recording): the layer's
        output value is never read -- only its graph is -- so the down projection's
        frozen-base product is skipped and the returned value is not the layer output.
        keep_u (the step's first forward): each projection's u = drop(x) A^T is kept until
        the recompute, which then uses it in place of forming it again (the same bits: the
        same kernels on the same inputs)."""
        sh = self.shape
        T = h.shape[0]
        keep = {} if (keep_u and self.keep_u and self.cfg.r > 0) else None
        given = self._u_kept.pop((l, micro), None) if recompute else None
        norm = rmsnorm_native if self.glue == "native" else rmsnorm
        xn = norm(h, self.ln1[l])
        q, k, v = self._lin_group(xn, l, views, ("q", "k", "v"), step, micro, keep, given)
        q = q.view(T, sh.heads, sh.head_dim)
        k = k.view(T, sh.kv_heads, sh.head_dim)
        v = v.view(T, sh.kv_heads, sh.head_dim)
        cos, sin = self.cos[:T], self.sin[:T]
        if self.glue == "native":
            q, k = _RoPE.apply(q, cos, sin), _RoPE.apply(k, cos, sin)
        else:
            q, k = rope(q, cos, sin), rope(k, cos, sin)
        att = causal_gqa_attention(q, k, v, self._mask_rep(T))
        h1 = self._lin(att, l, views, "o", step, micro, residual=h, keep=keep, given=given)
        xn2 = norm(h1, self.ln2[l])
        g, u = self._lin_group(xn2, l, views, ("gate", "up"), step, micro, keep, given)
        a = _SwiGLU.apply(g, u, True) if self.glue == "native" else torch.nn.functional.silu(g) * u
        out = self._lin(a, l, views, "down", step, micro, value_unused=recompute, residual=h1, keep=keep,
                        given=given)
        if keep is not None:
            self._u_kept[(l, micro)] = keep
        return out

    # -- base residency --------------------------------------------------------------
    def _views(self, l: int):
        if self.mode == "resident":
            return self.layout.views(self.dev_blobs[l])
        return self.layout.views(self.window.acquire_view(l))

    def _windows(self) -> List[int]:
        return list(range(0, self.shape.layers, self.window_blocks))

    # -- the step ----------------------------------------------------------------------
    def forward_backward(self, tokens: torch.Tensor, step: int, micro: int = 0) -> torch.Tensor:
        """One micro-batch: accumulates adapter gradients into .grad; returns the loss
        (device scalar)."""
        return self._forward_backward([tokens], step, [micro], 1.0)[0]

    def _forward_backward(self, toks: List[torch.Tensor], step: int, micros: List[int],
                          scale: float, update_layers: bool = False) -> List[torch.Tensor]:
        """Block-major pass over the micro-batches toks (dropout keys micros): each window is
        fetched once and runs every micro-batch before the next window, forward and
        backward.  Streamed, each layer is acquired just before its first use and released
        right after its last, so a window's slot refills layer by layer.  Each micro-batch's loss is scaled by `scale` before its backward (1.0:
        no scaling op); gradients accumulate into .grad, for every adapter in micro-batch
        order.  update_layers: run each layer's AdamW step as soon as the last micro-batch's
        backward of that layer is done (its gradients are then final).  Returns the
        unscaled losses."""
        L = self.shape.layers
        M = len(toks)
        wins = self._windows()
        self._u_kept = {}
        streamed = self.mode == "streamed"
        # the streamed lm_head's two-chunk ring, made before the forward's work so that its
        # first copies need not wait for the compute stream to reach the loss, and dropped
        # after the last loss so that the backward's peak does not hold it
        self._lm_ring = self._lm_ring_make()
        hs = [self._embed(t) for t in toks]
        bounds: List[List[torch.Tensor]] = [[] for _ in range(M)]
        ahead = self.n_slots
        if streamed:
            for w in wins[:ahead]:
                self.window.prefetch(w)
        with torch.no_grad():
            for wi, w in enumerate(wins):
                layers = range(w, min(w + self.window_blocks, L))
                views = {}
                for m in range(M):
                    for l in layers:
                        if l not in views:  # acquired just before first use: waits for this layer only
                            views[l] = self._views(l)
                        bounds[m].append(self._keep_bound(hs[m], m, l, M) if l % self.checkpoint_every == 0
                                         else None)
                        hs[m] = self.layer_forward(hs[m], l, views[l], step, micros[m], keep_u=True)
                        if streamed and m == M - 1 and self.layer_release:
                            self.window.release_layer(l)
                if streamed and not self.layer_release:
                    self.window.release(w)
                if streamed and wi + ahead < len(wins):
                    self.window.prefetch(wins[wi + ahead])
        dhs: List[torch.Tensor] = []
        losses: List[torch.Tensor] = []
        for m in range(M):
            hf = hs[m].detach().requires_grad_()
            with torch.enable_grad():
                norm = rmsnorm_native if self.glue == "native" else rmsnorm
                hn = norm(hf, self.lnf)
            loss = self._lm_loss_backward(hn, toks[m], scale)
            dhs.append(hf.grad)
            losses.append(loss)
        hs = hf = hn = None
        self._lm_ring = None
        rw = wins[::-1]
        if streamed:
            for w in rw[:ahead]:
                self.window.prefetch(w)
        for wi, w in enumerate(rw):
            layers = range(w, min(w + self.window_blocks, L))
            views = {}
            for m in range(M):
                for l in reversed(layers):
                    if bounds[m][l] is None:
                        # the top of a checkpoint group: its inputs again from the checkpoint
                        c = l - l % self.checkpoint_every
                        with torch.no_grad():
                            for j in range(c, l):
                                if j not in views:
                                    views[j] = self._views(j)
                                bounds[m][j] = self._bound(bounds[m][j])
                                bounds[m][j + 1] = self.layer_forward(bounds[m][j], j, views[j], step, micros[m])
                    if l not in views:
                        views[l] = self._views(l)
                    x_in = self._bound(bounds[m][l]).detach().requires_grad_()
                    bounds[m][l] = None
                    with torch.enable_grad():
                        out = self.layer_forward(x_in, l, views[l], step, micros[m], recompute=True)
                    out.backward(dhs[m])
                    dhs[m] = x_in.grad
                    x_in = out = None
                    if streamed and m == M - 1 and self.layer_release:
                        self.window.release_layer(l)
                    if update_layers and m == M - 1:
                        self._update_layer(l)
            if streamed and not self.layer_release:
                self.window.release(w)
            if streamed and wi + ahead < len(rw):
                self.window.prefetch(rw[wi + ahead])
        self._u_kept = {}
        return losses

    def _keep_bound(self, h: torch.Tensor, m: int, l: int, M: int):
        """Layer l's input as the backward will need it: h itself, or (offloaded) parked in
        pinned host memory by a kernel copy in stream order, after which h's memory is free."""
        if not self.offload_bounds or l >= self.shape.layers - self.device_bounds:
            return h
        T, H = h.shape
        L = self.shape.layers
        need = M * L * T * H
        if self._host_bounds is None or self._host_bounds.numel() < need:
            self._host_bounds = ops.pinned_empty(need * 4).view(torch.float32)
        host = self._host_bounds[(m * L + l) * T * H:(m * L + l + 1) * T * H].view(T, H)
        ops.kernel_copy(h, host)
        return _HostBound(host)

    def _bound(self, b) -> torch.Tensor:
        """A kept boundary on the device: as it is, or a parked one copied back."""
        if isinstance(b, _HostBound):
            return ops.kernel_copy(b.host, torch.empty(b.host.shape, dtype=b.host.dtype, device=self.dev))
        return b

    LM_CHUNK = 4224  # vocabulary rows per lm_head chunk (152064 = 36 x 4224)

    def _lm_ring_make(self):
        """Two device buffers of LM_CHUNK lm_head rows and the event after which the copy
        stream may write them (None when the lm_head is on the device)."""
        if self.lm_host is None:
            return None
        rows = min(self.LM_CHUNK, self.shape.vocab)
        ring = [torch.empty(rows, self.shape.hidden, dtype=torch.bfloat16, device=self.dev) for _ in range(2)]
        made = torch.cuda.Event()
        made.record(torch.cuda.current_stream(self.dev))
        return ring, made

    def _lm_chunks(self):
        """(first row, lm_head rows) over the vocabulary in order: views of the device
        lm_head, or, with the lm_head in pinned host memory, chunks copied through a
        two-buffer device ring on the copy stream (a buffer is refilled only after the
        work that read its previous chunk).  The ring is made at the start of the step's
        forward (see _forward_backward) and dropped after the loss, so its memory is free
        again for the backward, where the step's peak sits."""
        V = self.shape.vocab
        starts = list(range(0, V, self.LM_CHUNK))
        if self.lm_host is None:
            for c0 in starts:
                yield c0, self.lm[c0:c0 + self.LM_CHUNK]
            return
        cur = torch.cuda.current_stream(self.dev)
        ring, made = self._lm_ring if self._lm_ring is not None else self._lm_ring_make()
        read: List[Optional[torch.cuda.Event]] = [made, made]
        copied = {}

        def issue(i: int) -> None:
            b, c0 = i % 2, starts[i]
            rows = min(self.LM_CHUNK, V - c0)
            with torch.cuda.stream(self.copy_stream):
                self.copy_stream.wait_event(read[b])
                t0 = None
                if self.lm_copy_timing:
                    t0 = torch.cuda.Event(enable_timing=True)
                    t0.record(self.copy_stream)
                ring[b][:rows].copy_(self.lm_host[c0:c0 + rows], non_blocking=True)
                ev = torch.cuda.Event(enable_timing=self.lm_copy_timing)
                ev.record(self.copy_stream)
                if t0 is not None:
                    self._lm_copy_log.append((t0, ev, ring[b][:rows].nbytes))
            copied[i] = ev

        for i in range(min(2, len(starts))):
            issue(i)
        for i, c0 in enumerate(starts):
            rows = min(self.LM_CHUNK, V - c0)
            cur.wait_event(copied.pop(i))
            yield c0, ring[i % 2][:rows]
            ev = torch.cuda.Event()
            ev.record(cur)
            read[i % 2] = ev
            if i + 2 < len(starts):
                issue(i + 2)

    def lm_copy_stats(self) -> Dict[str, float]:
        """Bytes, copies and copy-stream milliseconds of the lm_head chunk copies timed since
        the last call (lm_copy_timing on; call after the device has synchronised)."""
        ms = sum(a.elapsed_time(b) for a, b, _ in self._lm_copy_log)
        out = {"bytes": float(sum(n for _, _, n in self._lm_copy_log)), "copies": len(self._lm_copy_log), "ms": ms}
        self._lm_copy_log = []
        return out

    def _lm_rows(self, idx_cpu: torch.Tensor) -> torch.Tensor:
        """lm_head rows idx (bf16 [len(idx), hidden]) on the device."""
        if self.lm_host is None:
            return self.lm.index_select(0, idx_cpu.to(self.dev, non_blocking=True))
        return self.lm_host.index_select(0, idx_cpu).pin_memory().to(self.dev, non_blocking=True)

    def _lm_loss_backward(self, hn: torch.Tensor, tokens: torch.Tensor, scale: float) -> torch.Tensor:
        """Mean next-token cross-entropy of the frozen lm_head over hn [T, hidden] (fp32),
        back-propagated into hn's graph (its gradient scaled by `scale`, in fp32).  Returns
        the (unscaled) loss.

        One pass over the lm_head, LM_CHUNK vocabulary rows at a time, with a running
        (online) softmax per token: the logits of a chunk (fp32: hn enters the bf16 product
        with the bf16 lm_head as a hi/lo pair of bf16 values, two products with fp32 output,
        ~2^-16 relative) update the running maximum m and, rescaled by exp(m_old - m_new)
        as the maximum grows, the sums over the non-target rows
            Zo = sum exp(logit - m),   U = sum exp(logit - m) * lm_row,
        and the target's own term Zt = exp(l_target - m).  With Z = Zo + Zt, the loss of a
        token is m + log Z - l_target and
            d loss / d h_t = (U_t - Zo_t * lm_target) / (Z_t * n),
        i.e. sum_v softmax_v lm_v - lm_target with 1 - softmax_target = Zo / Z taken from the
        non-target sum itself: a confident prediction loses nothing to cancellation.  U
        takes the probabilities as a bf16 hi/lo pair (two bf16 products with fp32 output),
        ~2^-16 relative.  The lm_head is thus read once per step and never needs to be
        resident: streamed, it comes from pinned host memory (see _lm_chunks)."""
        T, H = hn.shape
        n = T - 1
        tg_cpu = tokens[1:].cpu()
        tgt = tg_cpu.to(self.dev, non_blocking=True)
        h = hn.detach()[:n]
        h_hi = h.to(torch.bfloat16)
        h_lo = (h - h_hi.float()).to(torch.bfloat16)
        m = torch.full((n,), float("-inf"), device=self.dev)
        Zo = torch.zeros(n, device=self.dev)
        Zt = torch.zeros(n, device=self.dev)
        U = torch.zeros(n, H, device=self.dev)
        lt = torch.zeros(n, device=self.dev)
        for c0, lm_c in self._lm_chunks():
            rows = lm_c.shape[0]
            lm_t = lm_c.t()
            logits = torch.mm(h_hi, lm_t, out_dtype=torch.float32) + torch.mm(h_lo, lm_t, out_dtype=torch.float32)
            rel = tgt - c0
            hit = (rel >= 0) & (rel < rows)
            idx = rel.clamp(0, rows - 1)[:, None]
            lt = torch.where(hit, logits.gather(1, idx)[:, 0], lt)
            m_new = torch.maximum(m, logits.amax(1))
            a = torch.exp(m - m_new)
            p = torch.exp(logits - m_new[:, None])
            Zt = torch.where(hit, p.gather(1, idx)[:, 0], Zt * a)
            p.scatter_(1, idx, p.gather(1, idx) * (~hit)[:, None].float())  # the target's own term apart
            Zo = Zo * a + p.sum(1)
            p_hi = p.to(torch.bfloat16)
            p_lo = (p - p_hi.float()).to(torch.bfloat16)
            U = U * a[:, None] + torch.mm(p_hi, lm_c, out_dtype=torch.float32) + \
                torch.mm(p_lo, lm_c, out_dtype=torch.float32)
            m = m_new
        Z = Zo + Zt
        loss = (m + torch.log(Z) - lt).sum() / n
        dh = (U - Zo[:, None] * self._lm_rows(tg_cpu).float()) / Z[:, None] * (scale / n)
        g = torch.zeros_like(hn)
        g[:n] = dh
        hn.backward(g)
        return loss

    def params(self) -> List[torch.nn.Parameter]:
        return [p for d in self.A for p in d.values()] + [p for d in self.B for p in d.values()]

    def _layer_params(self, l: int) -> List[torch.nn.Parameter]:
        """Layer l's adapters: A of every projection, then B, in PROJS order."""
        return list(self.A[l].values()) + list(self.B[l].values())

    def _update_layer(self, l: int) -> None:
        """Layer l's gradients are final: its AdamW step (one library launch, which also
        writes the partial sums of g^2 into _gsq[l]) and, unless the gradients are kept,
        dropping them."""
        params = self._layer_params(l)
        if self._m[l] is None:
            self._m[l] = [torch.zeros_like(p) for p in params]
            self._v[l] = [torch.zeros_like(p) for p in params]
        grads = [p.grad if p.grad is not None else torch.zeros_like(p) for p in params]
        ops.adamw_step([p.detach() for p in params], grads, self._m[l], self._v[l], self.step_index + 1, LR, BETAS,
                       ADAM_EPS, WD, gsq=self._gsq[l])
        if not self.keep_grads:
            for p in params:
                p.grad = None

    def grad_norm(self) -> torch.Tensor:
        """The 2-norm over every adapter gradient of the last update: the square root of the
        sum of the partial sums of g^2 the layers' updates wrote."""
        return torch.sqrt(torch.cat(self._gsq).sum())

    def train_step(self, tokens: torch.Tensor, order: str = "block") -> Tuple[torch.Tensor, torch.Tensor]:
        """One optimizer step; returns (loss, grad_norm) device scalars.

        tokens [T]: one micro-batch.  tokens [M, T]: gradient accumulation over M
        micro-batches (micro-batch m keys its dropout masks with micro = m), loss = the mean
        of the micro-batch losses.  order "micro" runs the micro-batches one after another,
        each streaming the whole base; "block" (block-major) runs all of them through each
        window while it is resident, streaming the base once per optimizer step.  Both
        orders give the same bits: every micro-batch computes the same values either way
        and every adapter gradient is summed in micro-batch order."""
        if order not in ("micro", "block"):
            raise ValueError(f"order must be 'micro' or 'block', got {order!r}")
        for p in self.params():
            p.grad = None
        if tokens.dim() == 1:
            loss = self._forward_backward([tokens], self.step_index, [0], 1.0, update_layers=True)[0]
        else:
            M = tokens.shape[0]
            scale = 1.0 / M
            if order == "micro":
                losses = [self._forward_backward([tokens[m]], self.step_index, [m], scale)[0] for m in range(M)]
                for l in range(len(self.A)):
                    self._update_layer(l)
            else:
                losses = self._forward_backward([tokens[m] for m in range(M)], self.step_index, list(range(M)),
                                                scale, update_layers=True)
            loss = losses[0] * scale
            for lm in losses[1:]:
                loss = loss + lm * scale
        gn = self.grad_norm()
        self.step_index += 1
        return loss, gn

    def state_tensors(self) -> Dict[str, torch.Tensor]:
        """Everything the bitwise gate compares: adapters, grads, AdamW moments."""
        out = {}
        for l in range(self.shape.layers):
            for i, (nm, p) in enumerate([("A", p) for p in PROJS] + [("B", p) for p in PROJS]):
                prm = (self.A if nm == "A" else self.B)[l][p]
                out[f"{l}.{p}.{nm}"] = prm.detach()
                if prm.grad is not None:
                    out[f"{l}.{p}.{nm}.grad"] = prm.grad.detach()
                if self._m[l] is not None:
                    out[f"{l}.{p}.{nm}.exp_avg"] = self._m[l][i].detach()
                    out[f"{l}.{p}.{nm}.exp_avg_sq"] = self._v[l][i].detach()
        return out

    def close(self) -> None:
        """Destroys the window (waiting for its copies) and gives the pinned host base and
        the device blobs back; pinned memory goes back to the system, not to PyTorch's
        pinned-block cache, so a following stack of other layer sizes can pin its own."""
        if self.window is not None:
            self.window.close()
            self.window = None
        torch.cuda.synchronize(self.dev)
        had_host = bool(self.host_blobs) or self.lm_host is not None
        self.host_blobs = []
        self.dev_blobs = []
        self.lm_host = None
        if had_host:
            torch._C._host_emptyCache()


def random_tokens(seed: int, step: int, T: int, vocab: int, device) -> torch.Tensor:
    g = torch.Generator(device="cpu")
    g.manual_seed(seed * 7919 + step)
    return torch.randint(0, vocab, (T,), generator=g).to(device)


def smoke_step(device) -> None:
    """Two tiny layers, one window each: a streamed step must equal the resident one."""
    sh = Shape(hidden=128, heads=2, kv_heads=1, head_dim=64, inter=256, layers=2, vocab=256)
    out = []
    for mode in ("resident", "streamed"):
        st = Stack.random(sh, 32, seed=3, r=8, alpha=16.0, p_drop=0.1, window_blocks=1, mode=mode,
                          device=device)
        toks = random_tokens(3, 0, 32, sh.vocab, st.dev)
        loss, gn = st.train_step(toks)
        torch.cuda.synchronize()
        out.append((loss.item(), gn.item(), st.state_tensors()))
        st.close()
    (l0, g0, s0), (l1, g1, s1) = out
    assert l0 == l1 and g0 == g1, f"streamed step differs from resident: {l0} vs {l1}, {g0} vs {g1}"
    for k in s0:
        assert torch.equal(s0[k], s1[k]), f"streamed != resident for {k}"
    print(f"[smoke] streamed == resident (bitwise): loss {l0:.6f} grad-norm {g0:.6e}", flush=True)
