"""Benchmark: streamed NF4 + LoRA training step of a Qwen2.5-32B-shaped stack on one GPU.

Workload: 64 decoder layers (hidden 5120, 40/8 heads, SwiGLU 27648), random N(0, 0.02)
base quantized to NF4 and held in pinned host memory, streamed one block at a time through
a device arena of 32 slots (one computing, the others prefetching or kept for the
turnaround), the block-boundary activations below the top 2 layers parked in pinned host
memory between the forward and the backward, the frozen lm_head streamed from pinned host
memory by the loss, each layer's adapter gradients dropped after its AdamW step; LoRA r16
alpha32 dropout 0.0 on all seven projections;
batch 1 x 512 random tokens over a 152064-entry vocabulary; one AdamW step per
training step.  A step is the whole hot path: forward with streaming, loss, backward
with reload + recompute, AdamW.  tokens/s = 512 * steps / timed seconds.

Prints one JSON line (see the fields below); --gpus N > 1 exits: the library's path
runs on one GPU (no collectives).  --vendor-gemm instead compares the library's NF4 GEMMs at the step's projection
shapes with the vendor library's plain bf16 GEMM (torch.matmul -> hipBLASLt) of the same
dimensions.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

# The vendor BLAS behind torch's products (the step's attention and lm_head products) keeps
# one workspace per (handle, stream), 76 MiB each by default on this platform; these
# products run with 4 MiB, and the ~150 MB goes to the window instead.  Read when the first
# such product runs, so it is set before anything imports torch.
os.environ.setdefault("HIPBLASLT_WORKSPACE_SIZE", "4096")  # KiB

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "train tokens/s (s/step) streamed NF4-LoRA fwd+bwd, 32B shape; MFMA util"
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBPS = 8000.0
PAGES_A100_S_PER_STEP = 2.0489  # Official A100 results, Benchmark matrix, Qwen2.5-32B streamed
GEMM_SOURCES = ("memory_streamed_qlora_amd/csrc/gemm.hip", "memory_streamed_qlora_amd/csrc/device_common.hpp")
COUNTERS_FILE = "profiles/nf4_gemm_qwen32b_step_counters.md"


def gemm_source_hash() -> str:
    import hashlib

    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str):
    """HBM bytes per launch of `kernel` from the committed counter summary, if it was
    taken on the current kernel sources (else None)."""
    path = os.path.join(ROOT, COUNTERS_FILE)
    if not os.path.exists(path):
        return None
    want = gemm_source_hash()
    for line in open(path):
        parts = line.split()
        if len(parts) == 5 and parts[0] == "traffic_bytes_per_launch" and parts[1] == kernel:
            if parts[3] == "sources" and parts[4] == want:
                return float(parts[2])
    return None


# Qwen2.5 stacks of the workloads: (hidden, heads, kv heads, head dim, intermediate, layers,
# dropout, default window: layers per slot, slots, checkpoint every n layers, boundaries
# parked in host memory, boundaries kept on the device when parking).  The 32B and 72B windows hold the most layers whose peak stays
# under the pages' streamed peaks for those sizes (10.95 GB, A100 results, Benchmark matrix;
# 18.87 GB, "Poros" research post, memory paragraph); the 7B stack keeps the plain double
# buffer of 4-layer windows (7 slots would hold all 28 of its layers).
SHAPES = {"7b": (3584, 28, 4, 128, 18944, 28, 0.1, (4, 2, 1, False, 4)),
          "32b": (5120, 40, 8, 128, 27648, 64, 0.0, (1, 32, 1, True, 2)),
          "72b": (8192, 64, 8, 128, 29568, 80, 0.1, (1, 31, 1, True, 4))}

PROJ_NAMES = {(5120, 5120): "q/o", (1024, 5120): "k/v", (27648, 5120): "gate/up", (5120, 27648): "down",
              (7168, 5120): "q+k+v", (55296, 5120): "gate+up"}


def by_kernel(kt: dict) -> dict:
    """Aggregate the per-label timing ("<kernel> <shape>") per kernel."""
    agg = {}
    for label, v in kt.items():
        a = agg.setdefault(label.split(" ")[0], {"launches": 0, "total_ms": 0.0, "total_flops": 0.0,
                                                 "total_bytes": 0.0})
        for f in a:
            a[f] += v[f]
    return agg


def hbm_kernels(kt: dict, steps: int) -> dict:
    """Achieved HBM bandwidth (algorithmic bytes / time) of the memory-bound kernels."""
    out = {}
    for name, v in sorted(by_kernel(kt).items()):
        if v["total_flops"] > 0:
            continue
        gbs = v["total_bytes"] / (v["total_ms"] * 1e-3) / 1e9
        out[name] = {"launches_per_step": v["launches"] / steps, "ms_per_step": round(v["total_ms"] / steps, 2),
                     "avg_us": round(v["total_ms"] / v["launches"] * 1e3, 1),
                     "algorithmic_MB_per_launch": round(v["total_bytes"] / v["launches"] / 1e6, 2),
                     "GBps": round(gbs, 1), "frac": round(gbs / PEAK_HBM_GBPS, 4)}
    return out


def gemm_shapes(kt: dict, steps: int) -> list:
    """MFMA utilisation of every projection shape and direction in the timed region."""
    out = []
    for label, v in sorted(kt.items()):
        if v["total_flops"] == 0:
            continue
        kern, shape = label.split(" ")
        t, n, k = (int(x) for x in shape.split("x"))
        tf = v["total_flops"] / (v["total_ms"] * 1e-3) / 1e12
        out.append({"kernel": kern, "projection": PROJ_NAMES.get((n, k), f"{n}x{k}"), "t": t, "n": n, "k": k,
                    "launches_per_step": v["launches"] / steps,
                    "avg_us": round(v["total_ms"] / v["launches"] * 1e3, 1),
                    "tflops": round(tf, 1), "frac": round(tf / PEAK_BF16_TFLOPS, 4)})
    return out


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def h2d_ceiling_gbps(torch, s, nbytes=1 << 30, reps=10) -> float:
    """Median pinned host->device copy rate of one 1 GiB buffer with nothing else running,
    copied on stream s (the window's first copy stream)."""
    h = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    h.fill_(1)
    d = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    ts = []
    for i in range(reps + 2):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(s):
            e0.record()
            d.copy_(h, non_blocking=True)
            e1.record()
        e1.synchronize()
        if i >= 2:
            ts.append(e0.elapsed_time(e1))
    ts.sort()
    del h, d
    return nbytes / 1e6 / ts[len(ts) // 2]


def h2d_ceiling_under_compute_gbps(torch, s, nbytes=1 << 30, reps=5) -> float:
    """The same 1 GiB pinned copy while the compute stream runs bf16 GEMMs (queued before the
    copy and lasting longer than it): the rate the window's copies can expect during a step."""
    h = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    h.fill_(1)
    d = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    a = torch.randn(8192, 8192, device="cuda").to(torch.bfloat16)
    b = torch.randn(8192, 8192, device="cuda").to(torch.bfloat16)
    ts = []
    for i in range(reps + 1):
        torch.cuda.synchronize()
        for _ in range(48):                      # ~50 ms of matrix work on the compute stream
            torch.matmul(a, b)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(s):
            e0.record()
            d.copy_(h, non_blocking=True)
            e1.record()
        e1.synchronize()
        torch.cuda.synchronize()
        if i >= 1:
            ts.append(e0.elapsed_time(e1))
    ts.sort()
    del h, d, a, b
    return nbytes / 1e6 / ts[len(ts) // 2]


def copy_calibration(torch, nbytes=256 << 20) -> None:
    """A plain device copy of known size (256 MiB read + 256 MiB write) so hardware byte
    counters of the same run can be scaled."""
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    a.fill_(3)
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()


def cpu_baseline(seconds_hint=True) -> dict:
    """The oracle, untuned, on a bounded sample of the same workload: one Qwen2.5-32B-
    shaped layer at 512 tokens -- its first forward, the recompute and the backward
    (all seven NF4 + LoRA projections plus the block glue) -- then scaled to the step
    (64 layers; the lm_head and loss are added from one timed fp64 lm_head pass)."""
    import numpy as np

    import msq_inputs as mi
    from oracle import block as oblock
    from oracle import lora as olora
    from oracle import step as ostep

    try:
        from threadpoolctl import threadpool_info
        cores = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:
        cores = os.cpu_count() or 1
    sh, T = mi.QWEN25_32B, 512
    lo = mi.LoraSpec(16, 32.0, 0.0)
    t_setup = time.time()
    prm = mi.block_params(0, 4, 0, sh, lo)
    qp = oblock.quantize_params(prm)
    io = mi.block_io(0, 4, sh, T)
    log(f"cpu baseline setup {time.time() - t_setup:.1f}s")
    rk = olora.RngKey(seed=0, step=0)
    t0 = time.perf_counter()
    oblock.forward(io["x"], qp, sh, 0, lo.alpha, lo.p_drop, rk)
    _, cache = oblock.forward(io["x"], qp, sh, 0, lo.alpha, lo.p_drop, rk)
    oblock.backward(io["dy"], cache, qp, sh, 0, lo.alpha, lo.p_drop, rk)
    t_layer = time.perf_counter() - t0
    # lm_head + loss + its input gradient, on a 1/16 slice of the vocabulary, scaled
    V = sh.vocab // 16
    rng = np.random.default_rng(0)
    lm = mi.round_to_bf16((0.02 * rng.standard_normal((V, sh.hidden))).astype(np.float32))
    h = io["x"].astype(np.float64)
    t1 = time.perf_counter()
    logits = h @ lm.astype(np.float64).T
    toks = rng.integers(0, V, T)
    _, dlog = ostep.loss_and_dlogits(logits, toks)
    dlog @ lm.astype(np.float64)
    t_head = (time.perf_counter() - t1) * 16
    step_s = sh.layers * t_layer + t_head
    return {"value": T / step_s, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": (f"one Qwen2.5-32B-shaped layer at 512 tokens (forward, recompute, backward; "
                       f"{t_layer:.1f}s) x 64 layers + lm_head/loss on 1/16 of the vocabulary x 16 "
                       f"({t_head:.1f}s); extrapolated s/step {step_s:.0f}"),
            "s_per_step_extrapolated": step_s}


def h2d_busy(window, lm, ms_per_step: float, ceiling: float) -> dict:
    """Copy-stream busy time per step (events around each window copy and each lm_head
    chunk copy, taken after the copy's wait) and the H2D rate while copying, against the
    measured ceiling."""
    if not window or not window.get("copies_timed"):
        return {}
    # window copies: the union of their spans over the copy streams; the lm_head chunks are
    # added on top (they may overlap window copies on another stream, so this is an upper
    # bound on the busy time and a lower bound on the rate)
    busy = window["busy_ms"] + (lm["ms"] if lm else 0.0)
    nbytes = window["bytes_copied"] + (lm["bytes"] if lm else 0.0)
    rate = nbytes / (busy * 1e-3) / 1e9 if busy > 0 else 0.0
    return {"copy_busy_ms_per_step": round(busy, 1), "copy_busy_frac": round(busy / ms_per_step, 3),
            "GBps_while_copying": round(rate, 1), "frac_while_copying": round(rate / ceiling, 3)}


def rocprof_summary(d: str, timed: int = 5, total: int = 7, first: int = -1) -> int:
    """Summarise rocprofv3 CSV output found under directory d (kernel stats, per-dispatch
    kernel traces, counter collections, memory-copy traces) as markdown on stdout.  For a
    kernel trace of the bench, the GEMM kernels' average is also given over the dispatches
    of the timed steps: a run of `total` streamed steps (no resident leg) of which steps
    first .. first+timed-1 are timed (first defaults to total - timed: the last ones)."""
    import csv
    import glob

    for path in sorted(glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)):
        rows = list(csv.DictReader(open(path)))
        tot = sum(float(r["TotalDurationNs"]) for r in rows)
        print(f"### kernel stats ({os.path.relpath(path, d)})\n")
        print("| kernel | calls | avg us | total ms | % |")
        print("|---|---|---|---|---|")
        for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"]))[:25]:
            print(f"| {r['Name'][:90]} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                  f"{float(r['TotalDurationNs']) / 1e6:.1f} | {100 * float(r['TotalDurationNs']) / tot:.1f} |")
        print()
    for path in sorted(glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)):
        durs = {}
        for r in csv.DictReader(open(path)):
            for k in ("nf4_fwd_gemm", "nf4_bwd_gemm"):
                if f"::{k}(" in r["Kernel_Name"]:
                    durs.setdefault(k, []).append((int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
        print(f"### GEMM dispatches ({os.path.relpath(path, d)})\n")
        print(f"| kernel | dispatches | avg us (all) | dispatches of the {timed} timed of {total} steps | avg us (those) |")
        print("|---|---|---|---|---|")
        for k, v in sorted(durs.items()):
            v.sort()
            us = [(b - a) / 1e3 for a, b in v]
            per = len(us) // total
            f0 = total - timed if first < 0 else first
            last = us[f0 * per:(f0 + timed) * per]
            print(f"| {k} | {len(us)} | {sum(us) / len(us):.1f} | {len(last)} | {sum(last) / max(1, len(last)):.1f} |")
        print()
    for path in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
        agg = {}
        for r in csv.DictReader(open(path)):
            k = (r["Kernel_Name"][:90], r["Counter_Name"])
            a = agg.setdefault(k, [0, 0.0, set()])
            a[2].add(r.get("Dispatch_Id"))
            a[1] += float(r["Counter_Value"])
        print(f"### counters ({os.path.relpath(path, d)})\n")
        print("| kernel | counter | dispatches | avg per dispatch |")
        print("|---|---|---|---|")
        for (kname, cname), (_, total, disp) in sorted(agg.items(), key=lambda kv: -kv[1][1])[:30]:
            print(f"| {kname} | {cname} | {len(disp)} | {total / max(1, len(disp)):.1f} |")
        print()
    for path in sorted(glob.glob(os.path.join(d, "**", "*memory_copy_trace.csv"), recursive=True)):
        rows = list(csv.DictReader(open(path)))
        if not rows:
            continue
        cols = list(rows[0].keys())
        size_col = next((c for c in cols if c.lower() in ("bytes", "size", "copy_bytes")), None)
        print(f"### memory copies ({os.path.relpath(path, d)})\n\ncolumns: {', '.join(cols)}\n")
        print("| direction | copies | total GB | summed copy ms | union busy ms | avg GB/s (union) | first-to-last span ms |")
        print("|---|---|---|---|---|---|---|")
        by = {}
        for r in rows:
            by.setdefault(r.get("Direction", r.get("Kind", "?")), []).append(r)

        def union_ms(iv):
            iv = sorted(iv)
            tot, (cs, ce) = 0, iv[0]
            for a, b in iv[1:]:
                if a > ce:
                    tot, cs, ce = tot + ce - cs, a, b
                else:
                    ce = max(ce, b)
            return (tot + ce - cs) / 1e6

        for direc, rs in sorted(by.items()):
            iv = [(int(r["Start_Timestamp"]), int(r["End_Timestamp"])) for r in rs]
            busy = sum(b - a for a, b in iv) / 1e6
            ubusy = union_ms(iv)
            gb = sum(float(r[size_col]) for r in rs) / 1e9 if size_col else float("nan")
            rate = gb / (ubusy / 1e3) if ubusy > 0 else float("nan")
            span = (max(b for _, b in iv) - min(a for a, _ in iv)) / 1e6
            print(f"| {direc} | {len(rs)} | {gb:.2f} | {busy:.1f} | {ubusy:.1f} | {rate:.1f} | {span:.1f} |")
        print()
        # per stream, in start order: copy durations (the trace holds no sizes)
        print("| stream | copies | ms per copy: min | median | max |")
        print("|---|---|---|---|---|")
        bys = {}
        for r in rows:
            bys.setdefault(r.get("Stream_Id", "?"), []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e6)
        for sid, ds in sorted(bys.items()):
            ds.sort()
            print(f"| {sid} | {len(ds)} | {ds[0]:.2f} | {ds[len(ds) // 2]:.2f} | {ds[-1]:.2f} |")
        print()
    return 0


def window_copies(layers: int = 16, slots: int = 8, steps: int = 2) -> int:
    """The window's copies alone, for a profiler's memory-copy trace: `layers` pinned blobs of
    the Qwen2.5-32B layer size (274.28 MB) streamed through one-layer windows in `slots`
    slots on the stack's two copy streams, in a step's order (forward, then backward), each
    layer acquired and released on the compute stream with no work in between.  The H2D
    ceiling probes run first.  Prints one JSON line: bytes copied, copy busy time and GB/s,
    against the ceilings."""
    import torch

    from memory_streamed_qlora_amd import ops, stack as S

    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    cs = S.copy_streams(dev, 2)
    ceiling = h2d_ceiling_gbps(torch, cs[0])
    ceiling_busy = h2d_ceiling_under_compute_gbps(torch, cs[0])
    layout = S.LayerLayout(S.QWEN25_32B, "nf4")
    blobs = [ops.pinned_empty(layout.nbytes) for _ in range(layers)]
    for b in blobs:
        b.fill_(3)
    w = ops.BlockStreamWindow(blobs, 1, slots, copy_streams=cs)
    order = list(range(layers))
    torch.cuda.synchronize()
    s0 = w.stats()
    t0 = time.perf_counter()
    for _ in range(steps):
        for seq in (order, order[::-1]):
            for l in seq[:slots]:
                w.prefetch(l)
            for i, l in enumerate(seq):
                w.acquire(l)
                w.release_layer(l)
                if i + slots < len(seq):
                    w.prefetch(seq[i + slots])
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    s1 = w.stats()
    w.close()
    copied = s1["bytes_copied"] - s0["bytes_copied"]
    busy = s1["busy_ms"] - s0["busy_ms"]
    out = {"window_copies": {"layers": layers, "slots": slots, "copy_streams": 2, "steps": steps,
                             "blob_MB": round(layout.nbytes / 1e6, 2), "bytes_copied": copied,
                             "windows_copied": s1["windows_copied"] - s0["windows_copied"],
                             "windows_reused": s1["windows_reused"] - s0["windows_reused"],
                             "wall_s": round(dt, 3), "copy_busy_ms": round(busy, 1),
                             "GBps_while_copying": round(copied / (busy * 1e-3) / 1e9, 1) if busy else None,
                             "GBps_wall": round(copied / dt / 1e9, 1),
                             "ceiling_GBps": round(ceiling, 1), "ceiling_under_compute_GBps": round(ceiling_busy, 1)}}
    log(f"window copies: {copied / 1e9:.2f} GB in {dt * 1e3:.1f} ms ({out['window_copies']['GBps_wall']} GB/s; "
        f"{out['window_copies']['GBps_while_copying']} GB/s while copying), ceiling {ceiling:.1f} GB/s")
    print(json.dumps(out))
    return 0


def vendor_gemm(reps: int = 20) -> int:
    """The step's GEMM launches at T = 512 (Qwen2.5-32B shapes, projections grouped as the
    stack groups them) against torch.matmul in bf16 of the same M x N x K: the vendor's own
    dense GEMM with the weight already in bf16 (no dequantization, no LoRA term).  Ours:
    the NF4 GEMM kernel's average launch time (HIP events on its launches) and the whole
    library call (pack + products + GEMM + split reduction, torch events).  Prints one
    JSON line."""
    import torch

    from memory_streamed_qlora_amd import ops

    torch.cuda.set_device(0)
    T, H, I = 512, 5120, 27648
    g = torch.Generator(device="cuda").manual_seed(0)
    cfg = ops.Lora(16, 32.0, 0.0)

    def proj(n, k, i):
        W = (torch.randn(n, k, generator=g, device="cuda") * 0.02).to(torch.bfloat16)
        c, a = ops.nf4_quantize(W)
        return {"base": (c, a), "W": W, "A": torch.randn(16, k, generator=g, device="cuda") * 0.01,
                "B": torch.randn(n, 16, generator=g, device="cuda") * 0.01, "key": ops.rng_key(0, 0, 0, 0, i),
                "bias": None}

    x = torch.randn(T, H, generator=g, device="cuda").to(torch.bfloat16)
    a = torch.randn(T, I, generator=g, device="cuda").to(torch.bfloat16)
    qkv = [proj(H, H, 0), proj(1024, H, 1), proj(1024, H, 2)]
    o, gu, down = proj(H, H, 3), [proj(I, H, 4), proj(I, H, 5)], proj(H, I, 6)

    def dys(ps):
        return [dict(p, dy=torch.randn(T, p["W"].shape[0], generator=g, device="cuda").to(torch.bfloat16))
                for p in ps]

    def wcat(ps):
        return torch.cat([p["W"] for p in ps]).contiguous()

    cases = [  # (name, our call, vendor call)
        ("q+k+v fwd", lambda: ops.lora_fwd_group(x, qkv, cfg, want_u=False), (x, wcat(qkv).t())),
        ("o fwd", lambda: ops.nf4_lora_fwd(x, *o["base"], None, o["A"], o["B"], cfg, o["key"], want_u=False),
         (x, o["W"].t())),
        ("gate+up fwd", lambda: ops.lora_fwd_group(x, gu, cfg, want_u=False), (x, wcat(gu).t())),
        ("down fwd", lambda: ops.nf4_lora_fwd(a, *down["base"], None, down["A"], down["B"], cfg, down["key"],
                                              want_u=False), (a, down["W"].t())),
    ]
    qkv_b, gu_b = dys(qkv), dys(gu)
    dy_o, dy_d = dys([o])[0]["dy"], dys([down])[0]["dy"]
    cases += [
        ("q+k+v bwd", lambda: ops.lora_bwd_group(x, qkv_b, cfg), (torch.cat([p["dy"] for p in qkv_b], 1), wcat(qkv))),
        ("o bwd", lambda: ops.nf4_lora_bwd(dy_o, x, *o["base"], o["A"], o["B"], cfg, o["key"]), (dy_o, o["W"])),
        ("gate+up bwd", lambda: ops.lora_bwd_group(x, gu_b, cfg), (torch.cat([p["dy"] for p in gu_b], 1), wcat(gu))),
        ("down bwd", lambda: ops.nf4_lora_bwd(dy_d, a, *down["base"], down["A"], down["B"], cfg, down["key"]),
         (dy_d, down["W"])),
    ]

    def timed(fn) -> float:
        for _ in range(3):
            fn()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        s.record()
        for _ in range(reps):
            fn()
        e.record()
        torch.cuda.synchronize()
        return s.elapsed_time(e) / reps * 1e3  # us

    rows = []
    for name, ours, (lhs, rhs) in cases:
        m, kk = lhs.shape
        n = rhs.shape[1]
        flop = 2.0 * m * n * kk
        call_us = timed(ours)
        ops.timing_enable(True)
        ops.timing_collect()
        for _ in range(reps):
            ours()
        torch.cuda.synchronize()
        kt = by_kernel(ops.timing_collect())
        ops.timing_enable(False)
        gk = kt.get("nf4_fwd_gemm" if "fwd" in name else "nf4_bwd_gemm")
        gemm_us = gk["total_ms"] / gk["launches"] * 1e3
        vend_us = timed(lambda: torch.matmul(lhs, rhs))
        rows.append({"gemm": name, "m": m, "n": n, "k": kk, "nf4_gemm_us": round(gemm_us, 1),
                     "nf4_gemm_tflops": round(flop / gemm_us / 1e6, 1), "nf4_call_us": round(call_us, 1),
                     "hipblaslt_bf16_us": round(vend_us, 1), "hipblaslt_bf16_tflops": round(flop / vend_us / 1e6, 1)})
        log(json.dumps(rows[-1]))
    tot = {k: sum(r[k] for r in rows) for k in ("nf4_gemm_us", "nf4_call_us", "hipblaslt_bf16_us")}
    print(json.dumps({"vendor_gemm": rows, "per_layer_us": {k: round(v, 1) for k, v in tot.items()},
                      "note": "forward and backward launches of one 32B layer at T 512; hipBLASLt multiplies "
                              "bf16 weights (no dequantization, no LoRA term)"}))
    return 0


def skinny(reps: int = 50) -> int:
    """The small shapes of the path, whose roofline is HBM bandwidth, not the matrix cores:
    the single 896 x 896 NF4 + LoRA linear (r 16, alpha 32, dropout 0.0) and the seven
    projections of a Qwen2.5-0.5B-shaped block (q/o 896x896, k/v 128x896, gate/up 4864x896,
    down 896x4864, dropout 0.1), all at T = 512, forward and backward through the library
    entry points on the path the library picks by shape (and, for comparison, the time on
    each of the two paths, tiled and small-tile).  Per kernel: average launch time (HIP
    events on its launches), algorithmic bytes per launch (as the library records them) and
    the GB/s and TFLOP/s they give.  Prints one JSON line."""
    import torch

    from memory_streamed_qlora_amd import ops

    torch.cuda.set_device(0)
    T = 512
    g = torch.Generator(device="cuda").manual_seed(0)
    cases = [("cfg1 896x896", 896, 896, 0.0)] + [
        (f"0.5B {name}", k, n, 0.1) for name, k, n in
        (("q/o", 896, 896), ("k/v", 896, 128), ("gate/up", 896, 4864), ("down", 4864, 896))]
    rows = []
    for name, K, N, p in cases:
        cfg = ops.Lora(16, 32.0, p)
        W = (torch.randn(N, K, generator=g, device="cuda") * 0.02).to(torch.bfloat16)
        codes, absmax = ops.nf4_quantize(W)
        A = (torch.rand(16, K, generator=g, device="cuda") * 2 - 1) / K ** 0.5
        B = torch.randn(N, 16, generator=g, device="cuda") * 0.01
        x = torch.randn(T, K, generator=g, device="cuda").to(torch.bfloat16)
        dy = torch.randn(T, N, generator=g, device="cuda").to(torch.bfloat16)
        key = ops.rng_key(0, 0, 0, 0, 0)

        def step(path="auto"):
            y, u = ops.nf4_lora_fwd(x, codes, absmax, None, A, B, cfg, key, path=path)
            ops.nf4_lora_bwd(dy, x, codes, absmax, A, B, cfg, key, u=u, path=path)

        def timed(path):
            for _ in range(5):
                step(path)
            torch.cuda.synchronize()
            s_ev, e_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s_ev.record()
            for _ in range(reps):
                step(path)
            e_ev.record()
            torch.cuda.synchronize()
            return s_ev.elapsed_time(e_ev) / reps * 1e3

        per_path = {p_: round(timed(p_), 1) for p_ in ("tiled", "small")}
        call_us = timed("auto")
        # the same forward + backward captured once in a HIP graph and replayed: the GPU's
        # own time for the pair, without the host's per-call work (argument marshalling,
        # output allocation), which at these sizes takes about as long as the kernels
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for _ in range(3):
                step()
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        for _ in range(5):
            graph.replay()
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record()
        for _ in range(reps):
            graph.replay()
        g1.record()
        torch.cuda.synchronize()
        graph_us = g0.elapsed_time(g1) / reps * 1e3
        del graph
        ops.timing_enable(True)
        ops.timing_collect()
        for _ in range(reps):
            step()
        torch.cuda.synchronize()
        kt = by_kernel(ops.timing_collect())
        ops.timing_enable(False)
        kern = {}
        for kname, v in sorted(kt.items()):
            us = v["total_ms"] / v["launches"] * 1e3
            kern[kname] = {"launches_per_step": v["launches"] / reps, "avg_us": round(us, 2),
                           "algorithmic_MB_per_launch": round(v["total_bytes"] / v["launches"] / 1e6, 3),
                           "GBps": round(v["total_bytes"] / v["total_ms"] / 1e6, 1),
                           "hbm_frac": round(v["total_bytes"] / v["total_ms"] / 1e6 / PEAK_HBM_GBPS, 4),
                           **({"tflops": round(v["total_flops"] / v["total_ms"] / 1e9, 1)} if v["total_flops"] else {})}
        # the method's own bytes: what the forward and the backward read and write at the
        # boundary (x, the NF4 base, A, B, y, u; dy, x, base, A, B, u, dx, dA, dB), however
        # the library stages them internally
        r = 16
        base_b, a_b, b_b = N * K * 0.5625, r * K * 4, N * r * 4
        fwd_b = T * K * 2 + base_b + a_b + b_b + T * N * 2 + T * r * 4
        bwd_b = T * N * 2 + T * K * 2 + base_b + a_b + b_b + T * r * 4 + T * K * 2 + a_b + b_b
        method_gbps = (fwd_b + bwd_b) / (call_us * 1e-6) / 1e9
        rows.append({"shape": name, "t": T, "k": K, "n": N, "p_drop": p, "fwd_bwd_us": round(call_us, 1),
                     "fwd_bwd_us_graph": round(graph_us, 1),
                     "path": "small" if any(k_.startswith("small_") for k_ in kern) else "tiled",
                     "fwd_bwd_us_tiled": per_path["tiled"], "fwd_bwd_us_small": per_path["small"],
                     "method_MB": round((fwd_b + bwd_b) / 1e6, 3), "method_GBps": round(method_gbps, 1),
                     "method_GBps_graph": round((fwd_b + bwd_b) / (graph_us * 1e-6) / 1e9, 1),
                     "method_hbm_frac": round(method_gbps / PEAK_HBM_GBPS, 4), "kernels": kern})
        log(f"{name}: fwd+bwd {call_us:.1f} us, {graph_us:.1f} us as a replayed graph ({rows[-1]['path']}; tiled "
            f"{per_path['tiled']}, small {per_path['small']}), the method's {(fwd_b + bwd_b) / 1e6:.2f} MB at "
            f"{method_gbps:.0f} GB/s")
    print(json.dumps({"skinny": rows, "peak_hbm_GBps": PEAK_HBM_GBPS}))
    return 0


def main() -> int:
    if len(sys.argv) in (3, 5, 6) and sys.argv[1] == "--rocprof-summary":
        return rocprof_summary(sys.argv[2], *[int(a) for a in sys.argv[3:]])
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--shape", choices=tuple(SHAPES), default="32b",
                    help="Qwen2.5 stack shape: 32b (the headline), 7b or 72b (dropout 0.1, as their workloads state)")
    ap.add_argument("--layers", type=int, default=None, help="stack depth (default: the shape's)")
    ap.add_argument("--window-blocks", type=int, default=None,
                    help="layers per window slot (default: 1 at 32b and 72b, 4 at 7b)")
    ap.add_argument("--checkpoint-every", type=int, default=None,
                    help="the streamed step keeps every n-th layer's input for the backward and recomputes "
                         "the others (default 1; must divide --window-blocks)")
    ap.add_argument("--offload-bounds", choices=("on", "off"), default=None,
                    help="park the block-boundary activations (all but the top --device-bounds layers') in "
                         "pinned host memory during the forward (default: on at 32b and 72b, off at 7b)")
    ap.add_argument("--device-bounds", type=int, default=None,
                    help="with --offload-bounds: the top layers whose boundaries stay on the device "
                         "(default 2 at 32b, 4 at 72b)")
    ap.add_argument("--keep-grads", action="store_true",
                    help="keep every adapter gradient until the step ends (default: a layer's gradients are "
                         "dropped once its AdamW step inside the backward has used them)")
    ap.add_argument("--slots", type=int, default=None,
                    help="window slots in the device arena (default 32 at 32b, 31 at 72b: the most resident "
                         "layers whose peak stays under the pages' streamed peaks, 10.95 and 18.87 GB; 2 at 7b)")
    ap.add_argument("--copy-streams", type=int, default=2, help="copy streams of the window (layer l on stream l mod n)")
    ap.add_argument("--no-resident", action="store_true",
                    help="skip the resident leg (the same step with the whole base in device memory)")
    ap.add_argument("--no-literal-window", action="store_true",
                    help="skip the 32b leg with the two-slot window (4 layers x 2 slots)")
    ap.add_argument("--ga", type=int, default=1,
                    help="micro-batches of 512 tokens per optimizer step (gradient accumulation)")
    ap.add_argument("--order", choices=("block", "micro"), default="block",
                    help="accumulation loop order: block-major (one base stream per step) or micro-batch-major")
    ap.add_argument("--base", choices=("nf4", "bf16"), default="nf4",
                    help="frozen base format: NF4, or bf16 (the pages' bf16 streaming variant, 4x the bytes)")
    ap.add_argument("--glue", choices=("native", "torch"), default="native",
                    help="pointwise block glue: the library's fused kernels, or the unfused PyTorch chain")
    ap.add_argument("--window-release", action="store_true",
                    help="release whole windows instead of layer by layer")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-kernel-timing", action="store_true",
                    help="time the streamed steps without per-launch events (no roofline figures)")
    ap.add_argument("--lm-resident", action="store_true",
                    help="keep the frozen lm_head on the device in the streamed step (instead of streaming it)")
    ap.add_argument("--skinny", action="store_true",
                    help="only time the small (HBM-bound) shapes: the 896x896 linear and the 0.5B block's projections")
    ap.add_argument("--window-copies", action="store_true",
                    help="only stream 32B-sized layer blobs through the window (no compute), e.g. under a "
                         "profiler's memory-copy trace")
    ap.add_argument("--vendor-gemm", action="store_true",
                    help="only compare the NF4 GEMMs with hipBLASLt's bf16 GEMM at the step's shapes")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: the hot path runs on one GPU (the library has no multi-GPU path); --gpus must be 1", file=sys.stderr)
        return 2
    if args.vendor_gemm:
        return vendor_gemm()
    if args.skinny:
        return skinny()
    if args.window_copies:
        return window_copies()

    import statistics

    import torch

    from memory_streamed_qlora_amd import ops, stack as S

    torch.cuda.set_device(0)
    hid, heads, kvh, hd, inter, nl, p_drop, (wb_default, slots_default, ckpt_default, off_default,
                                             dbounds_default) = SHAPES[args.shape]
    if args.device_bounds is None:
        args.device_bounds = dbounds_default
    offload = off_default if args.offload_bounds is None else args.offload_bounds == "on"
    layers = args.layers or nl
    slots = args.slots or slots_default
    wblocks = args.window_blocks or wb_default
    ckpt = args.checkpoint_every or (ckpt_default if wblocks % ckpt_default == 0 else 1)
    shape = S.Shape(hid, heads, kvh, hd, inter, layers)
    size = args.shape.upper()
    T = 512
    # the window's copy streams first: a HIP stream keeps the hardware queue it is given on
    # first use (4 per process), so streams created before them could push one of them onto
    # the compute stream's queue; the ceiling copies run on the first of them
    cstreams = S.copy_streams(torch.device("cuda", 0), args.copy_streams)
    ceiling = h2d_ceiling_gbps(torch, cstreams[0])
    ceiling_busy = h2d_ceiling_under_compute_gbps(torch, cstreams[0])
    log(f"H2D ceiling (1 GiB pinned, median of 10): {ceiling:.1f} GB/s; under concurrent GEMMs: {ceiling_busy:.1f} GB/s")
    copy_calibration(torch)

    def batch(st, s: int):
        """One optimizer step's tokens: [T], or [ga, T] micro-batches."""
        if args.ga == 1:
            return S.random_tokens(0, s, T, shape.vocab, "cpu")
        return torch.stack([S.random_tokens(0, s * args.ga + m, T, shape.vocab, "cpu") for m in range(args.ga)])

    def run(mode: str, kernel_timing: bool, window_blocks: int, n_slots: int, checkpoint_every: int):
        t_build = time.time()
        st = S.Stack.random(shape, T, seed=0, cfg_id=4, r=16, alpha=32.0, p_drop=p_drop,
                            window_blocks=window_blocks, n_slots=n_slots, mode=mode, glue=args.glue,
                            base=args.base, layer_release=not args.window_release,
                            lm_stream=mode == "streamed" and not args.lm_resident, n_copy_streams=args.copy_streams,
                            keep_grads=args.keep_grads, checkpoint_every=checkpoint_every,
                            offload_bounds=offload and mode == "streamed" and n_slots == slots,
                            device_bounds=args.device_bounds)
        torch.cuda.synchronize()
        log(f"{mode} ({window_blocks} x {n_slots}, checkpoints every {checkpoint_every}): built {layers} layers "
            f"in {time.time() - t_build:.1f}s "
            f"(blob {st.layout.nbytes / 1e6:.2f} MB/layer)")
        per_step = 0
        for w in range(args.warmup):
            # the last warmup step of a timed leg counts its launches (timing on, times dropped)
            count = kernel_timing and w == args.warmup - 1
            if count:
                ops.timing_enable(True)
                ops.timing_collect()
            loss, gn = st.train_step(batch(st, w), order=args.order)
            torch.cuda.synchronize()
            if count:
                per_step = sum(v["launches"] for v in ops.timing_collect().values())
                ops.timing_enable(False)
            log(f"{mode}: warmup step {w} loss {loss.item():.4f} grad-norm {gn.item():.4e}")
        toks = [batch(st, 1000 + s) for s in range(args.steps)]
        stats0 = st.window.stats() if st.window else None
        st.lm_copy_timing = st.lm_host is not None
        st.lm_copy_stats()
        # the build's device temporaries leave the allocator's cache, so the reserved peak
        # below is the step's own
        if kernel_timing:
            # every timing event the timed steps need is made ahead (two per launch), so
            # that no event is created inside the timed region
            ops.timing_reserve(2 * max(per_step, 20000) * (args.steps + 1))
        torch.cuda.empty_cache()
        torch.cuda.reset_peak_memory_stats()
        # inside the timed region only the dense GEMM launches carry events (the roofline
        # kernel); the per-launch bookkeeping on the ~10^4 small launches of a step would
        # add host time to a step whose host issue is already close to its GPU time
        ops.timing_enable(2 if kernel_timing else 0)
        ops.timing_collect()
        free0 = torch.cuda.mem_get_info()[0]
        torch.cuda.synchronize()
        # one event per step boundary on the compute stream: per-step times without syncing
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        t0 = time.perf_counter()
        evs[0].record()
        losses = []
        for s in range(args.steps):
            loss, gn = st.train_step(toks[s], order=args.order)
            evs[s + 1].record()
            losses.append(loss)
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        ops.timing_enable(False)
        kt = ops.timing_collect()
        stats1 = st.window.stats() if st.window else None
        lmc = st.lm_copy_stats()
        step_ms = [evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)]
        kt_all = {}
        if kernel_timing:
            # after the timed region: two more steps with every launch timed, for the
            # memory-bound kernels' table
            ops.timing_enable(1)
            ops.timing_collect()
            for s in range(2):
                st.train_step(batch(st, 2000 + s), order=args.order)
            torch.cuda.synchronize()
            kt_all = ops.timing_collect()
            ops.timing_enable(False)
        out = {"seconds": dt, "losses": [l.item() for l in losses], "kernels": kt, "kernels_all": kt_all,
               "step_ms": step_ms,
               "peak_alloc_gb": torch.cuda.max_memory_allocated() / 1e9,
               "peak_reserved_gb": torch.cuda.max_memory_reserved() / 1e9,
               "window": None, "lm_copies": {k: v / args.steps for k, v in lmc.items()}}
        if stats0:
            out["window"] = {k: (stats1[k] - stats0[k]) / args.steps for k in stats1}
        log(f"{mode}: {args.steps} steps in {dt:.3f}s -> {dt / args.steps * 1e3:.1f} ms/step "
            f"(median {statistics.median(step_ms):.1f}); losses {[round(x, 4) for x in out['losses']]}")
        st.close()
        del st
        torch.cuda.empty_cache()
        return out

    def spread(step_ms):
        return {"median_ms": round(statistics.median(step_ms), 2),
                "std_ms": round(statistics.stdev(step_ms), 2) if len(step_ms) > 1 else 0.0,
                "min_ms": round(min(step_ms), 2), "max_ms": round(max(step_ms), 2)}

    # The streamed step carries the per-launch event timing the roofline needs, on the
    # GEMM launches only.  The other legs are timed without it: in the resident step the
    # extra host work per launch would make the step host-bound.
    streamed = run("streamed", not args.no_kernel_timing, wblocks, slots, ckpt)
    literal = (run("streamed", False, 4, 2, 1)
               if args.shape == "32b" and (wblocks, slots) != (4, 2) and not args.no_literal_window else None)
    # the resident step keeps every checkpoint (it has the memory): its losses must still
    # equal the streamed step's bit for bit
    resident = run("resident", False, 4, 2, 1) if not args.no_resident else None

    ms = streamed["seconds"] / args.steps * 1e3
    value = T * args.ga * args.steps / streamed["seconds"]
    # roofline: the kernel with the most time in the timed region (a dense dequant-MFMA
    # GEMM at this shape), against the MFMA bf16 peak
    shapes = gemm_shapes(streamed["kernels"], args.steps)
    hbm = hbm_kernels(streamed["kernels_all"], 2)
    kt = by_kernel(streamed["kernels"])
    roofline = None
    if kt:
        name = max(kt, key=lambda k: kt[k]["total_ms"])
        k = kt[name]
        avg_ms = k["total_ms"] / k["launches"]
        avg_flops = k["total_flops"] / k["launches"]
        achieved = avg_flops / (avg_ms * 1e-3) / 1e12
        roofline = {"bound": "mfma" if avg_flops > 0 else "hbm", "kernel": name, "achieved": round(achieved, 1),
                    "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                    "traffic": measured_traffic(name) if args.shape == "32b" else None,
                    "avg_launch_ms": round(avg_ms, 4),
                    "algorithmic_gflop_per_launch": round(avg_flops / 1e9, 3)}
    kernels = {n: {"launches": v["launches"], "avg_ms": v["total_ms"] / v["launches"],
                   "tflops": v["total_flops"] / (v["total_ms"] * 1e-3) / 1e12,
                   "algorithmic_MB_per_launch": v["total_bytes"] / v["launches"] / 1e6,
                   "ms_per_step": v["total_ms"] / args.steps} for n, v in kt.items() if v["total_flops"] > 0}
    lm_bytes = streamed["lm_copies"]["bytes"]
    h2d_bytes = (streamed["window"]["bytes_copied"] if streamed["window"] else 0) + lm_bytes
    h2d_rate = h2d_bytes / (ms * 1e-3) / 1e9
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": (round(value / (T / PAGES_A100_S_PER_STEP), 3)
                        if args.shape == "32b" and layers == 64 and args.ga == 1 and args.base == "nf4" else None),
        "dtype": "bf16",
        "data": "synthetic (random N(0,0.02) NF4 base, random adapters, random tokens)",
        "config": {"workload": (f"Qwen2.5-{size}-shaped streamed NF4+LoRA train step, windows of "
                                f"{wblocks} layers x {slots} slots"
                                + (f", checkpoints every {ckpt} layers" if ckpt > 1 else "")
                                + (f", boundaries below the top {args.device_bounds} layers parked in host memory"
                                   if offload else "")),
                   "layers": layers, "hidden": hid, "heads": heads, "kv_heads": kvh, "intermediate": inter,
                   "vocab": 152064, "seq_len": T, "batch": 1, "micro_batches": args.ga,
                   **({"accumulation_order": args.order} if args.ga > 1 else {}),
                   "window_layers_per_slot": wblocks, "window_slots": slots,
                   "window_layers_resident": wblocks * slots, "checkpoint_every": ckpt,
                   "boundaries_on_device": args.device_bounds if offload else layers,
                   "copy_streams": args.copy_streams,
                   "lora_r": 16, "lora_alpha": 32, "dropout": p_drop, "optimizer": "AdamW",
                   "adapter_grads": "kept to the step's end" if args.keep_grads else "dropped after each layer's update",
                   "base": args.base,
                   "glue": args.glue, "parallelism": "single GPU"},
        "step_time": spread(streamed["step_ms"]),
        "roofline": roofline,
        "h2d": {"bytes_per_step": int(h2d_bytes), "achieved_GBps": round(h2d_rate, 1),
                "ceiling_GBps": round(ceiling, 1), "ceiling_under_compute_GBps": round(ceiling_busy, 1),
                "frac": round(h2d_rate / ceiling, 3),
                "windows_copied_per_step": streamed["window"]["windows_copied"] if streamed["window"] else 0,
                "windows_reused_per_step": streamed["window"]["windows_reused"] if streamed["window"] else 0,
                "lm_head_bytes_per_step": int(lm_bytes),
                **h2d_busy(streamed["window"], streamed["lm_copies"], ms, ceiling)},
        "kernels": kernels,
        "gemm_shapes": shapes,
        "hbm_kernels": hbm,
        "peak_vram_gb": round(streamed["peak_alloc_gb"], 2),
        "peak_vram_reserved_gb": round(streamed["peak_reserved_gb"], 2),
        "baseline_context": {"value": round(T / PAGES_A100_S_PER_STEP, 1), "unit": "tokens/s",
                             "hardware": "NVIDIA A100 80GB PCIe", "s_per_step": PAGES_A100_S_PER_STEP},
    }
    if literal:
        lms = literal["seconds"] / args.steps * 1e3
        lw = literal["window"]
        result["window_2_slots"] = {"ms_per_step": round(lms, 2), **spread(literal["step_ms"]),
                                    "tokens_per_s": round(T * args.ga * args.steps / literal["seconds"], 2),
                                    "h2d_bytes_per_step": int(lw["bytes_copied"] + literal["lm_copies"]["bytes"]),
                                    "peak_vram_gb": round(literal["peak_alloc_gb"], 2),
                                    "losses_equal": literal["losses"] == streamed["losses"]}
    if resident:
        rms = resident["seconds"] / args.steps * 1e3
        result["resident"] = {"ms_per_step": round(rms, 2), **spread(resident["step_ms"]),
                              "tokens_per_s": round(T * args.ga * args.steps / resident["seconds"], 2),
                              "peak_vram_gb": round(resident["peak_alloc_gb"], 2),
                              "streamed_over_resident": round(ms / rms, 3),
                              "losses_equal": resident["losses"] == streamed["losses"]}
    if not args.no_cpu_baseline and args.shape == "32b":
        result["cpu_baseline"] = cpu_baseline()
    result["host"] = {"cpu": platform.processor() or platform.machine(), "nproc": os.cpu_count()}
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
