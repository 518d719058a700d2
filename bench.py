"""Throughput of exact attention, forward and forward+backward, on one MI355X.

A step is one pass of the whole hot path over one batch: fa_forward, then
fa_backward_prep and fa_backward_grads, on the causal workload B=4, H=16,
N=4096, d=128 (bf16 inputs drawn i.i.d. N(0,1) from seed 5, already resident
in HBM). The timed region is exactly --steps steps, bracketed by device
synchronisation and two HIP events on the launch stream.

Throughput counts matmul FLOPs only: forward 4*B*H*N^2*d, backward 2.5x that
(score recompute, dV, dP, dQ, dK), both halved under the causal mask.

Prints one JSON line. `value` is forward+backward TFLOP/s over the timed
steps, which hold nothing but the steps' launches; `fwd_tflops` the forward
alone on the same input. The duration of each launch kind (`ms`, and the
roofline's `avg_launch_ms`) is the mean of --steps launches of that kind
alone, back to back between two HIP events on the launch stream, right after
the timed steps: an event around every single launch would add the event's
own latency (about 10-15 us) to every launch. `roofline` describes the dominant kernel
(the one with the longest launches), `cpu_baseline` the fp64 CPU oracle
timed on a bounded sample of the same workload on this host.

A second object, `gqa`, times the same step on the grouped-query workload
B=4, H=32 query heads sharing H_kv=8 K/V heads, N=4096, d=128, causal (seed
6), through fa_forward_gqa, fa_backward_prep and fa_backward_grads_gqa; its
FLOP count is that of 32 heads. A third, `window`, times it on the local
workload B=4, H=16, N=4096, d=128 with a causal window of 1024 keys (seed
7) through the _window calls; its FLOP count is 4*d per visible (query,
key) pair, counted exactly.

A fourth, `fp8`, times the FP8 forward with incoherent processing
(fa_fp8_prepare, then fa_forward_fp8_prepared) on the causal forward
workload B=4, H=32, N=4096, d=128 (seed 3, signs drawn from seed 3) next to
the bf16 forward on the same input; its FLOP count is the forward's, and its
roofline peak the dense fp8 MFMA rate.

A fifth, `d256`, times the forward+backward step at head dimension 256:
B=4, H=8, N=4096, d=256, causal (seed 8), through the _gqa calls with
H_kv = H.

A sixth, `block_sparse`, times it on the causal workload B=4, H=16,
N=4096, d=128 (seed 9) with a block-sparse mask per query head (each
128 x 128 block below the diagonal kept with probability 1/2, the diagonal
blocks always) through the _block_sparse calls; its FLOP count is 4*d per
visible (query, key) pair, counted exactly from the mask.

A seventh, `fwd_configs`, times the forward alone (fa_forward) on the three
forward workloads: B=8, H=16, N=2048, d=64, no mask (seed 2); B=4, H=32,
N=4096, d=128, causal (seed 3); B=1, H=16, N=32768, d=128, causal (seed 4),
each with its own roofline.

Besides the back-to-back timing (the mean of --steps launches between two
HIP events, after --warmup untimed ones), every launch kind is also
timed --flush-iters times with the L2 and the 256 MB MALL flushed before
each launch (a 512 MiB write, not timed), reported as median and minimum
(`flushed`): the launches then read their inputs from HBM, as the first
kernel touching a tensor does.

Usage: python bench.py [--gpus 1] [--steps 50] [--warmup 100] [--no-cpu-baseline]
                       [--copy-calibration] [--no-gqa] [--gqa-only] [--no-window]
                       [--window-only] [--no-fp8] [--fp8-only] [--no-d256] [--d256-only]
                       [--no-block-sparse] [--block-sparse-only] [--no-fwd-configs]
                       [--fwd-configs-only] [--flush-iters 20]
The default warm-up (100 steps, about 0.13 s on the main workload) brings
the GPU to its steady clock first: with 5 warm-up steps the same 50 timed
steps read about 2% lower, and longer warm-ups (500, 2000) no higher.

--copy-calibration first runs a plain device copy of 1 GiB (torch's copy
kernel), whose FETCH_SIZE / WRITE_SIZE counters calibrate the HBM traffic
counters of the attention kernels in the same profiled run.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# MI355X dense bf16 MFMA peak: 256 CUs x 4 SIMDs x 1024 flop/clk x 2.4 GHz.
PEAK_BF16_TFLOPS = 2516.6
# dense fp8 MFMA peak: twice the bf16 rate.
PEAK_FP8_TFLOPS = 5033.2
FP8_WORKLOAD = "fwd_causal_b4h32n4096d128"
D256_WORKLOAD = "fwdbwd_causal_b4h8n4096d256"
WORKLOAD = "fwdbwd_causal_b4h16n4096d128"
GQA_WORKLOAD = "fwdbwd_causal_gqa_b4h32kv8n4096d128"
WINDOW_WORKLOAD = "fwdbwd_window1024_b4h16n4096d128"
BLOCK_SPARSE_WORKLOAD = "fwdbwd_causal_blocksparse50_b4h16n4096d128"
FWD_WORKLOADS = ["fwd_b8h16n2048d64", "fwd_causal_b4h32n4096d128", "fwd_causal_b1h16n32768d128"]
METRIC = "attention TFLOP/s (fwd, fwd+bwd) bf16 on 1 MI355X; % of MFMA peak"
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "hbm_traffic.json")
KERNEL_SOURCES = ["exact_io_aware_14_amd/csrc/fa_common.h", "exact_io_aware_14_amd/csrc/fa_fwd_kernel.h",
                  "exact_io_aware_14_amd/csrc/fa_fwd.hip", "exact_io_aware_14_amd/csrc/fa_fwd_w.hip",
                  "exact_io_aware_14_amd/csrc/fa_bwd_common.h", "exact_io_aware_14_amd/csrc/fa_bwd.hip",
                  "exact_io_aware_14_amd/csrc/fa_bwd_w.hip", "exact_io_aware_14_amd/csrc/fa_fp8.hip",
                  "exact_io_aware_14_amd/build.py"]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def visible_pairs(n, left, right):
    """(query, key) pairs of one head with i-left <= j <= i+right (-1: unbounded)."""
    total = 0
    for i in range(n):
        lo = 0 if left < 0 else max(0, i - left)
        hi = n - 1 if right < 0 else min(n - 1, i + right)
        total += hi - lo + 1
    return total


def block_sparse_pairs(w):
    """Visible (query, key) pairs of all heads of a block-sparse workload:
    per nonzero block of each head's mask, its pairs under the causal mask
    (all of them without it)."""
    import numpy as np

    from exact_io_aware_14_amd.inputs import MASK_BLOCK, workload_block_mask

    nb = (w.N + MASK_BLOCK - 1) // MASK_BLOCK
    i = np.arange(w.N)
    seen = (i[None, :] <= i[:, None]) if w.causal else np.ones((w.N, w.N), dtype=bool)
    blk = i // MASK_BLOCK
    per_block = np.zeros((nb, nb), dtype=np.int64)
    np.add.at(per_block, (blk[:, None].repeat(w.N, 1)[seen], blk[None, :].repeat(w.N, 0)[seen]),
              1)
    mask = workload_block_mask(w).numpy() != 0
    return int((mask * per_block).sum())


def counted_flops(w):
    if w.block_density > 0:
        fwd = 4.0 * w.d * block_sparse_pairs(w)
    elif w.window_left >= 0 or w.window_right >= 0:
        fwd = 4.0 * w.B * w.H * w.d * visible_pairs(w.N, w.window_left, w.window_right)
    else:
        fwd = 4.0 * w.B * w.H * w.N * w.N * w.d * (0.5 if w.causal else 1.0)
    return fwd, 2.5 * fwd


def fwd_kernel_name(w):
    """The forward kernel fa_forward launches on workload w, as the profiles
    name it: causal launches at d = 128 with at most 64 query blocks per head
    take two query blocks per workgroup (`pair`)."""
    if not w.causal:
        return f"fwd_kernel<{w.d},nomask>"
    pair = w.d == 128 and (w.N + 127) // 128 <= 64
    return f"fwd_kernel<{w.d},causal{',pair' if pair else ''}>"


def measured_traffic(kernel: str, src_hash: str, workload: str = WORKLOAD):
    """HBM bytes per launch of `kernel` on `workload` from the committed
    counter runs, if they were taken on the kernel sources as they are now;
    else None."""
    try:
        data = json.load(open(PROFILE_TRAFFIC))
    except (OSError, ValueError):
        return None
    if data.get("source_hash") != src_hash:
        return None
    entry = data.get("workloads", {}).get(workload, {}).get("kernels", {}).get(kernel)
    return None if entry is None else entry.get("bytes_per_launch")


def cpu_baseline(w, heads: int):
    """The fp64 oracle on `heads` whole heads of the workload (forward and
    backward), as TFLOP/s on the same counted-FLOP basis."""
    import numpy as np  # noqa: F401

    import oracle
    from exact_io_aware_14_amd.inputs import draw, to_f64

    q, k, v, do = draw(w.shape, w.seed, with_grad=True)
    try:
        from threadpoolctl import threadpool_info
        cores = max((i.get("num_threads") or 1) for i in threadpool_info()) if threadpool_info() else 1
    except Exception:  # threadpoolctl missing: numpy's BLAS default
        cores = os.cpu_count() or 1
    t0 = time.perf_counter()
    for i in range(heads):
        b, h = divmod(i, w.H)
        qf, kf, vf, gf = (to_f64(x[b, h]) for x in (q, k, v, do))
        oracle.forward_head(qf, kf, vf, w.scale, w.causal)
        oracle.backward_head(qf, kf, vf, gf, w.scale, w.causal)
    dt = time.perf_counter() - t0
    fwd, bwd = counted_flops(w)
    per_head = (fwd + bwd) / (w.B * w.H)
    return {"value": round(per_head * heads / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(cores),
            "kind": "oracle",
            "sample": f"{heads} of {w.B * w.H} heads of {WORKLOAD}, full forward and backward "
                      f"in fp64 numpy, {dt:.1f} s; the rate extrapolates linearly to all heads"}


def time_launches(launches, reps, stream):
    """Average ms of each callable in `launches`, each launched `reps` times
    back to back between two HIP events on `stream` (after one untimed
    launch). The launches are idempotent: they read inputs the step leaves in
    place and rewrite the same outputs."""
    import torch
    out = []
    for fn in launches:
        fn()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1) / reps)
    return out


def time_steps(step, launches, steps, warmup, stream):
    """`warmup` untimed steps, then `steps` steps between two HIP events (no
    event inside, so nothing but the step's own launches is timed): the mean
    ms per step. Then each launch kind of the step alone, back to back
    (time_launches): its mean ms per launch."""
    import torch
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    return time_launches(launches, steps, stream), e0.elapsed_time(e1) / steps


def measure_variant(name, steps, warmup):
    """The forward+backward step on a grouped-query or local-window workload,
    through the calls that take those arguments."""
    import torch

    import exact_io_aware_14_amd as fa
    from exact_io_aware_14_amd.inputs import by_name, draw, workload_block_mask

    w = by_name(name)
    dev = torch.device("cuda:0")
    q, k, v, do = (x.to(dev) for x in draw(w.shape, w.seed, with_grad=True, kv_heads=w.kv_heads))
    sparse = w.block_density > 0
    bm = workload_block_mask(w).to(dev) if sparse else None
    o = torch.empty_like(q)
    lse = torch.empty(w.shape[:3], dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(fa.fa_backward_workspace_size(*w.shape), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    window = w.window_left >= 0 or w.window_right >= 0
    win = (w.window_left, w.window_right)
    causal_win = (-1, 0) if w.causal else (-1, -1)

    def fwd():
        if sparse:
            fa.fa_forward_block_sparse(q, k, v, bm, *causal_win, w.scale, o, lse, stream=stream)
        elif window:
            fa.fa_forward_window(q, k, v, *win, w.scale, o, lse, stream=stream)
        else:
            fa.fa_forward_gqa(q, k, v, w.scale, w.causal, o, lse, stream=stream)

    def prep():
        fa.fa_backward_prep(o, do, lse, ws, stream=stream)

    def grads():
        if sparse:
            fa.fa_backward_grads_block_sparse(q, k, v, do, lse, ws, bm, *causal_win, w.scale, dq,
                                              dk, dv, stream=stream)
        elif window:
            fa.fa_backward_grads_window(q, k, v, do, lse, ws, *win, w.scale, dq, dk, dv,
                                        stream=stream)
        else:
            fa.fa_backward_grads_gqa(q, k, v, do, lse, ws, w.scale, w.causal, dq, dk, dv,
                                     stream=stream)

    def step():
        fwd()
        prep()
        grads()

    (fwd_ms, prep_ms, grads_ms), step_ms = time_steps(step, [fwd, prep, grads], steps, warmup,
                                                      stream)
    fwd_f, bwd_f = counted_flops(w)
    out = {"workload": w.name, "B": w.B, "H": w.H, "H_kv": w.kv_heads, "N": w.N, "d": w.d}
    if window:
        out["window"] = [w.window_left, w.window_right]
    else:
        out["causal"] = w.causal
    if sparse:
        out["block_density"] = w.block_density
        out["mask_blocks_kept"] = round(float(bm.float().mean()), 4)
    out.update({"steps": steps,
                "fwdbwd_tflops": round((fwd_f + bwd_f) / (step_ms * 1e-3) / 1e12, 2),
                "fwd_tflops": round(fwd_f / (fwd_ms * 1e-3) / 1e12, 2),
                "bwd_tflops": round(bwd_f / ((prep_ms + grads_ms) * 1e-3) / 1e12, 2),
                "ms": {"fwd": round(fwd_ms, 4), "bwd_prep": round(prep_ms, 4),
                       "bwd_grads": round(grads_ms, 4)}})
    return out


def measure_fp8(steps, warmup):
    """The FP8 forward (prepare + attention) and the bf16 forward on the same
    causal input; each launch kind timed back to back between HIP events."""
    import torch

    import exact_io_aware_14_amd as fa
    from exact_io_aware_14_amd.inputs import by_name, draw, draw_signs

    w = by_name(FP8_WORKLOAD)
    dev = torch.device("cuda:0")
    q, k, v = (x.to(dev) for x in draw(w.shape, w.seed))
    signs = draw_signs(w.d, w.seed)
    shape = (w.B, w.H, w.H, w.N, w.d)
    ws = torch.empty(fa.fa_forward_fp8_workspace_size(*shape), dtype=torch.uint8, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty(w.shape[:3], dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def prepare():
        fa.fa_fp8_prepare(q, k, v, signs, ws, stream=stream)

    def attention():
        fa.fa_forward_fp8_prepared(ws, shape, w.scale, w.causal, o, lse, stream=stream)

    def bf16():
        fa.fa_forward(q, k, v, w.scale, w.causal, o, lse, stream=stream)

    def step():
        prepare()
        attention()
        bf16()

    (prep_ms, attn_ms, bf16_ms), _ = time_steps(step, [prepare, attention, bf16], steps, warmup,
                                                stream)
    fwd_f, _ = counted_flops(w)
    attn = fwd_f / (attn_ms * 1e-3) / 1e12
    return {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "causal": w.causal,
            "steps": steps,
            "fwd_tflops": round(fwd_f / ((prep_ms + attn_ms) * 1e-3) / 1e12, 2),
            "attention_tflops": round(attn, 2),
            "bf16_fwd_tflops": round(fwd_f / (bf16_ms * 1e-3) / 1e12, 2),
            "speedup_vs_bf16": round(bf16_ms / (prep_ms + attn_ms), 3),
            "ms": {"prepare": round(prep_ms, 4), "attention": round(attn_ms, 4),
                   "bf16_fwd": round(bf16_ms, 4)},
            "roofline": {"bound": "mfma", "kernel": "fwd_fp8_kernel<128,causal>",
                         "achieved": round(attn, 2), "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(attn / PEAK_FP8_TFLOPS, 4),
                         "traffic": measured_traffic("fwd_fp8_kernel<128,causal>",
                                                     kernel_source_hash(), FP8_WORKLOAD),
                         "avg_launch_ms": round(attn_ms, 4)}}


_FLUSH = None


def flush_caches():
    """Write 512 MiB (twice the 256 MB MALL, far above the L2s) so that the
    next launch finds none of its inputs in any cache."""
    import torch
    global _FLUSH
    if _FLUSH is None:
        _FLUSH = torch.empty(1 << 27, dtype=torch.float32, device="cuda")
    _FLUSH.zero_()


def time_flushed(launches, iters, stream):
    """Each callable in `launches` timed `iters` times with HIP events around
    it, the caches flushed before each launch: {index: (median_ms, min_ms)}.
    The launches run in order within an iteration, so each one reads what
    the previous one wrote."""
    import statistics

    import torch
    times = [[] for _ in launches]
    for _ in range(iters):
        for j, fn in enumerate(launches):
            flush_caches()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            times[j].append(e0.elapsed_time(e1))
    return [(statistics.median(t), min(t)) for t in times]


def measure_forward(name, steps, warmup, flush_iters):
    """fa_forward alone on a forward workload: the mean of `steps`
    back-to-back launches (between two HIP events) and the flushed median."""
    import torch

    import exact_io_aware_14_amd as fa
    from exact_io_aware_14_amd.inputs import by_name, draw

    w = by_name(name)
    dev = torch.device("cuda:0")
    q, k, v = (x.to(dev) for x in draw(w.shape, w.seed))
    o = torch.empty_like(q)
    lse = torch.empty(w.shape[:3], dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def launch():
        fa.fa_forward(q, k, v, w.scale, w.causal, o, lse, stream=stream)

    for _ in range(warmup):
        launch()
    torch.cuda.synchronize()
    ms, = time_launches([launch], steps, stream)
    (fl_med, fl_min), = time_flushed([launch], flush_iters, stream) if flush_iters else [(None, None)]
    fwd_f, _ = counted_flops(w)
    tflops = fwd_f / (ms * 1e-3) / 1e12
    kname = fwd_kernel_name(w)
    out = {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "causal": w.causal,
           "steps": steps, "ms": round(ms, 4), "fwd_tflops": round(tflops, 2),
           "fwd_frac_of_peak": round(tflops / PEAK_BF16_TFLOPS, 4)}
    if fl_med is not None:
        out["flushed"] = {"iters": flush_iters, "median_ms": round(fl_med, 4),
                          "min_ms": round(fl_min, 4),
                          "fwd_tflops_median": round(fwd_f / (fl_med * 1e-3) / 1e12, 2)}
    out["roofline"] = {"bound": "mfma", "kernel": kname, "achieved": round(tflops, 2),
                       "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                       "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                       "traffic": measured_traffic(kname, kernel_source_hash(), w.name),
                       "avg_launch_ms": round(ms, 4)}
    return out


def copy_calibration():
    """A plain device copy of 1 GiB (read 1 GiB, write 1 GiB), run once."""
    import torch
    src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=40)
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--no-gqa", action="store_true")
    ap.add_argument("--gqa-only", action="store_true",
                    help="time only the grouped-query step (for its profile)")
    ap.add_argument("--no-window", action="store_true")
    ap.add_argument("--window-only", action="store_true",
                    help="time only the local-window step (for its profile)")
    ap.add_argument("--no-d256", action="store_true")
    ap.add_argument("--d256-only", action="store_true",
                    help="time only the head-dimension-256 step (for its profile)")
    ap.add_argument("--no-block-sparse", action="store_true")
    ap.add_argument("--block-sparse-only", action="store_true",
                    help="time only the block-sparse step (for its profile)")
    ap.add_argument("--no-fwd-configs", action="store_true")
    ap.add_argument("--fwd-configs-only", action="store_true",
                    help="time only the forward workloads (for their profiles)")
    ap.add_argument("--flush-iters", type=int, default=20,
                    help="flushed-cache timings per launch kind (0: none)")
    ap.add_argument("--no-fp8", action="store_true")
    ap.add_argument("--fp8-only", action="store_true",
                    help="time only the FP8 forward (for its profile)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        sys.exit("bench.py measures one GPU only: there is no multi-GPU path here "
                 "(attention heads would shard across GPUs with no exchange)")
    if args.copy_calibration:
        copy_calibration()
    if args.gqa_only:
        print(json.dumps({"gqa": measure_variant(GQA_WORKLOAD, args.steps, args.warmup)}),
              flush=True)
        return
    if args.d256_only:
        print(json.dumps({"d256": measure_variant(D256_WORKLOAD, args.steps, args.warmup)}),
              flush=True)
        return
    if args.fwd_configs_only:
        print(json.dumps({"fwd_configs": {n: measure_forward(n, args.steps, args.warmup,
                                                             args.flush_iters)
                                          for n in FWD_WORKLOADS}}), flush=True)
        return
    if args.fp8_only:
        print(json.dumps({"fp8": measure_fp8(args.steps, args.warmup)}), flush=True)
        return
    if args.window_only:
        print(json.dumps({"window": measure_variant(WINDOW_WORKLOAD, args.steps, args.warmup)}),
              flush=True)
        return
    if args.block_sparse_only:
        print(json.dumps({"block_sparse": measure_variant(BLOCK_SPARSE_WORKLOAD, args.steps,
                                                          args.warmup)}), flush=True)
        return

    import torch

    from exact_io_aware_14_amd import (fa_backward_grads, fa_backward_prep,
                                       fa_backward_workspace_size, fa_forward)
    from exact_io_aware_14_amd.inputs import by_name, draw

    w = by_name(WORKLOAD)
    dev = torch.device("cuda:0")
    q, k, v, do = (x.to(dev) for x in draw(w.shape, w.seed, with_grad=True))
    o = torch.empty_like(q)
    lse = torch.empty(w.shape[:3], dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(fa_backward_workspace_size(*w.shape), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def fwd():
        fa_forward(q, k, v, w.scale, w.causal, o, lse, stream=stream)

    def prep():
        fa_backward_prep(o, do, lse, ws, stream=stream)

    def grads():
        fa_backward_grads(q, k, v, do, lse, ws, w.scale, w.causal, dq, dk, dv, stream=stream)

    def step():
        fwd()
        prep()
        grads()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # the timed region: exactly --steps steps, nothing else inside
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for _ in range(args.steps):
        step()
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0

    total_ms = t_start.elapsed_time(t_end)
    ms_step = total_ms / args.steps
    # each launch kind alone, --steps launches back to back (time_launches)
    fwd_ms, prep_ms, grads_ms = time_launches([fwd, prep, grads], args.steps, stream)
    fwd_f, bwd_f = counted_flops(w)
    value = (fwd_f + bwd_f) / (ms_step * 1e-3) / 1e12
    fwd_tflops = fwd_f / (fwd_ms * 1e-3) / 1e12
    bwd_tflops = bwd_f / ((prep_ms + grads_ms) * 1e-3) / 1e12

    flushed = None
    if args.flush_iters:
        parts = time_flushed(
            [lambda: fa_forward(q, k, v, w.scale, w.causal, o, lse, stream=stream),
             lambda: fa_backward_prep(o, do, lse, ws, stream=stream),
             lambda: fa_backward_grads(q, k, v, do, lse, ws, w.scale, w.causal, dq, dk, dv,
                                       stream=stream)], args.flush_iters, stream)
        (f_med, f_min), (p_med, p_min), (g_med, g_min) = parts
        flushed = {"iters": args.flush_iters,
                   "median_ms": {"fwd": round(f_med, 4), "bwd_prep": round(p_med, 4),
                                 "bwd_grads": round(g_med, 4)},
                   "min_ms": {"fwd": round(f_min, 4), "bwd_prep": round(p_min, 4),
                              "bwd_grads": round(g_min, 4)},
                   "fwdbwd_tflops_median": round((fwd_f + bwd_f) /
                                                 ((f_med + p_med + g_med) * 1e-3) / 1e12, 2),
                   "fwd_tflops_median": round(fwd_f / (f_med * 1e-3) / 1e12, 2)}

    src_hash = kernel_source_hash()
    if grads_ms >= fwd_ms:
        kname, kflops, kms = "bwd_grads_kernel<128,causal>", bwd_f, grads_ms
    else:
        kname, kflops, kms = fwd_kernel_name(w), fwd_f, fwd_ms
    achieved = kflops / (kms * 1e-3) / 1e12
    roofline = {"bound": "mfma", "kernel": kname, "achieved": round(achieved, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": measured_traffic(kname, src_hash),
                "avg_launch_ms": round(kms, 4)}

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": WORKLOAD, "B": w.B, "H": w.H, "N": w.N, "d": w.d,
                   "causal": w.causal, "seed": w.seed, "scale": w.scale},
        "frac_of_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "fwd_tflops": round(fwd_tflops, 2),
        "fwd_frac_of_peak": round(fwd_tflops / PEAK_BF16_TFLOPS, 4),
        "bwd_tflops": round(bwd_tflops, 2),
        "ms": {"fwd": round(fwd_ms, 4), "bwd_prep": round(prep_ms, 4),
               "bwd_grads": round(grads_ms, 4)},
        "wall_s_timed": round(wall, 3),
        "kernel_source_hash": src_hash,
        "roofline": roofline,
    }
    if flushed is not None:
        out["flushed"] = flushed
    if not args.no_gqa:
        out["gqa"] = measure_variant(GQA_WORKLOAD, args.steps, args.warmup)
    if not args.no_window:
        out["window"] = measure_variant(WINDOW_WORKLOAD, args.steps, args.warmup)
    if not args.no_d256:
        out["d256"] = measure_variant(D256_WORKLOAD, args.steps, args.warmup)
    if not args.no_block_sparse:
        out["block_sparse"] = measure_variant(BLOCK_SPARSE_WORKLOAD, args.steps, args.warmup)
    if not args.no_fp8:
        out["fp8"] = measure_fp8(args.steps, args.warmup)
    if not args.no_fwd_configs:
        out["fwd_configs"] = {n: measure_forward(n, args.steps, args.warmup, args.flush_iters)
                              for n in FWD_WORKLOADS}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_heads)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
