"""Throughput of the spatial self-attention block on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config I] [--no-cpu]
                    [--eager] [--options relpos,qknorm,rope]

A step is one ssa_forward over one batch of the selected workload (GroupNorm
statistics, QKV projection, flash attention, output projection + residual;
where the library fuses them, projection and attention are one kernel), with
inputs already resident in HBM.  The default workload is the high-resolution
one (B2 C640 96x96 G32 n10), the largest of the five.  W untimed steps (and
more untimed steps for --settle seconds, so the GPU's clocks have ramped up),
then exactly K steps between two device synchronisations; the value is block
TFLOP/s (8BTC^2 + 4BT^2C flops per step).  The K steps are captured once into
a HIP graph and replayed (every kernel of every step runs; only the host
launch gaps between them go), as a deployment would run the block; the rate
of K eager ssa_forward calls is reported beside it (`other_launch`), and
--eager makes that one the value.  Prints one JSON line.

Also reported:
* the distribution of single-step times (median, min, max) over separately
  timed eager steps, each between two events on the launch stream;
* per-kernel average durations from HIP events on the launch stream, each
  stage the step runs replayed back-to-back from a HIP graph so host launch
  overhead is not counted; the dominant kernel's roofline (algorithmic flops
  per launch over its average duration, against MI355X's dense bf16 MFMA
  peak), with HBM traffic from the stored rocprofv3 counter summary when it
  was taken on the current kernel sources;
* GroupNorm-statistics GB/s, warm (back-to-back launches) and cold (a 512 MiB
  buffer written before each launch, which evicts x from the caches);
* the fp64 CPU oracle's rate on a bounded sample of the same workload.

With --options the step is ssa_forward_ex with the listed optional steps
(2-D relative-position logit bias, per-head query/key normalisation, rotary
embeddings; tensors drawn as in the tests), and the per-kernel times come from
ssa_forward_stage_ex with the same options.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # 256 CU x 4096 flop/clk x 2.4 GHz, dense
PEAK_FP32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
DEFAULT_CONFIG = 4          # high-res: B2 C640 96x96 G32 n10 (d=64), bf16: the largest workload


# The sources each stage's kernels are built from (its .hip file and the
# headers it includes): stored counters stay valid while these are unchanged.
STAGE_SOURCES = {
    "gn_stats": ("gn_stats.hip", "ssa_internal.h"),
    "qkv": ("projections.hip", "qk_post.hip", "ssa_internal.h"),
    "attention": ("attention.hip", "attn_core.h", "ssa_internal.h"),
    "qkv_attention": ("fused.hip", "attn_core.h", "ssa_internal.h"),
    "out_proj": ("projections.hip", "ssa_internal.h"),
}


def source_digest(stage: str = None) -> str:
    """Hash of the kernel sources (all, or those of one stage's kernels), to
    tell whether stored counters still apply."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "spatial_self_attention_amd", "csrc")
    files = sorted(os.listdir(csrc)) if stage is None else sorted(STAGE_SOURCES[stage])
    for f in files:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode())
            h.update(fh.read())
    return h.hexdigest()[:16]


def stage_work(wl):
    """Algorithmic work per launch of each stage: (kind, amount)."""
    B, C, T = wl.B, wl.C, wl.T
    es = 4 if wl.dtype == "f32" else 2
    return {
        "gn_stats": ("bytes", B * C * T * es),
        "qkv": ("flops", 6 * B * T * C * C),
        "attention": ("flops", 4 * B * T * T * C),
        "qkv_attention": ("flops", 6 * B * T * C * C + 4 * B * T * T * C),
        "out_proj": ("flops", 2 * B * T * C * C),
    }


# Kernel names (as rocprofv3 prints them) behind each stage, for the counters.
STAGE_KERNELS = {
    "gn_stats": "gn_stats_wave_kernel / gn_stats_kernel / gn_seg_kernel (+ gn_finalize_kernel "
                "when segments are split)",
    "qkv": "gemm_bf16_kernel<0, *>",
    "attention": "attn_bf16_kernel / attn2_bf16_kernel / attnpp_bf16_kernel (+ attn_merge_kernel "
                 "when the tiles of a partial last round are cut into key ranges)",
    "qkv_attention": "fused_bf16_kernel",
    "out_proj": "gemm_bf16_kernel<1, 0>",
}


def stored_traffic(stage: str, wl_name: str, options=()):
    """HBM bytes per launch from the committed counter summary, or None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        data = json.load(open(path))
    except ValueError:
        return None
    key = f"{wl_name}|{stage}" + (f"|{'+'.join(options)}" if options else "")
    ent = data.get("entries", {}).get(key)
    if ent is None or ent.get("source_digest") != source_digest(stage):
        return None
    return ent.get("bytes_per_launch")


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return int(max([i.get("num_threads", 1) for i in threadpool_info()] or [1]))
    except Exception:
        return os.cpu_count() or 1


def cpu_baseline(wl, seed, opts=None, budget_s=12.0):
    """The fp64 oracle as it is, on a bounded sample of the workload: chunks of
    consecutive query rows of one sample at a time (oracle.forward_pixels:
    GroupNorm statistics and K, V of the whole sample, Q, the scores, the
    softmax, P V and the output projection for the chunk's rows), walking the
    samples' rows in order while the time budget lasts.  A whole high-res
    sample at once would hold 6.8 GB of fp64 probabilities.  The rate counts
    the block's algorithmic flops per output pixel times the pixels produced."""
    import numpy as np

    from oracle import forward_pixels
    from spatial_self_attention_amd.inputs import draw, options_f64, to_f64
    # at most 2^21 scores per head and call (the oracle holds them all in fp64)
    R = min(wl.T, max(64, (1 << 21) // wl.T))
    one = wl.replace(B=1)
    per_pixel = one.flops() / wl.T
    kw = options_f64(opts) if opts is not None else {}
    done_rows, el, calls = 0, 0.0, 0
    b, r0 = 0, 0
    x, p = draw(wl, seed)  # the same inputs as the GPU's batch
    cache = {}
    while el < budget_s:
        if b not in cache:  # one sample upcast at a time
            cache.clear()
            cache[b] = to_f64(x[b:b + 1], p)
        x64, p64 = cache[b]
        rows = np.arange(r0, min(r0 + R, wl.T))
        t1 = time.perf_counter()
        forward_pixels(x64, p64, wl.num_groups, wl.num_heads, 0, rows, **kw)
        el += time.perf_counter() - t1
        done_rows += len(rows)
        calls += 1
        r0 += R
        if r0 >= wl.T:
            r0, b = 0, (b + 1) % wl.B
    return {"value": round(done_rows * per_pixel / el / 1e12, 5), "unit": "TFLOP/s",
            "cores": blas_threads(), "kind": "oracle",
            "sample": f"{calls} oracle.forward_pixels calls of up to {R} consecutive query rows "
                      f"of one sample of {wl.name} ({done_rows} output pixels, "
                      f"{done_rows / wl.T:.2f} samples' worth), fp64 NumPy, {el:.1f} s of "
                      f"oracle time; each call recomputes its sample's GroupNorm, K and V; "
                      f"the rate counts the block's flops per pixel (1/T of a sample's)",
            "pixels_per_s": round(done_rows / el, 1), "os_cpu_count": os.cpu_count()}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--settle", type=float, default=0.5, metavar="SECONDS",
                    help="untimed steps for this long after the warm-up steps (clock ramp)")
    ap.add_argument("--config", type=int, default=DEFAULT_CONFIG)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--options", default="",
                    help="comma list of optional steps to switch on: relpos, qknorm, rope")
    ap.add_argument("--eager", action="store_true",
                    help="time K eager launches of the step instead of K steps replayed from "
                         "one HIP graph (both are measured; this picks which one is `value`)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run 10 device-to-device copies of BYTES each (the reference "
                         "kernel for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE to HBM bytes)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the block runs on a single MI355X here, and "
              "--gpus N with N > 1 is not supported; run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        import torch
        src = torch.ones(args.copy_calibration // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": src.numel() * 4, "copies": 10}), flush=True)
        return

    import torch

    import spatial_self_attention_amd as ssa
    from spatial_self_attention_amd.inputs import WORKLOADS, default_seed, draw, draw_options

    wl = WORKLOADS[args.config]
    seed = default_seed(args.config)
    dev = torch.device("cuda:0")
    x, p = draw(wl, seed)
    xg = x.to(dev)
    pg = {k: v.to(dev) for k, v in p.items()}
    out = torch.empty_like(xg)
    ws = ssa.workspace_for(xg, wl.num_groups, wl.num_heads)
    stream = torch.cuda.current_stream(dev)
    names = [o for o in args.options.split(",") if o]
    unknown = set(names) - {"relpos", "qknorm", "rope"}
    if unknown:
        ap.error(f"unknown options {sorted(unknown)}")
    opts, od = None, None
    if names:
        od = draw_options(wl, seed, rel_pos="relpos" in names, qk_norm="qknorm" in names,
                          rope="rope" in names)
        odg = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in od.items()}
        opts = ssa.make_options(xg, wl.num_heads, odg["rel_pos_table"], odg["q_norm_gamma"],
                                odg["k_norm_gamma"], odg["rope"])

    def step():  # on torch's current stream (the capture stream inside a graph)
        ssa.forward_into(xg, pg, wl.num_groups, wl.num_heads, out, ws, options=opts)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # then keep stepping (untimed) for --settle seconds: a few warm-up steps of
    # a short workload end before the GPU's clocks have ramped up
    t_end = time.perf_counter() + args.settle
    while time.perf_counter() < t_end:
        for _ in range(20):
            step()
        torch.cuda.synchronize()

    def timed(graph: bool) -> float:
        """Seconds for exactly K steps between two device synchronisations."""
        if graph:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for _ in range(args.steps):
                    step()
            torch.cuda.synchronize()
            g.replay()  # untimed: the first replay uploads the graph
            torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record(stream)
        if graph:
            g.replay()
        else:
            for _ in range(args.steps):
                step()
        e1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return max(wall, e0.elapsed_time(e1) / 1e3)

    # The step as a deployment runs it: captured once into a HIP graph (all of
    # its kernels, every step), so host launch gaps do not sit between them;
    # the eager rate (one ssa_forward call per step) is reported beside it.
    el = {"graph": timed(True), "eager": timed(False)}
    launch = "eager" if args.eager else "graph"
    elapsed = el[launch]
    ms_per_step = elapsed / args.steps * 1e3
    tflops = wl.flops() * args.steps / elapsed / 1e12
    other = "graph" if launch == "eager" else "eager"
    alt = {"launch": other, "value": round(wl.flops() * args.steps / el[other] / 1e12, 3),
           "ms_per_step": round(el[other] / args.steps * 1e3, 5)}

    # ---- single-step times: events around each of N eager steps ----
    nstep = max(20, min(args.steps, 100))
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(nstep)]
    for a, b in evs:
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    st_ms = sorted(a.elapsed_time(b) for a, b in evs)
    step_ms = {"median": round(statistics.median(st_ms), 5), "min": round(st_ms[0], 5),
               "max": round(st_ms[-1], 5), "steps": nstep, "launch": "eager, events per step"}

    # ---- per-kernel durations: each stage replayed back-to-back from a graph ----
    reps = max(20, min(args.steps, 200))
    per_stage = {}
    stages = ssa.forward_stages(xg, wl.num_groups, wl.num_heads, options=opts)
    for stage in stages:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(reps):
                ssa.forward_into(xg, pg, wl.num_groups, wl.num_heads, out, ws, stage=stage,
                                 options=opts)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        g.replay()
        b.record(stream)
        torch.cuda.synchronize()
        per_stage[stage] = a.elapsed_time(b) / 1e3 / reps
        del g

    # ---- GroupNorm statistics cold: a 512 MiB write before each launch ----
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    cold = []
    for i in range(20):
        flush.fill_(i & 0xFF)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        ssa.forward_into(xg, pg, wl.num_groups, wl.num_heads, out, ws, stage="gn_stats")
        b.record(stream)
        torch.cuda.synchronize()
        cold.append(a.elapsed_time(b) / 1e3)
    del flush
    # restore a full, consistent result in `out`
    step()
    torch.cuda.synchronize()

    work = stage_work(wl)
    dom = max((s for s in stages if s != "gn_stats"), key=lambda s: per_stage[s])
    kind, amount = work[dom]
    peak = PEAK_BF16_TFLOPS if wl.dtype == "bf16" else PEAK_FP32_TFLOPS
    achieved = amount / per_stage[dom] / 1e12
    traffic = stored_traffic(dom, wl.name, tuple(names))
    roofline = {"bound": "mfma", "kernel": STAGE_KERNELS[dom], "achieved": round(achieved, 2),
                "peak": peak, "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                "traffic": traffic, "avg_launch_us": round(per_stage[dom] * 1e6, 2),
                "algorithmic_per_launch": amount}
    gn_bytes = work["gn_stats"][1]
    kernels = {s: {"avg_us": round(t * 1e6, 2),
                   ("TFLOP/s" if work[s][0] == "flops" else "GB/s"):
                       round(work[s][1] / t / (1e12 if work[s][0] == "flops" else 1e9), 2)}
               for s, t in per_stage.items()}
    cold_med = statistics.median(cold)

    line = {
        "metric": "block TFLOP/s",
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded, workload distributions)",
        "config": {"workload": wl.name, "B": wl.B, "C": wl.C, "H": wl.H, "W": wl.W,
                   "num_groups": wl.num_groups, "num_heads": wl.num_heads, "d": wl.d,
                   "launch": launch, "options": names},
        "other_launch": alt,
        "step_ms": step_ms,
        "pixels_per_s": round(wl.B * wl.T / elapsed * args.steps, 1),
        "pct_bf16_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "gn_stats_GBps": round(gn_bytes / per_stage["gn_stats"] / 1e9, 1),
        "gn_stats_cold_GBps": round(gn_bytes / cold_med / 1e9, 1),
        "kernels": kernels,
        "roofline": roofline,
        "cpu_baseline": None,
        "source_digest": source_digest(),
    }
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(wl, seed, od)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
