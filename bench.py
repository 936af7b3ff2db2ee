"""Benchmark of the parameter-preparation hot path on one MI355X.

One step = one wt_prepare replay over the whole workload (shard gather +
projection fusion + 128x128-tile E4M3 quantization + packing into the
destination region), inputs already resident in HBM, destination written in
place (zero-copy). Default workload: one GPU's share of a Kimi-K2-shaped MoE
layer (96 experts, gate_up [4096x7168] fused from w1/w3, w2 [7168x2048],
8 row shards each; 8.46 GB of BF16).

Prints ONE JSON line on stdout. The CPU baseline is the oracle (plain C,
test infrastructure) run over the same workload bytes on the host's cores,
and its image is compared byte for byte with the GPU's output.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E peak


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="kimi_k2_moe",
                    choices=["kimi_k2_moe", "dense_7b", "dense_layer_h1024", "ragged_stress", "mla_many_small",
                             "mla_many_small_device", "act_dispatch_decode", "act_tokens_4096"])
    ap.add_argument("--dst-mode", default="zero-copy", choices=["zero-copy", "staged"],
                    help="how prepared bytes reach the destination region")
    ap.add_argument("--dst-kind", default="device", choices=["device", "pinned"],
                    help="destination region in device memory or pinned host memory")
    ap.add_argument("--watermark-mb", type=int, default=0, help="pipeline watermark (0 = library default)")
    ap.add_argument("--chunk-mb", type=int, default=0, help="pipeline chunk target (0 = library default)")
    ap.add_argument("--load-hint", type=int, default=0, help="wt_plan_options.load_hint (0 = library default)")
    ap.add_argument("--tile-group", type=int, default=0, help="wt_plan_options.tile_group (0 = library default)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="instead of the workload, time a plain device-to-device copy of BYTES (counter calibration)")
    ap.add_argument("--cpu-threads", type=int, default=0,
                    help="oracle threads for the all-cores leg (0 = the CPU share: min(16, usable cores))")
    ap.add_argument("--no-secondary", action="store_true",
                    help="time only the chosen workload (default: after the Kimi-K2 share, also the dense 7B "
                         "model, the ragged set and the pinned-host MLA pipeline, each verified)")
    ap.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "traffic.json"),
                    help="HBM bytes per launch measured with rocprofv3 counters for the current kernel")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the preparation path does not "
              "shard across GPUs; run it with --gpus 1.", file=sys.stderr)
        return 2

    import torch
    from bf16_fp8_weight_amd import wt  # noqa: F401  (raises when the library is not built)

    torch.cuda.set_device(0)
    if args.calibrate_copy:
        return _copy_calibration(args.calibrate_copy, args.steps, args.warmup)
    if args.workload.startswith("act_"):
        return _bench_act(args)
    res = _bench_prepare(args.workload, args, traffic_json=args.traffic_json, progress=True)
    res.pop("_wl")
    cpu, verified = res.pop("cpu_baseline"), res.pop("verified_vs_oracle")
    secondary = None
    if not args.no_secondary and args.workload == "kimi_k2_moe":
        secondary = {}
        for name in ("dense_7b", "ragged_stress", "mla_many_small"):
            r = _bench_prepare(name, args, baseline=False)
            r.pop("_wl")
            r.pop("cpu_baseline")
            secondary[name] = r
        if any(r["verified_vs_oracle"] is False for r in secondary.values()):
            verified = False

    line = {
        "metric": "prepared BF16 GB/s (shard gather+fuse+FP8 quant+pack) and % of HBM peak",
        "value": res["value"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic: seeded N(0, 0.02) BF16, random weights of the stated shapes",
        "config": res["config"],
        "pct_hbm_peak": res["roofline"]["frac"],
        "roofline": res["roofline"],
        "cpu_baseline": cpu,
        "verified_vs_oracle": verified,
    }
    if "pipeline" in res:
        line["pipeline"] = res["pipeline"]
    if secondary is not None:
        line["secondary"] = secondary
    print(json.dumps(line), flush=True)
    return 0 if verified in (None, True) else 1


def _shards_per_tensor(wl):
    counts = sorted({len(p.shard_rows) for o in wl.outputs for p in o.parts})
    return counts[0] if len(counts) == 1 else f"{counts[0]}-{counts[-1]}"


def _bench_prepare(name: str, args, traffic_json: str | None = None, progress: bool = False,
                   baseline: bool = True) -> dict:
    """Builds workload `name` on the GPU, times args.steps replays of its plan
    (HIP events on the launch stream around every replay, wall clock around
    all of them), then compares the whole destination image with the oracle's
    (and, with baseline=True, times the oracle as the CPU baseline)."""
    import torch
    from bf16_fp8_weight_amd import workloads as W
    from bf16_fp8_weight_amd import wt

    t0 = time.time()
    if name == "mla_many_small_device":
        wl = W.mla_many_small(device="cuda", host=False)
    else:
        wl = W.WORKLOADS[name](device="cuda")
    torch.cuda.synchronize()
    log(f"workload {wl.name}: {len(wl.outputs)} outputs, {wl.input_bytes / 1e9:.3f} GB BF16 in, "
        f"{wl.n_tiles} tiles, generated in {time.time() - t0:.1f}s")

    if args.dst_kind == "device":
        dst = torch.full((wl.dst_bytes,), 0xA5, dtype=torch.uint8, device="cuda")
        dst_kind = wt.WT_MEM_DEVICE
    else:
        dst = torch.full((wl.dst_bytes,), 0xA5, dtype=torch.uint8).pin_memory()
        dst_kind = wt.WT_MEM_PINNED_HOST
    opts = wt.wt_plan_options_init()
    opts.dst_write_mode = wt.WT_DST_STAGED if args.dst_mode == "staged" else wt.WT_DST_ZERO_COPY
    if args.watermark_mb:
        opts.watermark_bytes = args.watermark_mb << 20
    if args.chunk_mb:
        opts.chunk_bytes = args.chunk_mb << 20
    opts.load_hint = args.load_hint
    opts.tile_group = args.tile_group
    plan = wt.Plan(wl, dst, dst_kind, opts)
    info = plan.info()
    log(f"plan: {info}")
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream

    for _ in range(args.warmup):
        plan.prepare(sp)
    torch.cuda.synchronize()

    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_begin = time.perf_counter()
    for i in range(args.steps):
        starts[i].record(stream)
        plan.prepare(sp)
        ends[i].record(stream)
    torch.cuda.synchronize()
    t_total = time.perf_counter() - t_begin
    launch_ms = sorted(s.elapsed_time(e) for s, e in zip(starts, ends))
    avg_launch_s = sum(launch_ms) / len(launch_ms) / 1e3
    med_launch_ms = launch_ms[len(launch_ms) // 2] if len(launch_ms) % 2 else \
        (launch_ms[len(launch_ms) // 2 - 1] + launch_ms[len(launch_ms) // 2]) / 2
    ms_per_step = t_total / args.steps * 1e3

    in_bytes = wl.input_bytes
    alg_bytes = wl.algorithmic_bytes
    value = in_bytes / (t_total / args.steps) / 1e9          # prepared BF16 GB/s, whole job
    achieved = alg_bytes / avg_launch_s / 1e9                # algorithmic HBM GB/s of the launch
    log(f"{wl.name} steps {args.steps}: {ms_per_step:.4f} ms/step wall, launch avg {avg_launch_s * 1e3:.4f} ms "
        f"(median {med_launch_ms:.4f}, min {launch_ms[0]:.4f}, max {launch_ms[-1]:.4f}); prepared {value:.1f} GB/s; "
        f"HBM {achieved:.1f} GB/s = {achieved / HBM_PEAK_GBPS:.3f} of peak")

    out = {"_wl": wl}
    if wl.shard_mem == "host":
        out["pipeline"] = _h2d_ceiling(wl, ms_per_step, args.steps)
    if progress and info["n_units"] > 1:
        out.setdefault("pipeline", {})["progress"] = _progress_timeline(plan, info["n_units"], sp)

    traffic = None
    if traffic_json:
        try:
            with open(traffic_json) as f:
                tj = json.load(f)
            if tj.get("workload") == wl.name and tj.get("kernel_source_sha") == _kernel_sha():
                traffic = tj.get("bytes_per_launch")
        except (OSError, ValueError):
            pass

    cpu, verified = None, None
    if not args.no_cpu_baseline:
        cpu, verified = _verify(wl, dst, args.cpu_threads, baseline=baseline)
    plan.close()

    out.update({
        "value": round(value, 2),
        "ms_per_step": round(ms_per_step, 5),
        "config": {
            "workload": wl.name,
            "outputs": len(wl.outputs),
            "input_bytes": in_bytes,
            "output_bytes": wl.output_bytes,
            "tiles": wl.n_tiles,
            "shards_per_tensor": _shards_per_tensor(wl),
            "dst_mode": f"{args.dst_mode}, {args.dst_kind} destination, {wl.shard_mem}-resident shards",
        },
        "roofline": {
            "bound": "h2d" if wl.shard_mem == "host" else "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": alg_bytes,
            "avg_launch_ms": round(avg_launch_s * 1e3, 5),
            "median_launch_ms": round(med_launch_ms, 5),
            "min_launch_ms": round(launch_ms[0], 5),
            "launches_per_step": info["n_launches"],
        },
        "cpu_baseline": cpu,
        "verified_vs_oracle": verified,
    })
    if wl.shard_mem == "host":
        # bound by the host link: the fraction that matters is the overlap with a bare copy
        out["roofline"]["frac_note"] = "HBM fraction of a host-link-bound replay; see pipeline.overlap_eff"
    del dst
    torch.cuda.empty_cache()
    return out


def _h2d_ceiling(wl, ms_per_step: float, steps: int) -> dict:
    """Times a bare host-to-device copy of the workload's pinned shard arena
    (the same bytes the pipeline's first stage moves) and relates it to the
    pipeline's time per step."""
    import torch

    arena = wl.arena
    dev = torch.empty(arena.numel(), dtype=torch.uint8, device="cuda")
    dev.copy_(arena, non_blocking=True)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = max(3, min(steps, 10))
    s.record()
    for _ in range(n):
        dev.copy_(arena, non_blocking=True)
    e.record()
    torch.cuda.synchronize()
    t_h2d = s.elapsed_time(e) / n
    out = {"h2d_ms": round(t_h2d, 4), "h2d_GBps": round(arena.numel() / t_h2d / 1e6, 2),
           "pipeline_ms": round(ms_per_step, 4), "overlap_eff": round(t_h2d / ms_per_step, 4),
           "arena_bytes": int(arena.numel())}
    log(f"pipeline: bare H2D of the {arena.numel() / 1e9:.3f} GB arena {t_h2d:.3f} ms "
        f"({out['h2d_GBps']} GB/s); pipeline {ms_per_step:.3f} ms; overlap efficiency {out['overlap_eff']}")
    return out


def _progress_timeline(plan, n_units: int, stream: int) -> dict:
    """One more replay with completion counters attached: the host polls each
    unit's word in order and records when it saw it, i.e. when that part of
    the destination region could start its transfer."""
    import torch
    from bf16_fp8_weight_amd import wt

    words = torch.zeros(n_units, dtype=torch.int64).pin_memory()
    wt.wt_plan_set_progress(plan.handle, words.data_ptr(), n_units)
    torch.cuda.synchronize()
    seen = []
    t0 = time.perf_counter()
    plan.prepare(stream)
    for u in range(n_units):
        if not wt.wt_progress_wait(words.data_ptr() + 8 * u, 1, 60 * 10**9):
            raise RuntimeError(f"completion unit {u} not reached within 60 s")
        seen.append((time.perf_counter() - t0) * 1e3)
    torch.cuda.synchronize()
    t_sync = (time.perf_counter() - t0) * 1e3
    wt.wt_plan_set_progress(plan.handle, 0, 0)
    gaps = sorted(b - a for a, b in zip(seen, seen[1:])) or [0.0]
    out = {"units": n_units, "first_unit_ms": round(seen[0], 3), "last_unit_ms": round(seen[-1], 3),
           "median_gap_ms": round(gaps[len(gaps) // 2], 3), "replay_sync_ms": round(t_sync, 3)}
    log(f"progress: {n_units} units; first seen by the host at {seen[0]:.3f} ms, last at {seen[-1]:.3f} ms, "
        f"replay synchronized at {t_sync:.3f} ms")
    return out


def _copy_calibration(nbytes: int, steps: int, warmup: int) -> int:
    """Plain copy of nbytes (reads nbytes, writes nbytes) on the current stream."""
    import torch

    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    for _ in range(warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(steps):
        dst.copy_(src)
    e.record()
    torch.cuda.synchronize()
    t = s.elapsed_time(e) / 1e3 / steps
    print(json.dumps({"metric": "copy_calibration", "bytes_copied": nbytes, "ms_per_copy": round(t * 1e3, 5),
                      "GBps_read_plus_write": round(2 * nbytes / t / 1e9, 1)}), flush=True)
    return 0


def _kernel_sha() -> str:
    from bf16_fp8_weight_amd.traffic import kernel_sha

    return kernel_sha()


def _cpu_info() -> dict:
    """The host's CPU: model name, logical cores, and the cores this process
    may use (its affinity mask). One GPU's share of a GPU machine is 16 threads."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count() or 1
    return {"cpu_model": model, "machine_cores": os.cpu_count(), "usable_cores": usable}


def _verify(wl, dst, threads: int, baseline: bool = True):
    """Runs the oracle over the whole workload on the host, one thread per
    output on the CPU share (min(16, usable cores) threads unless given), and
    compares its image with the GPU's destination byte for byte. With
    baseline=True it also reports that run as the CPU baseline, next to a
    single-threaded run of the oracle over a bounded sample of the outputs."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import oracle
    import oracle_glue

    oracle.build(force=False)
    ci = _cpu_info()
    n = threads or max(1, min(16, ci["usable_cores"]))
    t0 = time.time()
    outs = oracle_glue.oracle_outputs(wl)  # D2H of the shard bytes (not timed)
    log(f"cpu baseline: copied {wl.input_bytes / 1e9:.2f} GB of shards to host in {time.time() - t0:.1f}s")
    img = np.full(wl.dst_bytes, 0xA5, dtype=np.uint8)
    t1 = time.perf_counter()
    with ThreadPoolExecutor(n) as ex:
        list(ex.map(lambda o: oracle.prepare([o], wl.dst_bytes, img), outs))
    dt = time.perf_counter() - t1
    got = dst.cpu().numpy()
    ok = bool(np.array_equal(got, img))
    del got
    log(f"{wl.name}: oracle {dt:.2f}s on {n} threads = {wl.input_bytes / dt / 1e9:.3f} GB/s; GPU output "
        f"{'identical to' if ok else 'DIFFERS from'} the oracle image")
    if not baseline:
        return None, ok
    # single thread: the outputs in table order until 512 MB of BF16 input
    # (or all of them), into a scratch image
    in_bytes = [sum(p.rows for p in o.parts) * o.cols * 2 for o in wl.outputs]
    k, acc = 0, 0
    while k < len(outs) and acc < (512 << 20):
        acc += in_bytes[k]
        k += 1
    scratch = np.zeros(wl.dst_bytes, dtype=np.uint8)
    t2 = time.perf_counter()
    oracle.prepare(outs[:k], wl.dst_bytes, scratch)
    dt1 = time.perf_counter() - t2
    log(f"{wl.name}: oracle single-threaded {dt1:.2f}s over {k} outputs ({acc / 1e9:.3f} GB) = "
        f"{acc / dt1 / 1e9:.3f} GB/s; CPU {ci['cpu_model']}, {ci['machine_cores']} logical cores, "
        f"{ci['usable_cores']} usable")
    return {
        "value": round(wl.input_bytes / dt / 1e9, 4),
        "unit": "GB/s",
        "cores": n,
        "kind": "oracle",
        "sample": f"the whole workload ({len(outs)} outputs, {wl.input_bytes} B BF16), one thread per output "
                  f"on {n} threads",
        "seconds": round(dt, 2),
        "threads": n,
        "all_cores_GBps": round(wl.input_bytes / dt / 1e9, 4),
        "single_thread_GBps": round(acc / dt1 / 1e9, 4),
        "single_thread_sample": f"the first {k} outputs in table order ({acc} B BF16), one thread",
        "single_thread_seconds": round(dt1, 2),
        **ci,
    }, ok


def _bench_act(args) -> int:
    """Block-scaled FP8 quantization of token activations: one launch per
    step, timed with HIP events on the launch stream around every launch."""
    import numpy as np
    import torch
    from bf16_fp8_weight_amd import workloads as W
    from bf16_fp8_weight_amd import wt

    if args.workload == "act_dispatch_decode":
        wl = W.act_dispatch(device="cuda")
    else:
        wl = W.act_tokens(device="cuda", tokens=4096)
    H, n_out = wl.hidden, wl.n_out
    if wl.interleaved:
        buf = torch.full((n_out * wl.slot,), 0xA5, dtype=torch.uint8, device="cuda")
        q_ptr, s_ptr = buf.data_ptr(), buf.data_ptr() + H
    else:
        qt = torch.full((n_out * H,), 0xA5, dtype=torch.uint8, device="cuda")
        st = torch.full((n_out * 4 * wl.nb,), 0xA5, dtype=torch.uint8, device="cuda")
        q_ptr, s_ptr = qt.data_ptr(), st.data_ptr()
    idx_ptr = wl.index.data_ptr() if wl.index is not None else 0
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream

    def launch():
        wt.wt_quantize_act_b128(wl.x.data_ptr(), wl.tokens, H, H, idx_ptr, n_out, q_ptr, wl.q_stride, s_ptr,
                                wl.s_stride, sp)

    for _ in range(args.warmup):
        launch()
    torch.cuda.synchronize()
    # A launch lasts microseconds: one event pair around back-to-back launches
    # measures the kernel's throughput; a pair around each launch would add
    # the event and dispatch overhead (reported beside it).
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        launch()
    e1.record(stream)
    torch.cuda.synchronize()
    t_total = time.perf_counter() - t0
    avg_s = e0.elapsed_time(e1) / args.steps / 1e3
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    for i in range(args.steps):
        starts[i].record(stream)
        launch()
        ends[i].record(stream)
    torch.cuda.synchronize()
    bracketed = sum(a.elapsed_time(b) for a, b in zip(starts, ends)) / args.steps / 1e3
    # the same launches replayed from a HIP graph (no host launch cost between them)
    n_graph = 100
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        launch_on = lambda st: wt.wt_quantize_act_b128(wl.x.data_ptr(), wl.tokens, H, H, idx_ptr, n_out, q_ptr,
                                                       wl.q_stride, s_ptr, wl.s_stride, st)
        launch_on(side.cuda_stream)
    side.synchronize()
    with torch.cuda.graph(graph):
        for _ in range(n_graph):
            launch_on(torch.cuda.current_stream().cuda_stream)
    graph.replay()
    torch.cuda.synchronize()
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    g0.record(stream)
    for _ in range(5):
        graph.replay()
    g1.record(stream)
    torch.cuda.synchronize()
    graph_s = g0.elapsed_time(g1) / (5 * n_graph) / 1e3
    del graph
    value = wl.input_bytes / avg_s / 1e9
    achieved = wl.algorithmic_bytes / avg_s / 1e9
    log(f"{wl.name}: {n_out} rows; back-to-back {avg_s * 1e6:.2f} us/launch, bracketed one by one "
        f"{bracketed * 1e6:.2f} us, from a graph {graph_s * 1e6:.2f} us; host wall {t_total / args.steps * 1e6:.2f} "
        f"us/launch; HBM {achieved:.1f} GB/s = {achieved / HBM_PEAK_GBPS:.3f} "
        f"({wl.algorithmic_bytes / graph_s / 1e9 / HBM_PEAK_GBPS:.3f} from the graph)")

    cpu = None
    verified = None
    if not args.no_cpu_baseline:
        sys.path.insert(0, os.path.join(ROOT, "tests"))
        import oracle

        oracle.build(force=False)
        x = wl.x.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        idx = wl.index.cpu().numpy() if wl.index is not None else None
        nb = wl.nb
        wq = np.full((n_out, H), 0xA5, dtype=np.uint8)
        ws = np.full((n_out, 4 * nb), 0xA5, dtype=np.uint8)
        t1 = time.perf_counter()
        oracle.quantize_act(x, cols=H, index=idx, n_out=n_out, q=wq, scales=ws)
        dt = time.perf_counter() - t1
        if wl.interleaved:
            got = buf.cpu().numpy().reshape(n_out, wl.slot)
            gq, gs = got[:, :H], got[:, H:H + 4 * nb]
        else:
            gq, gs = qt.cpu().numpy().reshape(n_out, H), st.cpu().numpy().reshape(n_out, 4 * nb)
        verified = bool(np.array_equal(gq, wq) and np.array_equal(gs, ws))
        cpu = {"value": round(wl.input_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
               "sample": f"the whole workload ({n_out} rows x {H}), one thread", "seconds": round(dt, 3),
               "threads": 1, "single_thread_GBps": round(wl.input_bytes / dt / 1e9, 4), **_cpu_info()}
        log(f"cpu baseline: oracle {dt:.3f}s; GPU output {'identical to' if verified else 'DIFFERS from'} the oracle")

    line = {
        "metric": "quantized BF16 activation GB/s (1x128 block-scaled FP8, gather into send slots) and % of HBM peak",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(avg_s * 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic: seeded Student-t(3) activations with 8 outlier channels x50",
        "config": {"workload": wl.name, "tokens": wl.tokens, "hidden": H, "rows_out": n_out,
                   "layout": "interleaved send slots" if wl.interleaved else "separate codes and scales"},
        "pct_hbm_peak": round(achieved / HBM_PEAK_GBPS, 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": None,
                     "algorithmic_bytes_per_launch": wl.algorithmic_bytes, "avg_launch_ms": round(avg_s * 1e3, 6),
                     "launches_per_step": 1, "bracketed_launch_ms": round(bracketed * 1e3, 6),
                     "graph_launch_ms": round(graph_s * 1e3, 6),
                     "graph_frac": round(wl.algorithmic_bytes / graph_s / 1e9 / HBM_PEAK_GBPS, 4),
                     "host_wall_ms_per_launch": round(t_total / args.steps * 1e3, 6)},
        "cpu_baseline": cpu,
        "verified_vs_oracle": verified,
    }
    print(json.dumps(line), flush=True)
    return 0 if verified in (None, True) else 1


if __name__ == "__main__":
    sys.exit(main())
