"""Benchmark of the NVFP4 block-scaled grouped GEMM on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload I] [--all]

A step is one call of the grouped GEMM (the whole hot path) on one batch of
seeded synthetic input that is already resident in HBM. The headline workload
is the largest grouped configuration (G=2: 4096x4096x8192 and 2048x7168x4096).
Timed calls rotate over enough input/output sets (>= 1 GiB in total) that the
256 MiB last-level cache cannot serve repeated calls ("cold"); the same-buffer
("hot") number is reported beside it.

Prints ONE JSON line on stdout. The roofline fraction uses the MI355X dense
f16 MFMA peak (the MFMA precision of the kernel) and the kernel's average
duration, timed with HIP events on the stream the kernel is launched on.
``cpu_baseline`` times the CPU oracle on the host cores on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "TFLOPS (2·Σm·n·k) and µs/call per grouped-GEMM config; % of MFMA peak"
PEAK_F16_TFLOPS = 2500.0  # MI355X dense f16/bf16 MFMA (published)
PEAK_FP4_TFLOPS = 10100.0  # MI355X dense fp4 MFMA (published)
PEAK_HBM_GBS = 8000.0
COLD_BYTES = 1 << 30
# Per-workload rows time at least this much back-to-back work (see time_workload).
PER_CONFIG_MIN_TIMED_MS = 2.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic(shapes):
    """FLOPs (2*m*n*k*l, real m) and bytes (A, B, tiled SFA/SFB and C, each once)."""
    fl = sum(2 * m * n * k * l for (m, n, k, l) in shapes)
    by = 0
    for (m, n, k, l) in shapes:
        by += l * (m * k // 2 + n * k // 2 + 2 * m * n)
        by += l * (-(-m // 128) * 128 + -(-n // 128) * 128) * (k // 16)
    return fl, by


def percentile(v, p):
    return float(np.percentile(np.asarray(v), p))


def fmt_us(v):
    return "n/a" if v is None else f"{v:.1f}"


def settle(call, seconds):
    """Runs the hot path back to back for about ``seconds`` before the warm-up
    steps. After the GPU has idled (input generation and upload take seconds
    on the host), its power management lets the first millisecond or so run at
    a high clock, then cuts the clock hard and takes some 10-20 ms to reach
    its steady state: the GEMM kernel's duration on the dense workload goes
    ~310 us -> ~390 us -> ~320 us over the first ~40 calls (rocprofv3 kernel
    trace of bench.py --steps 20 --warmup 5). A few warm-up steps end inside
    that dip, so the timed steps would measure the controller's transient, not
    the kernel. Returns the number of calls made."""
    import torch
    if seconds <= 0:
        return 0
    n = 0
    t0 = time.perf_counter()
    for _ in range(4):
        call(n)
        n += 1
    torch.cuda.synchronize()
    per = max((time.perf_counter() - t0) / 4, 1e-6)
    # the rest in one go (no synchronisation, so the GPU never idles)
    for _ in range(max(0, int(seconds / per) - 4)):
        call(n)
        n += 1
    torch.cuda.synchronize()
    return n


def time_workload(idx, steps, warmup, tile_config=-1, cold=True, split_mode=None, device_tables=False,
                  super_batch=False, pow2=False, settle_s=0.0, from_idle=False, min_timed_ms=0.0):
    """Times the grouped GEMM on workload ``idx``. ``device_tables``: through
    nvfp4_grouped_gemm_device (group tables in device memory); ``super_batch``:
    the groups of 15 calls of the workload in one launch (device tables);
    ``pow2``: the workload with power-of-two scales through
    nvfp4_grouped_gemm_pow2 (its status word checked afterwards).
    ``settle_s``: seconds of back-to-back calls before the warm-up steps (see
    settle). ``min_timed_ms``: time at least that much work, more than
    ``steps`` calls if need be (the per-call time is estimated from the
    settle): 20 calls of a few microseconds are a window of the same order as
    the latencies around it. ``from_idle``: also time ``steps`` calls after
    only the warm-up steps, straight after the input set-up (before the
    settle), as a run without the settle would."""
    import torch

    import moe_matmul_amd as mm
    from moe_matmul_amd import device as dev
    from moe_matmul_amd import synth

    device_tables = device_tables or super_batch
    if super_batch:
        shapes, groups = synth.make_super_batch(idx)
    elif pow2:
        shapes, groups = synth.make_workload(idx, scale_codes=synth.POW2_SCALE_CODES)
    else:
        shapes, groups = synth.make_workload(idx)
    base = dev.upload(shapes, groups)
    flops, nbytes = algorithmic(shapes)
    sets = [base]
    if cold:
        nsets = max(1, -(-COLD_BYTES // nbytes))
        for _ in range(nsets - 1):
            cp = []
            for d in base:
                e = {k: (v.clone() if hasattr(v, "clone") else v) for k, v in d.items() if k != "c"}
                e["c"] = e["c_store"][d["c_guard"]: d["c_guard"] + d["c"].numel()]
                cp.append(e)
            sets.append(cp)
    stream = torch.cuda.current_stream()
    # argument tables marshalled once, so the timed loop measures the library
    (ps,) = mm.prepare(problem_sizes=shapes)
    ptrs = [mm.prepare(ptrs_abc=a, ptrs_sfa_sfb=f) for a, f in (dev.pointer_tables(s) for s in sets)]
    ws = dev.workspace_for(shapes) if (split_mode is not None or pow2) else None
    tables = [dev.device_tables(shapes, s) for s in sets] if device_tables else None
    status = torch.zeros(1, dtype=torch.int32, device="cuda")

    def call(i, st=stream):
        if device_tables:
            t = tables[i % len(tables)]
            mm.nvfp4_grouped_gemm_device(t[0].data_ptr(), t[1].data_ptr(), t[2].data_ptr(), len(shapes), tile_config,
                                         0, st)
            return
        abc, sf = ptrs[i % len(ptrs)]
        if pow2:
            mm.nvfp4_grouped_gemm_pow2(ps, abc, sf, status.data_ptr(), len(shapes), ws.data_ptr(), ws.numel(),
                                       tile_config, -1 if split_mode is None else split_mode, st)
        elif split_mode is None:
            mm.nvfp4_grouped_gemm_config(ps, abc, sf, len(shapes), st, tile_config)
        else:
            mm.nvfp4_grouped_gemm_ex(ps, abc, sf, len(shapes), ws.data_ptr(), ws.numel(), tile_config,
                                     split_mode, st)

    idle_ms = None
    if from_idle:
        for i in range(warmup):
            call(i)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for i in range(steps):
            call(i)
        b.record(stream)
        torch.cuda.synchronize()
        idle_ms = a.elapsed_time(b) / steps
    settle_t0 = time.perf_counter()
    settle_calls = settle(call, settle_s)
    settle_wall = time.perf_counter() - settle_t0
    timed_steps = steps
    if min_timed_ms > 0 and settle_calls > 0:
        per_call_s = settle_wall / settle_calls
        timed_steps = min(max(steps, -(-int(min_timed_ms * 1e-3 * 1e6) // max(int(per_call_s * 1e6), 1))), 5000)
    for i in range(warmup):
        call(i)
    torch.cuda.synchronize()
    # The timed region: exactly `steps` back-to-back calls between two events.
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(timed_steps):
        call(i)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = start.elapsed_time(end)
    # Per-call distribution from a separate pass with an event after every call
    # (the events add a little time between calls, so they stay out of the
    # timed region).
    reps = min(steps, 100)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    evs[0].record(stream)
    for i in range(reps):
        call(i)
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    per_call = [evs[i].elapsed_time(evs[i + 1]) for i in range(reps)]  # ms
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    if device_tables:
        cfg = tile_config
        if cfg < 0:  # the entry point's default: 256x256 tiles (header of the C ABI)
            cfg = next(c for c in range(mm.nvfp4_num_tile_configs())
                       if (mm.nvfp4_tile_config_info(c)["bm"], mm.nvfp4_tile_config_info(c)["bn"]) == (256, 256))
        p0 = [0x1000] * 5
        geo = dict(config=cfg, split=0, grid=cus,
                   total_tiles=sum(mm.nvfp4_device_group_tiles(s, p0, tile_config) for s in shapes))
    else:
        # without a workspace (split_mode None: nvfp4_grouped_gemm_config) the library plans whole tiles
        geo = mm.nvfp4_launch_geometry(shapes, cus, tile_config, 0 if split_mode is None else split_mode)
    avg_s = total_ms / timed_steps / 1e3
    # The same calls replayed from a captured HIP graph: GPU time per call
    # without host launch overhead (what matters for the microsecond-sized
    # workloads).
    graph_us = None
    if split_mode is None:
        reps = min(steps, 50)
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            call(0, side)  # warm the side stream outside capture
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            for i in range(reps):
                call(i, side)
        g.replay()
        torch.cuda.synchronize()
        # capture idled the GPU: a few replays (at least ~30 ms of GPU time, the
        # power-management transient, but no more than 20 graphs: a thousand
        # queued replays of a graph of microsecond kernels made the next one
        # several times slower) before the timed one
        if settle_s > 0:
            t_rep = time.perf_counter()
            g.replay()
            torch.cuda.synchronize()
            t_replay = max(time.perf_counter() - t_rep, 1e-6)
            for _ in range(min(20, int(min(settle_s, 0.03) / t_replay) + 1)):
                g.replay()
            torch.cuda.synchronize()
        ga, gb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ga.record(stream)
        g.replay()
        gb.record(stream)
        torch.cuda.synchronize()
        graph_us = ga.elapsed_time(gb) / reps * 1e3
        del g
    name = synth.WORKLOADS[idx]["name"]
    if super_batch:
        name = f"superbatch{synth.SUPER_BATCH_COPIES}x_{name}"
    if pow2:
        name = f"{name}_pow2scales"
        if int(status.item()) != 0:
            raise RuntimeError(f"{name}: the power-of-two entry point reported a scale outside its set")
    return dict(
        workload=name, device_tables=device_tables, pow2=pow2, shapes=[list(s) for s in shapes], flops=flops, bytes=nbytes,
        total_ms=total_ms, wall_s=wall, ms_per_call=total_ms / timed_steps, timed_steps=timed_steps,
        us_median=percentile(per_call, 50) * 1e3, us_p10=percentile(per_call, 10) * 1e3, us_p90=percentile(per_call, 90) * 1e3,
        tflops=flops / avg_s / 1e12, gbs=nbytes / avg_s / 1e9, sets=len(sets), tile_config=geo["config"],
        tiles=geo["total_tiles"], grid=geo["grid"], split=geo["split"], graph_us_per_call=graph_us,
        settle_calls=settle_calls, settle_s=settle_wall, from_idle_ms_per_call=idle_ms,
    )


def config_row(idx, r):
    """One workload's row of the JSON line: time per call, throughput, and the
    fraction of the roofline that bounds it (the dense f16 MFMA peak or HBM,
    whichever takes longer for the algorithmic FLOPs and bytes)."""
    t = r["ms_per_call"] / 1e3
    t_mfma = r["flops"] / (PEAK_F16_TFLOPS * 1e12)
    t_hbm = r["bytes"] / (PEAK_HBM_GBS * 1e9)
    bound = "mfma" if t_mfma >= t_hbm else "hbm"
    return {
        "workload": r["workload"], "index": idx, "shapes_mnkl": r["shapes"],
        "us_per_call": {"timed_mean": round(r["ms_per_call"] * 1e3, 2), "median": round(r["us_median"], 2),
                        "graph_replay": None if r["graph_us_per_call"] is None else round(r["graph_us_per_call"], 2)},
        "timed_calls": r["timed_steps"],
        "tflops": round(r["tflops"], 2), "algorithmic_gbs": round(r["gbs"], 1),
        "roofline": {"bound": bound, "frac": round(max(t_mfma, t_hbm) / t, 4),
                     "mfma_frac": round(t_mfma / t, 4), "hbm_frac": round(t_hbm / t, 4),
                     "roofline_us": round(max(t_mfma, t_hbm) * 1e6, 3)},
        "plan": {"tile_config": r["tile_config"], "stream_k": bool(r["split"]), "tiles": r["tiles"], "grid": r["grid"]},
    }


def cpu_model():
    """The host CPU's model name (Linux), or the platform's processor string."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(idx, max_rows=None, min_seconds=10.0):
    """The CPU oracle, as it stands, on workload ``idx`` (rows capped per group)."""
    from threadpoolctl import threadpool_info

    import oracle.nvfp4_oracle as O
    from moe_matmul_amd import synth

    shapes, groups = synth.make_workload(idx)
    fl = 0
    reps = 0
    t0 = time.perf_counter()
    # repeat the whole sample until at least min_seconds of CPU work
    while reps == 0 or time.perf_counter() - t0 < min_seconds:
        for (m, n, k, l), g in zip(shapes, groups):
            rows = m if max_rows is None else min(m, max_rows)
            O.gemm_group(m, n, k, l, g["a"], g["b"], g["sfa"], g["sfb"], rows=np.arange(rows))
            fl += 2 * rows * n * k * l
        reps += 1
    dt = time.perf_counter() - t0
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    sample = (f"{synth.WORKLOADS[idx]['name']}, " +
              ("all rows" if max_rows is None else f"first {max_rows} rows per group") +
              f", {reps} pass(es), {fl / 1e9:.1f} GFLOP of C in {dt:.1f} s (float64 dequant + BLAS, C and S)"
              f"; BLAS threads {threads} of {os.cpu_count()} host CPUs, {cpu_model()}")
    return dict(value=fl / dt / 1e12, unit="TFLOP/s", cores=int(threads), kind="oracle", sample=sample,
                seconds=dt, cpu_count=os.cpu_count())


def copy_calibration(nbytes=1 << 30, reps=3):
    """A plain device-to-device copy of known size (nbytes read, nbytes written),
    for scaling the HBM traffic counters (FETCH_SIZE / WRITE_SIZE) of the GEMM
    kernel. Before each copy a 512 MiB buffer is overwritten, so the source is
    not resident in the 256 MiB last-level cache."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    src.random_(0, 256)
    dst = torch.empty_like(src)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    for r in range(reps):
        flush.fill_(r)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
    log(f"[bench] copy calibration: {reps} copies of {nbytes} bytes")


def load_traffic(workload_name):
    """HBM traffic per launch measured with rocprofv3 counters, if it was taken
    on the current kernel source (matched by hash); else None."""
    import hashlib
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    src = os.path.join(ROOT, "moe_matmul_amd", "csrc", "nvfp4_grouped_gemm.hip")
    digest = hashlib.sha256(open(src, "rb").read()).hexdigest()
    rec = json.load(open(p)).get(workload_name)
    if not rec or rec.get("source_sha256") != digest:
        return None
    return rec.get("bytes_per_launch")


def mainloop_probe(iters_f16=2000, iters_fp4=400, reps=5):
    """Times the inner loops of the two exact ways of applying the per-16 E4M3
    scales (libnvfp4_mainloop_probe.so) on every compute unit, and reads what
    the scaled FP4 conversion does with scales that are not powers of two."""
    import torch

    from moe_matmul_amd import probe

    grid = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.empty(grid * probe.SINK_PER_WORKGROUP, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    names = {probe.VARIANT_DEQUANT_F16: "(b) exact f16 dequantisation + v_mfma_f32_32x32x16_f16",
             probe.VARIANT_FP4_VALU: "(a) FP4 v_mfma_scale per 16-block + scale factors on the VALU",
             probe.VARIANT_BARE_F16: "bare v_mfma_f32_32x32x16_f16 loop (no dequantisation)",
             probe.VARIANT_BARE_FP4: "bare v_mfma_scale_f32_32x32x64_f8f6f4 loop, one 16-block per 32-K slice",
             probe.VARIANT_BARE_F16_16X16: "bare v_mfma_f32_16x16x32_f16 loop (same work per iteration)",
             probe.VARIANT_DEQUANT_128X64: "(b) on a 128x64 wave tile, one wave per SIMD",
             probe.VARIANT_DEQUANT_128X64_2W: "(b) on a 128x64 wave tile, two waves per SIMD",
             probe.VARIANT_DEQUANT_SHARED_B: "(b) on 64x128 wave tiles, B dequantised once and shared in LDS",
             probe.VARIANT_DEQUANT_SHARED_B_AHEAD: "the same with the exchange a step ahead",
             probe.VARIANT_BARE_F16_6BIT: "bare f16 loop, operands with 6 significant bits (like a * s)",
             probe.VARIANT_BARE_BF16_6BIT: "bare v_mfma_f32_32x32x16_bf16 loop, operands with 6 significant bits"}
    out = {"grid": grid, "variants": []}
    for v, iters in ((probe.VARIANT_BARE_F16, iters_f16), (probe.VARIANT_DEQUANT_F16, iters_f16),
                     (probe.VARIANT_FP4_VALU, iters_fp4), (probe.VARIANT_BARE_FP4, iters_f16),
                     (probe.VARIANT_BARE_F16_16X16, iters_f16), (probe.VARIANT_DEQUANT_128X64, iters_f16),
                     (probe.VARIANT_DEQUANT_128X64_2W, iters_f16), (probe.VARIANT_DEQUANT_SHARED_B, iters_f16),
                     (probe.VARIANT_DEQUANT_SHARED_B_AHEAD, iters_f16), (probe.VARIANT_BARE_F16_6BIT, iters_f16),
                     (probe.VARIANT_BARE_BF16_6BIT, iters_f16)):
        probe.nvfp4_probe_mainloop(v, iters, grid, sink.data_ptr(), stream.cuda_stream)  # warm-up
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record(stream)
        for _ in range(reps):
            probe.nvfp4_probe_mainloop(v, iters, grid, sink.data_ptr(), stream.cuda_stream)
        end.record(stream)
        torch.cuda.synchronize()
        ms = start.elapsed_time(end) / reps
        tf = probe.nvfp4_probe_flops_per_iteration(v) * iters * grid / (ms / 1e3) / 1e12
        out["variants"].append({"variant": v, "what": names[v], "iters": iters, "ms": ms, "tflops": tf,
                                "frac_f16_peak": tf / PEAK_F16_TFLOPS, "frac_fp4_peak": tf / PEAK_FP4_TFLOPS})
        log(f"[probe] {names[v]}: {tf:.0f} TFLOP/s of 32x32x16 work ({100 * tf / PEAK_F16_TFLOPS:.1f}% of the "
            f"f16 MFMA peak), {ms:.2f} ms for {iters} iterations on {grid} workgroups")
    scales = [1.0, 1.5, 1.875, 3.0, 0.75, 448.0]
    sc = torch.tensor(scales, dtype=torch.float32, device="cuda")
    res = torch.empty(len(scales), dtype=torch.int16, device="cuda")
    probe.nvfp4_probe_cvt_scale(sc.data_ptr(), len(scales), res.data_ptr(), stream.cuda_stream)
    torch.cuda.synchronize()
    got = res.cpu().view(torch.float16).float().tolist()
    out["cvt_scale"] = {"fp4_value": 1.0, "scales": scales, "results": got}
    log(f"[probe] v_cvt_scalef32_pk_f16_fp4 of 1.0 under scales {scales}: {got}")
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=4)
    ap.add_argument("--tile-config", type=int, default=-1)
    ap.add_argument("--all", action="store_true", help="also time every workload (to stderr / --out)")
    ap.add_argument("--super-batch", action="store_true",
                    help="also time 15 calls of workload 2 merged into one 120-group launch (device tables)")
    ap.add_argument("--pow2", action="store_true",
                    help="also time workloads 2-4 with power-of-two scales through nvfp4_grouped_gemm_pow2")
    ap.add_argument("--pow2-workloads", default="2,3,4", help="workloads of the --pow2 legs")
    ap.add_argument("--no-pow2-line", action="store_true",
                    help="leave out the power-of-two-scale leg of the headline workload from the JSON line")
    ap.add_argument("--sweep", action="store_true",
                    help="time every workload under every tile configuration and split mode (to stderr / --out)")
    ap.add_argument("--out", default=None, help="write the per-workload details as JSON here")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=None, help="cap rows per group of the CPU sample")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="minimum CPU work of the baseline leg")
    ap.add_argument("--mainloop-probe", action="store_true",
                    help="also time the inner loops of the two exact scale applications (measurement kernels)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain device copy of known size (counter calibration)")
    ap.add_argument("--settle", type=float, default=0.3,
                    help="seconds of untimed back-to-back calls before each leg's warm-up steps, so the timed "
                         "steps run at the GPU's steady-state clock (0 disables)")
    ap.add_argument("--no-per-config", action="store_true",
                    help="leave out the rows of the other workloads (0-3) from the JSON line")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}): "
              "the grouped GEMM library has no multi-GPU path", file=sys.stderr)
        sys.exit(2)

    import torch
    import moe_matmul_amd as mm
    from moe_matmul_amd import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    mm.load_library()

    if args.copy_calibration:
        copy_calibration()
    head = time_workload(args.workload, args.steps, args.warmup, args.tile_config, cold=True, settle_s=args.settle,
                         from_idle=True)
    hot = time_workload(args.workload, args.steps, args.warmup, args.tile_config, cold=False, settle_s=args.settle)
    log(f"[bench] cold {head['tflops']:.1f} TFLOP/s {head['ms_per_call'] * 1e3:.1f} us/call "
        f"(median of single calls {head['us_median']:.1f}; from idle, without the settle, "
        f"{head['from_idle_ms_per_call'] * 1e3:.1f}); "
        f"hot {hot['tflops']:.1f} TFLOP/s; graph replay {fmt_us(head['graph_us_per_call'])} us/call; "
        f"settle {head['settle_calls']} calls in {head['settle_s']:.2f} s")
    details = {"headline": head, "hot": hot}
    rows = []
    if not args.no_per_config:
        for i in range(5):
            if i == args.workload:
                r = head
            else:
                r = time_workload(i, args.steps, args.warmup, -1, cold=True, settle_s=args.settle,
                                  min_timed_ms=PER_CONFIG_MIN_TIMED_MS)
            rows.append(config_row(i, r))
            log(f"[bench] workload {i} {r['workload']}: {r['ms_per_call'] * 1e3:.2f} us/call over "
                f"{r['timed_steps']} calls (median "
                f"{r['us_median']:.2f}, graph replay {fmt_us(r['graph_us_per_call'])}), {r['tflops']:.1f} TFLOP/s, "
                f"{rows[-1]['roofline']['bound']}-bound, frac {rows[-1]['roofline']['frac']:.3f}")
        details["per_config"] = rows
    p2 = None
    if not args.no_pow2_line:
        # the same workload with power-of-two scales through the MX entry point
        p2 = time_workload(args.workload, max(20, args.steps // 2), args.warmup, args.tile_config, cold=True,
                           pow2=True, settle_s=args.settle)
        log(f"[bench] power-of-two scales (nvfp4_grouped_gemm_pow2): {p2['tflops']:.1f} TFLOP/s "
            f"{p2['ms_per_call'] * 1e3:.1f} us/call (median {p2['us_median']:.1f})")
        details["pow2_headline"] = p2
    if args.all:
        allres = []
        for i in range(5):
            for sm in (None, 0, 1):
                r = time_workload(i, max(20, args.steps // 2), 5, -1, cold=True, split_mode=sm)
                r["forced_split"] = sm
                allres.append(r)
                log(f"[bench] workload {i} {r['workload']} split={'auto' if sm is None else sm}: "
                    f"{r['tflops']:.1f} TFLOP/s, {r['ms_per_call'] * 1e3:.1f} us/call, median {r['us_median']:.1f} "
                    f"(p10 {r['us_p10']:.1f}, p90 {r['us_p90']:.1f}), {r['gbs']:.0f} GB/s, cfg {r['tile_config']}, "
                    f"split {r['split']}, {r['tiles']} tiles, grid {r['grid']}, "
                    f"graph replay {fmt_us(r['graph_us_per_call'])} us/call")
        cus = torch.cuda.get_device_properties(0).multi_processor_count
        for i in range(5):
            # the tile configuration the by-value entry point's heuristic picks
            cfg = mm.nvfp4_select_tile_config(synth.workload_shapes(i), cus)
            r = time_workload(i, max(20, args.steps // 2), 5, cfg, cold=True, device_tables=True)
            allres.append(r)
            log(f"[bench] workload {i} {r['workload']} device tables: {r['tflops']:.1f} TFLOP/s, "
                f"{r['ms_per_call'] * 1e3:.1f} us/call, median {r['us_median']:.1f}, cfg {r['tile_config']}, "
                f"{r['tiles']} tiles, graph replay {fmt_us(r['graph_us_per_call'])} us/call")
        details["all"] = allres
    if args.all or args.pow2:
        pres = []
        for i in [int(x) for x in args.pow2_workloads.split(",") if x.strip()]:
            r = time_workload(i, max(20, args.steps // 2), 5, -1, cold=True, pow2=True)
            pres.append(r)
            log(f"[bench] workload {i} {r['workload']} (nvfp4_grouped_gemm_pow2): {r['tflops']:.1f} TFLOP/s, "
                f"{r['ms_per_call'] * 1e3:.1f} us/call, median {r['us_median']:.1f}, cfg {r['tile_config']}, "
                f"split {r['split']}, {r['tiles']} tiles, graph replay {fmt_us(r['graph_us_per_call'])} us/call, "
                f"{100 * r['tflops'] / PEAK_FP4_TFLOPS:.1f}% of the FP4 MFMA peak")
        details["pow2"] = pres
    if args.all or args.super_batch:
        sb = time_workload(2, max(10, args.steps // 10), 3, args.tile_config, cold=True, super_batch=True)
        log(f"[bench] super-batch {sb['workload']} ({len(sb['shapes'])} groups, device tables): "
            f"{sb['tflops']:.1f} TFLOP/s, {sb['ms_per_call'] * 1e3:.1f} us/call, median {sb['us_median']:.1f}, "
            f"cfg {sb['tile_config']}, {sb['tiles']} tiles, "
            f"{100 * sb['tflops'] / PEAK_F16_TFLOPS:.1f}% of the f16 MFMA peak")
        details["super_batch"] = sb

    if args.sweep:
        sweep = []
        for i in range(5):
            for cfg in range(mm.nvfp4_num_tile_configs()):
                for sm in (0, 1):
                    r = time_workload(i, 20, 3, cfg, cold=True, split_mode=sm)
                    sweep.append(r)
                    log(f"[sweep] wl{i} cfg{cfg} split{sm}: {r['ms_per_call'] * 1e3:8.1f} us {r['tflops']:7.1f} TFLOP/s "
                        f"tiles {r['tiles']} grid {r['grid']}")
        details["sweep"] = sweep

    if args.mainloop_probe:
        details["mainloop_probe"] = mainloop_probe()

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args.workload, args.cpu_rows, args.cpu_seconds)
        log(f"[bench] cpu oracle {cpu['value'] * 1e3:.1f} GFLOP/s on {cpu['cores']} threads in {cpu['seconds']:.1f} s")

    achieved = head["flops"] / (head["total_ms"] / args.steps / 1e3) / 1e12
    traffic = load_traffic(head["workload"])
    line = {
        "metric": METRIC,
        "value": round(head["tflops"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_call"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": head["workload"],
            "groups": len(head["shapes"]),
            "shapes_mnkl": head["shapes"],
            "operands": "FP4 E2M1 A/B, E4M3 scale per 16 K, fp32 accumulate, fp16 C",
            "mfma": "v_mfma_f32_32x32x16_f16 on exactly dequantised operands",
            "tile_config": head["tile_config"],
            "stream_k": bool(head["split"]),
            "tiles": head["tiles"],
            "grid": head["grid"],
            "cache": f"cold: {head['sets']} rotating input/output sets",
        },
        "us_per_call": {"timed_mean": round(head["ms_per_call"] * 1e3, 2),
                        "median": round(head["us_median"], 2), "p10": round(head["us_p10"], 2),
                        "p90": round(head["us_p90"], 2),
                        "graph_replay": None if head["graph_us_per_call"] is None
                        else round(head["graph_us_per_call"], 2),
                        "timed_mean_from_idle": round(head["from_idle_ms_per_call"] * 1e3, 2)},
        "settle": {"seconds": round(head["settle_s"], 3), "calls": head["settle_calls"],
                   "why": "untimed back-to-back calls before the warm-up steps: after idling, the GPU's power "
                          "management runs the first ~1 ms fast, then throttles for ~10-20 ms before its steady "
                          "state; timed_mean_from_idle is the same K steps right after the input set-up"},
        "hot": {"value": round(hot["tflops"], 2), "us_median": round(hot["us_median"], 2)},
        "algorithmic_gbs": round(head["gbs"], 1),
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": PEAK_F16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_F16_TFLOPS, 4),
            "traffic": traffic,
        },
        "pow2_scales": None if p2 is None else {
            "entry_point": "nvfp4_grouped_gemm_pow2",
            "workload": p2["workload"],
            "scales": "E4M3 codes with mantissa 0 (2^-3 .. 2^3), same shapes and operand bytes distribution",
            "mfma": "v_mfma_scale_f32_32x32x64_f8f6f4 (E2M1, E8M0 scales), one 16-block per 32-K lane slice",
            "value": round(p2["tflops"], 2), "unit": "TFLOP/s",
            "us_per_call": round(p2["ms_per_call"] * 1e3, 2), "us_median": round(p2["us_median"], 2),
            "roofline": {"bound": "mfma", "achieved": round(p2["tflops"], 2), "peak": PEAK_FP4_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(p2["tflops"] / PEAK_FP4_TFLOPS, 4),
                         "usable_peak": PEAK_FP4_TFLOPS / 2, "traffic": load_traffic(p2["workload"]),
                         "note": "half of every FP4 MFMA's K is zero padding (16-element scale blocks on a "
                                 "32-element scale slice), so this instruction form tops out at half the FP4 peak"},
        },
        "per_config": rows,
        "cpu_baseline": None if cpu is None else {k: (round(v, 6) if isinstance(v, float) else v)
                                                  for k, v in cpu.items() if k in ("value", "unit", "cores",
                                                                                   "kind", "sample")},
    }
    if args.out:
        with open(args.out, "w") as f:
            json.dump(dict(details, cpu_baseline=cpu, line=line), f, indent=1)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
