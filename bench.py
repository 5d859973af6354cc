"""Benchmark: frames/s of the integer motion + PSNR sums on 3840x2160 8-bit 4:2:0, one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c3] [--moments]
                    [--motion-v2] [--no-cpu] [--no-probe] [--no-streaming]
    python bench.py --workload c3 --traffic-from FETCH.csv WRITE.csv   (host only, see below)

A step is one pass of the whole path over one batch: one iir_submit_clip of the 50-frame clip
(resident in HBM before timing starts) and one iir_collect of its 50 results; step k is submitted
before step k-1 is collected, so the host work overlaps the GPU. W untimed steps, then K timed
steps between two device synchronisations. Prints one JSON line.

roofline: the main kernel's algorithmic bytes per launch (every ref and dist sample read once,
plus the blurred-luma state read and written once per launch) divided by its mean duration,
measured with HIP events on the context's stream, against the 8 TB/s HBM peak. traffic: HBM bytes
per launch from the committed rocprofv3 counter summary for this workload, reported only while
the kernel source still matches the one the counters were taken on.
ceilings_GBps: the memory ceilings measured by the library's probes (16-byte non-temporal reads,
writes and copies of a 1 GiB buffer), and roofline.frac_of_read_ceiling the kernel's achieved
bandwidth against the read ceiling (skip with --no-probe).
streaming: the same frames submitted one pair per call (one launch per frame, the motion state
crossing launches through the device ring): frames/s of a context without events, and the
kernel time per launch from a second context with an event pair per launch (skip with
--no-streaming); `coalesced` is the same with iir_set_coalesce recording 8 pairs per launch. Not
the headline value, which is the batch of 50.
--traffic-from turns two rocprofv3 counter-collection CSVs of `bench.py --probe` runs (one with
--pmc FETCH_SIZE, one with --pmc WRITE_SIZE) into profiles/frames_kernel_<workload>_traffic.json:
each counter's mean KiB per main-kernel dispatch, scaled by what the same counter reads for the
copy probe (probe_copy moves a known 1 GiB in and 1 GiB out per dispatch).
cpu_baseline: the plain C oracle (single thread) over the same frames, on the host.
--moments runs the same workload with the luma moments summed in the same pass (IIR_FLAG_MOMENTS):
the bytes moved are the same, the arithmetic per sample grows; its traffic summary is kept under
the workload name with a _moments suffix. --motion-v2 replaces the blurred-frame SAD by motion v2
(the filter of the frame difference; 8 to 16 bits), suffix _v2; its state across launches is the
last reference luma frame (W H samples read and written once per launch) instead of the blurred
plane (2 bytes per pixel each way).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
# the frames kernel's sources: its templates and the units that instantiate them
KERNEL_SRCS = [os.path.join(ROOT, "integer_image_reductions_amd", "csrc", n) for n in
               ("iir_frames.h", "iir_frames_8.hip", "iir_frames_8_one.hip", "iir_frames_10.hip",
                "iir_frames_16.hip", "iir_frames_8_v2.hip", "iir_frames_10_v2.hip",
                "iir_frames_16_v2.hip")]

WORKLOADS = {
    "c3": "3840x2160 8-bit 4:2:0, 50 frame pairs, motion SAD + Y/U/V SSE",
    "c4": "3840x2160 10-bit 4:2:0 (uint16), 50 frame pairs, motion SAD + Y/U/V SSE",
    "c2": "1920x1080 8-bit 4:2:0, 48 frame pairs, motion SAD + Y/U/V SSE",
    "c1": "576x324 8-bit 4:2:0, 10 frame pairs, motion SAD + Y/U/V SSE",
    "c5": "960x544 8-bit 4:2:0, 301-frame resident clip, motion SAD + Y/U/V SSE",
    "c6": "3840x2160 16-bit 4:2:0 (uint16), 50 frame pairs, motion SAD + Y/U/V SSE "
          "(the 16-bit path at the 4K shape; not one of the pages' clips)",
}


def describe(workload: str, moments: bool, motion_v2: bool) -> str:
    text = WORKLOADS[workload]
    if motion_v2:
        text = text.replace("motion SAD", "motion v2 SAD")
    return text + (" + luma moments" if moments else "")


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def _code_only(text: str) -> str:
    """C++ source without its comments and with whitespace runs collapsed: a comment edit does not
    change the compiled kernel, so it must not void the counters taken on it."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_sha() -> str:
    """Hash of the frames kernel's code (its sources with the comments stripped)."""
    h = hashlib.sha256()
    for path in KERNEL_SRCS:
        with open(path, encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
        h.update(b"\0")
    return h.hexdigest()


def algorithmic_bytes(w: int, h: int, bpc: int, frames: int, motion_v2: bool = False) -> int:
    """Bytes one launch must move: each sample of the 6 planes of every frame pair read once, and
    the state carried between launches read once and written once: the blurred luma (uint16 per
    luma pixel), or with motion v2 the last reference luma frame (one sample per pixel)."""
    b = 1 if bpc == 8 else 2
    n, nc = w * h, ((w + 1) // 2) * ((h + 1) // 2)
    state = 2 * b * n if motion_v2 else 4 * n
    return frames * 2 * b * (n + 2 * nc) + state


def load_traffic(workload: str):
    path = os.path.join(ROOT, "profiles", f"frames_kernel_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("kernel_sha256") != kernel_sha():
        log("traffic counters were taken on a different kernel source; reporting null")
        return None
    return d.get("hbm_bytes_per_launch")


PROBE_BYTES = 1 << 30


def _counter_means(path: str, counter: str):
    """Mean counter value (KiB) per dispatch of the main kernel and of the copy probe."""
    import csv
    main, copy = [], []
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            v = float(r["Counter_Value"])
            if "frames_kernel" in r["Kernel_Name"]:
                main.append(v)
            elif "probe_copy" in r["Kernel_Name"]:
                copy.append(v)
    if not main or not copy:
        raise SystemExit(f"{path}: no {counter} rows for frames_kernel and probe_copy")
    return sum(main) / len(main), len(main), sum(copy) / len(copy), len(copy)


def write_traffic(workload: str, moments: bool, motion_v2: bool, fetch_csv: str,
                  write_csv: str, out_dir: str = None) -> dict:
    fm, fn, fc, fcn = _counter_means(fetch_csv, "FETCH_SIZE")
    wm, wn, wc, wcn = _counter_means(write_csv, "WRITE_SIZE")
    f_scale = PROBE_BYTES / (fc * 1024.0)
    w_scale = PROBE_BYTES / (wc * 1024.0)
    fetch_b, write_b = fm * 1024.0 * f_scale, wm * 1024.0 * w_scale
    wl = workload + ("_moments" if moments else "") + ("_v2" if motion_v2 else "")
    flag = (" --moments" if moments else "") + (" --motion-v2" if motion_v2 else "")
    d = {
        "workload": describe(workload, moments, motion_v2),
        "kernel_sha256": kernel_sha(),
        "fetch_kib_per_launch": fm, "fetch_dispatches": fn,
        "write_kib_per_launch": wm, "write_dispatches": wn,
        "copy_probe_bytes": PROBE_BYTES,
        "copy_probe_fetch_kib": fc, "copy_probe_write_kib": wc,
        "fetch_scale": f_scale, "write_scale": w_scale,
        "hbm_fetch_bytes_per_launch": fetch_b, "hbm_write_bytes_per_launch": write_b,
        "hbm_bytes_per_launch": fetch_b + write_b,
        "algorithmic_bytes_per_launch": None,
        "commands": [
            f"rocprofv3 --pmc {c} --output-format csv -d <dir_{c}> -o run -- python3 -u bench.py "
            f"--workload {workload}{flag} --steps 5 --warmup 1 --no-cpu --probe"
            for c in ("FETCH_SIZE", "WRITE_SIZE")] + [
            f"python bench.py --workload {workload}{flag} --traffic-from "
            "<dir_FETCH_SIZE>/run_counter_collection.csv <dir_WRITE_SIZE>/run_counter_collection.csv"],
    }
    import synth
    c = synth.CONFIGS[workload]
    d["algorithmic_bytes_per_launch"] = algorithmic_bytes(c["width"], c["height"], c["bpc"],
                                                          c["frames"], motion_v2)
    out_dir = out_dir or os.path.join(ROOT, "profiles")
    os.makedirs(out_dir, exist_ok=True)
    path = os.path.join(out_dir, f"frames_kernel_{wl}_traffic.json")
    with open(path, "w") as f:
        json.dump(d, f, indent=1)
        f.write("\n")
    return d


def launch_distribution(series, warm) -> dict:
    """Per-launch kernel microseconds of the timed launches: min, median, max, the means of the
    first and second halves, and the whole series (and the untimed warm-up launches before it),
    so a transient at the start of a run shows beside the mean."""
    us = [1e3 * v for v in series]
    s = sorted(us)
    n = len(s)
    med = s[n // 2] if n % 2 else 0.5 * (s[n // 2 - 1] + s[n // 2])
    h = max(n // 2, 1)
    return {"min": s[0], "median": med, "max": s[-1],
            "mean_first_half": sum(us[:h]) / h,
            "mean_second_half": sum(us[h:]) / max(n - h, 1) if n > 1 else us[0],
            "series": [round(v, 1) for v in us],
            "warmup_series": [round(1e3 * v, 1) for v in warm]}


def timed_upload(clip, ref, dist) -> dict:
    """Host-to-device copy of the whole clip (6 planes of every frame pair) from pinned host
    memory into the device planes the benchmark reads, timed with events on the current stream.
    It rewrites the same values; it is reported beside the kernel, never in `value`."""
    import numpy as np
    import torch
    src = []
    for host, devs in ((clip.ref, ref), (clip.dist, dist)):
        for a, d in zip(host, devs):
            a = np.ascontiguousarray(a)
            if a.dtype == np.uint16:
                a = a.view(np.int16)
            p = torch.from_numpy(a).pin_memory()
            src.append((p, d))
    nbytes = sum(p.numel() * p.element_size() for p, _ in src)
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for p, d in src:
        d.copy_(p, non_blocking=True)
    e1.record(s)
    e1.synchronize()
    ms = e0.elapsed_time(e1)
    return {"bytes": nbytes, "ms": ms, "GBps": nbytes / (ms * 1e-3) / 1e9,
            "us_per_frame_pair": 1e3 * ms / clip.frames,
            "source": "pinned host memory, one copy per plane of the whole clip"}


def measure_ceilings(dev) -> dict:
    """Read, write and copy ceilings (GB/s) of the library's probes over a 1 GiB buffer."""
    import torch
    import integer_image_reductions_amd as iir
    nbytes = PROBE_BYTES
    a = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    b = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    a.fill_(1)
    ceil = {}
    for mode, name, mult in ((0, "read", 1), (1, "write", 1), (2, "copy", 2)):
        ms = iir.probe_bandwidth(mode, a, b, iters=20)
        ceil[name] = mult * nbytes / (ms * 1e-3) / 1e9
    del a, b
    return ceil


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(clip, max_seconds: float = 20.0, moments: bool = False,
                 motion_v2: bool = False, min_seconds: float = 10.0):
    """The oracle over the leading frames of the same clip that fit `max_seconds` (the whole clip
    when it fits, repeated up to about `min_seconds` of work), single-threaded; frames/s. With
    moments, also the oracle's luma moments of every ref and dist frame."""
    import oracle

    def run(c):
        if motion_v2:
            oracle.clip_v2(c.ref, c.dist, clip.bpc)
        else:
            oracle.clip(c.ref, c.dist, clip.bpc)
        if moments:
            for t in range(c.frames):
                oracle.moments(c.ref[0][t], clip.bpc)
                oracle.moments(c.dist[0][t], clip.bpc)

    # one thread on one core: pin this process to a single CPU for the leg, then restore
    saved = os.sched_getaffinity(0)
    core = min(saved)
    os.sched_setaffinity(0, {core})
    try:
        return _cpu_leg(clip, run, max_seconds, min_seconds, core, len(saved))
    finally:
        os.sched_setaffinity(0, saved)


def _cpu_leg(clip, run, max_seconds, min_seconds, core, allowed):
    one = clip.slice(0, 1)
    t0 = time.perf_counter()
    run(one)
    per_frame = time.perf_counter() - t0
    n = max(1, min(clip.frames, int(max_seconds / max(per_frame, 1e-6))))
    passes = 1
    if n == clip.frames:
        est = max(per_frame * n, 1e-6)
        passes = max(1, min(int(max_seconds / est), math.ceil(min_seconds / est)))
    sub = clip.slice(0, n)
    t0 = time.perf_counter()
    for _ in range(passes):
        run(sub)
    dt = time.perf_counter() - t0
    return {"value": n * passes / dt, "unit": "frames/s", "cores": 1, "kind": "oracle",
            "pinned_cpu": core, "nproc": os.cpu_count(), "affinity_cpus": allowed,
            "cpu_model": cpu_model(),
            "sample": f"first {n} of {clip.frames} frame pairs of the same workload, "
                      f"{passes} pass{'es' if passes > 1 else ''}, single-threaded C oracle "
                      f"({dt:.1f} s)"}


def streaming(ref, dist, clip, moments: bool, motion_v2: bool, rounds: int = 6) -> dict:
    """Every frame pair its own submission (one launch per frame; the motion state crosses the
    launches through the device ring), in two contexts. The first records no events: frames/s
    over `rounds` passes of the clip, each pass submitted whole and collected once. The second
    brackets every launch with HIP events: the mean kernel time per launch against that launch's
    algorithmic bytes (one frame pair plus the state read and written), and its own frames/s,
    which the events slow down."""
    import torch
    import integer_image_reductions_amd as iir
    F = clip.frames
    group = min(F, 64)  # a context holds at most 64 pending submissions

    def passes(timing: bool, coalesce: int = 1):
        ctx = iir.Context(clip.width, clip.height, clip.bpc, max_batch=group, timing=timing,
                          moments=moments, motion_v2=motion_v2, coalesce=coalesce)
        frames = [ctx.prepare_clip(tuple(p[t:t + 1] for p in ref),
                                   tuple(p[t:t + 1] for p in dist)) for t in range(F)]

        def one_pass():
            for g in range(0, F, group):
                for fr in frames[g:g + group]:
                    ctx.submit_prepared(fr)
                ctx.collect()

        one_pass()
        torch.cuda.synchronize()
        if timing:
            ctx.kernel_stats(reset=True)
        t0 = time.perf_counter()
        for _ in range(rounds):
            one_pass()
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        stats = ctx.kernel_stats() if timing else None
        ctx.close()
        return rounds * F / dt, stats

    fps, _ = passes(False)
    fps_timed, (launches, total_ms) = passes(True)
    coalesce = min(8, group)
    fps_coalesced, _ = passes(False, coalesce)
    kernel_us = 1e3 * total_ms / max(launches, 1)
    alg = algorithmic_bytes(clip.width, clip.height, clip.bpc, 1, motion_v2)
    return {"frames_per_s": fps, "us_per_frame": 1e6 / fps,
            "kernel_us_per_launch": kernel_us, "launches": launches,
            "frames_per_s_with_events": fps_timed,
            "coalesced": {"frames_per_launch": coalesce, "frames_per_s": fps_coalesced,
                          "us_per_frame": 1e6 / fps_coalesced,
                          "mode": "the same one-pair submissions with iir_set_coalesce: "
                                  f"{coalesce} recorded pairs per launch"},
            "algorithmic_bytes_per_launch": alg,
            "achieved_GBps": alg / (kernel_us * 1e-6) / 1e9,
            "mode": f"one frame pair per submission, {group} submissions then one collect, "
                    f"{rounds} passes over {F} frames; frames/s without events, kernel time from "
                    f"a second context with an event pair per launch"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="c3", choices=sorted(WORKLOADS))
    ap.add_argument("--moments", action="store_true",
                    help="also sum the luma moments in the same pass (IIR_FLAG_MOMENTS)")
    ap.add_argument("--motion-v2", action="store_true",
                    help="motion v2 (filter of the frame difference) instead of the blurred SAD")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--probe", action="store_true",
                    help="measure the memory ceilings (the default; kept for older commands)")
    ap.add_argument("--no-probe", action="store_true", help="skip the memory-ceiling probes")
    ap.add_argument("--probe-first", action="store_true",
                    help="measure the memory ceilings before the frames launches, not after")
    ap.add_argument("--no-streaming", action="store_true",
                    help="skip timing one frame pair per submission (one launch per frame)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the HBM traffic summary from two counter CSVs and exit")
    args = ap.parse_args()

    wl = args.workload + ("_moments" if args.moments else "") + ("_v2" if args.motion_v2 else "")
    if args.traffic_from:
        print(json.dumps(write_traffic(args.workload, args.moments, args.motion_v2,
                                       *args.traffic_from)))
        return

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path would shard by frames: each GPU a run of frames plus the one before "
              "it, with no collective)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    import integer_image_reductions_amd as iir

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)

    log("generating", args.workload)
    clip = synth.make_clip(args.workload)
    ref, dist = iir.upload_planes(clip.ref, dev), iir.upload_planes(clip.dist, dev)
    torch.cuda.synchronize()
    F, W, H, bpc = clip.frames, clip.width, clip.height, clip.bpc
    log("uploaded", F, "frame pairs")
    upload = timed_upload(clip, ref, dist)
    log(f"upload {upload['GBps']:.1f} GB/s from pinned host memory")

    ceilings = None
    if args.probe_first and not args.no_probe:
        ceilings = measure_ceilings(dev)
        log("ceilings measured before the frames launches")

    # two batches in flight: step k is submitted before step k-1 is collected
    ctx = iir.Context(W, H, bpc, max_batch=2 * F, timing=True, moments=args.moments,
                      motion_v2=args.motion_v2)
    geo = ctx.geometry()
    chunks = ctx.plan_chunks(F)
    clip_dev = ctx.prepare_clip(ref, dist)
    warm = []
    for _ in range(args.warmup):
        ctx.submit_prepared(clip_dev)
        ctx.collect(F)
        warm.append(ctx.kernel_time_ms())
    torch.cuda.synchronize()
    ctx.kernel_stats(reset=True)
    series = []
    t0 = time.perf_counter()
    ctx.submit_prepared(clip_dev)
    for _ in range(args.steps - 1):
        ctx.submit_prepared(clip_dev)
        ctx.collect(F)
        series.append(ctx.kernel_time_ms())
    ctx.collect(F)
    series.append(ctx.kernel_time_ms())
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    launches, total_ms = ctx.kernel_stats()
    assert launches == args.steps == len(series), (launches, args.steps, len(series))
    ms_step = 1000.0 * elapsed / args.steps
    frames_per_s = F * args.steps / elapsed
    kernel_ms = total_ms / launches
    alg = algorithmic_bytes(W, H, bpc, F, args.motion_v2)
    achieved = alg / (kernel_ms * 1e-3) / 1e9
    dist_us = launch_distribution(series, warm)
    log(f"kernel {kernel_ms * 1e3:.1f} us/launch (mean of {launches}; median "
        f"{dist_us['median']:.1f}, min {dist_us['min']:.1f}, max {dist_us['max']:.1f}), "
        f"step {ms_step * 1e3:.1f} us, {achieved:.0f} GB/s")

    out = {
        "metric": "frames/s at 3840x2160 4:2:0 motion+PSNR; achieved HBM GB/s vs peak",
        "value": frames_per_s,
        "unit": "frames/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u8" if bpc == 8 else "u16",
        "data": "synthetic (seeded value-noise clip of the workload's shape; see synth.py)",
        "config": {"workload": describe(args.workload, args.moments, args.motion_v2),
                   "width": W, "height": H, "bpc": bpc,
                   "frames_per_step": F, "chroma": "4:2:0", "tiles": geo["tiles"],
                   "time_chunks": chunks, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": load_traffic(wl),
                     "kernel": "frames_kernel", "kernel_us": kernel_ms * 1e3,
                     "algorithmic_bytes_per_launch": alg,
                     "frac_of_median_launch": alg / (dist_us["median"] * 1e-6) / 1e9
                     / HBM_PEAK_GBS},
        "launch_us": dist_us,
        "upload": upload,
    }
    if not args.no_probe:
        ceil = ceilings if ceilings is not None else measure_ceilings(dev)
        out["ceilings_GBps"] = ceil
        out["roofline"]["frac_of_read_ceiling"] = achieved / ceil["read"]
    ctx.close()
    if not args.no_streaming:
        log("streaming submissions")
        out["streaming"] = streaming(ref, dist, clip, args.moments, args.motion_v2)
    if not args.no_cpu:
        log("cpu baseline")
        out["cpu_baseline"] = cpu_baseline(clip, moments=args.moments, motion_v2=args.motion_v2)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
