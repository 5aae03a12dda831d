#!/usr/bin/env python3
"""Benchmark of the hero-fusion library on one MI355X.

Workload (one "step"): the transpose fusion pair
  * out = transpose(exp(x), {1,0}), x f32[4096,4096] ~ N(0,1), row-major in/out;
  * out = transpose(x, {0,2,1}),    x bf16[64,512,1024] ~ N(0,1), row-major in/out;
each executed once, through the C ABI, on torch's current stream.

Inputs are generated on the host (seeded), copied to HBM before timing, and
rotated over several buffer sets so that no launch finds its operands in the
256 MB Infinity Cache left there by the previous launch.  The timed region
is bracketed by torch.cuda.synchronize(); inside it the launches of each
fusion run back to back between one pair of HIP events on the launch stream,
which gives each kernel's average launch time.

Prints ONE JSON line (metric, value in GB/s of algorithmic bytes, roofline
of the dominant kernel, the oracle's CPU baseline).  Per-config hero numbers
for the other workloads go into "heroes" (and to stderr).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
MALL_BYTES = 256 << 20


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def device_params(params):
    import numpy as np
    import torch
    out = []
    for p in params:
        b = p.view(np.int16) if p.dtype == np.uint16 else p
        out.append(torch.from_numpy(np.ascontiguousarray(b)).cuda())
    return out


class Case:
    """One compiled fusion with rotating resident buffer sets."""

    def __init__(self, make, args=(), kwargs=None, sets=None, transform=None):
        import torch
        import compiler_hlo_amd as H
        self.spec, self.params, self.meta = make(*args, **(kwargs or {}))
        if transform:
            self.params = transform(self.params)
        self.fusion = H.Fusion(self.spec.nodes)
        self.plan = self.fusion.plan()
        # one workspace: every launch of the case runs on one stream
        self.ws = torch.empty(max(1, self.plan["workspace_bytes"]), dtype=torch.uint8, device="cuda")
        self.bytes = self.plan["algorithmic_bytes"]
        work = self.bytes
        if sets is None:
            sets = max(2, min(64, math.ceil(3 * MALL_BYTES / max(work, 1))))
        self.sets = []
        base = device_params(self.params)
        ws_ptr = self.ws.data_ptr() if self.plan["workspace_bytes"] else 0
        self.launches = []
        for s in range(sets):
            ins = base if s == 0 else [t.clone() for t in base]
            out = self.fusion(*ins, workspace=self.ws)
            self.sets.append((ins, out))
            # the argument array of each set is built once: the timed loop
            # only calls hf_fusion_launch
            self.launches.append(self.fusion.prepare([t.data_ptr() for t in ins], out.data_ptr(), ws_ptr))
        torch.cuda.synchronize()
        self.k = 0

    def launch(self, stream):
        self.launches[self.k % len(self.launches)](stream.cuda_stream)
        self.k += 1


def copy_case(dtype, dims):
    """A fusion whose root is its parameter: a plain copy of known size (the
    calibration kernel for the HBM counters)."""
    import numpy as np
    import workloads as W

    def make():
        spec = W.Spec()
        spec.parameter(0, dtype, dims)
        n = W.numel(dims)
        g = W.rng(99)
        if dtype == "f32":
            x = W.normal_f32(g, n)
        elif dtype == "s8":
            x = W.integers(g, n, -128, 127, np.int8)
        elif dtype == "s4":
            x = W.integers(g, (n + 1) // 2, 0, 255, np.uint8)
        else:
            x = W.normal_bf16(g, n)
        name = "copy_%s_%s" % (dtype, "x".join(map(str, dims)))
        nbytes = (n + 1) // 2 if dtype == "s4" else n * W.nbytes_of(dtype)
        return spec, [x], {"name": name, "elements": n, "bytes": 2 * nbytes}
    return make


def iota_case(n):
    """iota s32[n] with no parameters: a kernel that only writes 4n bytes
    (n = 1: one workgroup; n = 262144: 1024 workgroups), for the per-launch
    floor."""
    import workloads as W

    def make():
        spec = W.Spec()
        spec.iota(0, "s32", [n])
        return spec, [], {"name": "iota_s32_%d" % n, "elements": n, "bytes": 4 * n}
    return make


def workload_makers():
    """Every named workload: (maker, kwargs, params transform)."""
    import workloads as W
    return {
        "transpose_exp_f32": (W.transpose_exp_f32, {}, None),
        "transpose_bf16_021": (W.transpose_bf16_021, {}, None),
        "row_reduce_exp_add_bf16": (W.row_reduce_exp_add_bf16, {}, None),
        "column_reduce_max_f32": (W.column_reduce_max_f32, {}, None),
        "column_reduce_max_f32_colmajor": (W.column_reduce_max_f32, {"m2m": (0, 1)},
                                           lambda ps: [ps[0].reshape(16384, 4096).T.copy().ravel()]),
        "quant_dequant_bias_requant": (W.quant_dequant_bias_requant, {}, None),
        "quant_dequant_bias_requant_s4": (W.quant_dequant_bias_requant_s4, {}, None),
        "loop_log_transpose_add": (W.loop_log_transpose_add, {}, None),
        "gelu_bf16": (W.gelu_bf16, {}, None),
        "transpose3d_exp_abs": (W.transpose3d_exp_abs, {}, None),
        "pad_reverse_concat_f32": (W.pad_reverse_concat_f32, {}, None),
        "pad_reverse_concat_minor_f32": (W.pad_reverse_concat_minor_f32, {}, None),
        "quantized_add_i8": (W.quantized_add_i8, {}, None),
        "row_mean_f32": (W.row_mean_f32, {}, None),
        "argmax_rows_bf16": (W.argmax_rows_bf16, {}, None),
        "copy_f32_4096x4096": (copy_case("f32", [4096, 4096]), {}, None),
        "copy_bf16_64x512x1024": (copy_case("bf16", [64, 512, 1024]), {}, None),
        "copy_f32_4250x128": (copy_case("f32", [4250, 128]), {}, None),
        "copy_s8_4096x4096": (copy_case("s8", [4096, 4096]), {}, None),
        "copy_s4_4096x4096": (copy_case("s4", [4096, 4096]), {}, None),
        "copy_s8_8192x8192": (copy_case("s8", [8192, 8192]), {}, None),
        "copy_s8_16384x32768": (copy_case("s8", [16384, 32768]), {}, None),
        "iota_s32_1": (iota_case(1), {}, None),
        "iota_s32_262144": (iota_case(262144), {}, None),
    }


def read_pmc_csv(run_dir, counter):
    """Mean value of `counter` per dispatch for each hf_* kernel in a rocprofv3
    --pmc run written with --output-format csv."""
    import csv
    import glob
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit("no counter_collection.csv under %s" % run_dir)
    per = {}
    for f in files:
        for r in csv.DictReader(open(f)):
            name = r.get("Kernel_Name", "")
            if r.get("Counter_Name") != counter or not name.startswith("hf_"):
                continue
            per.setdefault(name, []).append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in per.items()}


def read_kernel_stats(path):
    """{kernel name: average ns} from a rocprofv3 --kernel-trace --stats
    *_kernel_stats.csv."""
    import csv
    return {r["Name"]: float(r["AverageNs"]) for r in csv.DictReader(open(path))}


def kernel_name_of(source: str) -> str:
    for line in source.splitlines():
        if line.startswith("#define HF_KERNEL_NAME "):
            return line.split()[2]
    raise ValueError("no kernel name in the generated source")


def write_traffic(pmc_root, names, stats_csv=None):
    """Turn rocprofv3 runs into profiles/traffic.json.

    Expects <pmc_root>/<workload>/<COUNTER>/ for COUNTER in FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch), including the f32 copy.  Each counter is
    scaled by the ratio that makes the copy's reading equal its known bytes
    (read 4n, write 4n); a launch's traffic sums its kernels (a column reduce
    with segments has a fold kernel too).  With stats_csv (the
    *_kernel_stats.csv of a --kernel-trace --stats run of this bench), each
    record also gets the kernel-trace average of its kernels per launch."""
    import compiler_hlo_amd as H
    makers = workload_makers()
    stats = read_kernel_stats(stats_csv) if stats_csv else {}
    cal = {}
    for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
        got = read_pmc_csv(os.path.join(pmc_root, "copy_f32_4096x4096", ctr), ctr)
        kib = sum(got.values())
        cal[ctr] = (4 * 4096 * 4096) / (kib * 1024.0)
    out = {"_calibration": {"kernel": "copy f32[4096,4096] (read 64 MiB, write 64 MiB)",
                            "fetch_factor": round(cal["FETCH_SIZE"], 5),
                            "write_factor": round(cal["WRITE_SIZE"], 5)}}
    for name in names:
        mk, kw, tr = makers[name]
        spec, _, _ = mk(**kw)
        f = H.Fusion(spec.nodes, mode="compile")
        rec = {"source_fnv1a": fnv1a(f.source()), "algorithmic_bytes": f.plan()["algorithmic_bytes"]}
        total = 0.0
        for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
            got = read_pmc_csv(os.path.join(pmc_root, name, ctr), ctr)
            kib = sum(got.values())
            rec[ctr + "_KiB"] = round(kib, 1)
            b = kib * 1024.0 * cal[ctr]
            rec[ctr.split("_")[0].lower() + "_bytes"] = round(b)
            total += b
        rec["bytes_per_launch"] = round(total)
        rec["traffic_over_algorithmic"] = round(total / rec["algorithmic_bytes"], 4)
        kname = kernel_name_of(f.source())
        mine = [v for k, v in stats.items() if k == kname or k == kname + "_fold"]
        if mine:
            rec["kernel"] = kname
            rec["trace_avg_us"] = round(sum(mine) / 1e3, 3)
        out[name] = rec
        log("%-32s fetch %.1f MB write %.1f MB  x%.3f of algorithmic" % (
            name, rec["fetch_bytes"] / 1e6, rec["write_bytes"] / 1e6, rec["traffic_over_algorithmic"]))
    path = os.path.join(ROOT, "profiles", "traffic.json")
    json.dump(out, open(path, "w"), indent=1, sort_keys=True)
    log("wrote", path)


SETTLE_SECONDS = 0.25


def settle(cases, seconds=SETTLE_SECONDS):
    """Run the cases, untimed, for `seconds` of wall time.  After an idle gap
    (a kernel compile, a host-side step) the GPU's clocks take a few tens of
    milliseconds of load to return to their sustained level: measured on the
    row sum of exp(x) + bias over bf16[8,1,1280,16384], the first ~25 ms of
    launches ran 10-30% slower.  A timing that starts cold
    measures that ramp instead of the kernel."""
    import torch
    stream = torch.cuda.current_stream()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            for c in cases:
                c.launch(stream)
        torch.cuda.synchronize()


def time_cases(cases, steps, warmup):
    """Time `steps` steps; a step launches every case once.  Before the
    `warmup` steps the cases run for SETTLE_SECONDS (see settle).  Inside the
    timed region the launches are grouped by case (all of case 0, then all of
    case 1, ...) with one HIP event pair around each group on the launch
    stream, so the per-case average launch time carries no per-launch event
    overhead.  Returns (wall seconds per step, [mean seconds per launch of
    each case])."""
    import torch
    stream = torch.cuda.current_stream()
    settle(cases)
    for _ in range(warmup):
        for c in cases:
            c.launch(stream)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(len(cases) + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    evs[0].record(stream)
    for i, c in enumerate(cases):
        for _ in range(steps):
            c.launch(stream)
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    per = [evs[i].elapsed_time(evs[i + 1]) / steps / 1e3 for i in range(len(cases))]
    return wall, per


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(makers, min_seconds=10.0):
    """The oracle, as it stands, single-threaded, on the full workload of one
    step, repeated until at least `min_seconds` of CPU work (a few steps).
    Only evaluation is timed.  The calling thread is pinned to one core (the
    first this process may use) for the measurement and unpinned after."""
    import oracle
    cases = [make() for make in makers]
    allowed = os.sched_getaffinity(0)
    core = min(allowed)
    os.sched_setaffinity(0, {core})
    try:
        total_bytes, total_t, reps = 0, 0.0, 0
        while total_t < min_seconds or reps == 0:
            for spec, params, meta in cases:
                t0 = time.perf_counter()
                oracle.evaluate(spec.nodes, params)
                total_t += time.perf_counter() - t0
                total_bytes += meta["bytes"]
            reps += 1
    finally:
        os.sched_setaffinity(0, allowed)
    return {"value": round(total_bytes / total_t / 1e9, 4), "unit": "GB/s", "cores": 1,
            "kind": "oracle", "cpu_model": cpu_model(), "host_cores": os.cpu_count(),
            "pinned_core": core,
            "sample": "%d full steps (exp-transpose f32[4096,4096] + transpose bf16[64,512,1024]); "
                      "%.1f s on 1 thread pinned to core %d of %d" % (reps, total_t, core, os.cpu_count())}


def load_profile(name, source_hash):
    """The rocprofv3 record of a workload in profiles/traffic.json (HBM
    traffic per launch from FETCH_SIZE and WRITE_SIZE, the kernel-trace
    average), kept with the hash of the kernel source it was taken on; {}
    once the kernel has changed."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        t = json.load(open(path))[name]
    except Exception:
        return {}
    return t if t.get("source_fnv1a") == source_hash else {}


def load_traffic(name, source_hash):
    """HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, calibrated), or None."""
    return load_profile(name, source_hash).get("bytes_per_launch")


# The configurations the 70% gate applies to, by workload.
GATED = {"C2a": "transpose_exp_f32", "C2b": "transpose_bf16_021", "C3": "row_reduce_exp_add_bf16",
         "C4r": "column_reduce_max_f32", "C5": "quant_dequant_bias_requant"}


def roofline_entry(case_name, hero, nbytes, seconds, source_hash):
    """The HBM roofline of one workload's launch: algorithmic bytes over the
    events time per launch, against 8 TB/s, with the rocprofv3 kernel time and
    traffic of the same kernel source when profiles/traffic.json has them."""
    prof = load_profile(case_name, source_hash)
    achieved = nbytes / seconds / 1e9
    traffic = prof.get("bytes_per_launch")
    return {"workload": case_name, "hero": hero, "bound": "hbm", "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
            "algorithmic_bytes": nbytes, "avg_launch_us": round(seconds * 1e6, 3),
            "trace_avg_us": prof.get("trace_avg_us"), "traffic": traffic,
            "traffic_ratio": round(traffic / nbytes, 4) if traffic else None}


def fnv1a(s: str) -> str:
    h = 1469598103934665603
    for c in s.encode():
        h ^= c
        h = (h * 1099511628211) & 0xFFFFFFFFFFFFFFFF
    return "%016x" % h


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-heroes", action="store_true", help="skip the per-config hero table")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--only", default=None, help="time one named workload alone (profiling)")
    ap.add_argument("--traffic", default=None, metavar="PMC_DIR",
                    help="write profiles/traffic.json from rocprofv3 --pmc runs under PMC_DIR (no GPU)")
    ap.add_argument("--stats", default=None, metavar="CSV",
                    help="with --traffic: the *_kernel_stats.csv of a --kernel-trace --stats run of this bench")
    a = ap.parse_args()
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build runs on one GPU only (the fusion is a single-device hot path); "
              "--gpus %d is not supported" % a.gpus, file=sys.stderr)
        sys.exit(2)
    if a.traffic:
        write_traffic(a.traffic, [n for n in workload_makers() if not n.startswith(("copy_", "iota_"))], a.stats)
        return

    import torch
    assert torch.cuda.is_available(), "bench.py needs the GPU"
    torch.cuda.set_device(0)

    if a.only:
        mk, kw, tr = workload_makers()[a.only]
        c = Case(mk, kwargs=kw, transform=tr)
        wall, per = time_cases([c], a.steps, a.warmup)
        log("%s: %.2f us/launch (events), %.1f GB/s" % (a.only, per[0] * 1e6, c.bytes / per[0] / 1e9))
        return

    import workloads as W
    log("building workloads ...")
    c2a = Case(W.transpose_exp_f32)
    c2b = Case(W.transpose_bf16_021)
    cases = [c2a, c2b]
    wall, per = time_cases(cases, a.steps, a.warmup)
    step_bytes = c2a.bytes + c2b.bytes
    value = step_bytes / wall / 1e9
    dom = max(range(2), key=lambda i: per[i])
    dc = cases[dom]
    achieved = dc.bytes / per[dom] / 1e9
    name = dc.meta["name"]
    traffic = load_traffic(name, fnv1a(dc.fusion.source()))
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic,
            "kernel": name, "algorithmic_bytes": dc.bytes,
            "avg_launch_us": round(per[dom] * 1e6, 3),
            "trace_avg_us": load_profile(name, fnv1a(dc.fusion.source())).get("trace_avg_us")}
    rooflines = {}
    for i, c in enumerate(cases):
        for cfg, wl in GATED.items():
            if wl == c.meta["name"]:
                rooflines[cfg] = roofline_entry(wl, c.plan["hero"], c.bytes, per[i], fnv1a(c.fusion.source()))
    log("step: %.2f us wall; %s %.2f us (%.1f GB/s), %s %.2f us (%.1f GB/s)" % (
        wall * 1e6, c2a.meta["name"], per[0] * 1e6, c2a.bytes / per[0] / 1e9,
        c2b.meta["name"], per[1] * 1e6, c2b.bytes / per[1] / 1e9))

    sets_used = {c.meta["name"]: len(c.sets) for c in cases}
    heroes = {}
    for i, c in enumerate(cases):
        heroes[c.meta["name"]] = {
            "hero": c.plan["hero"], "us": round(per[i] * 1e6, 3),
            "GBps": round(c.bytes / per[i] / 1e9, 1), "frac": round(c.bytes / per[i] / 1e9 / PEAK_HBM_GBS, 4),
            "elements_per_s": float("%.4g" % (c.plan["elements"] / per[i])),
            "traffic": load_traffic(c.meta["name"], fnv1a(c.fusion.source()))}
    del cases, c2a, c2b
    torch.cuda.empty_cache()
    if not a.no_heroes:
        makers = workload_makers()
        others = ["copy_f32_4096x4096", "copy_bf16_64x512x1024", "loop_log_transpose_add",
                  "row_reduce_exp_add_bf16", "column_reduce_max_f32", "column_reduce_max_f32_colmajor",
                  "quant_dequant_bias_requant", "quant_dequant_bias_requant_s4", "gelu_bf16",
                  "transpose3d_exp_abs", "pad_reverse_concat_f32", "pad_reverse_concat_minor_f32",
                  "quantized_add_i8", "row_mean_f32", "argmax_rows_bf16"]
        for key in others:
            mk, kw, tr = makers[key]
            c = Case(mk, kwargs=kw, transform=tr)
            _, p = time_cases([c], 100, 10)
            for cfg, wl in GATED.items():
                if wl == key:
                    rooflines[cfg] = roofline_entry(wl, c.plan["hero"], c.bytes, p[0], fnv1a(c.fusion.source()))
            heroes[key] = {"hero": c.plan["hero"], "us": round(p[0] * 1e6, 3),
                           "GBps": round(c.bytes / p[0] / 1e9, 1),
                           "frac": round(c.bytes / p[0] / 1e9 / PEAK_HBM_GBS, 4),
                           "elements_per_s": float("%.4g" % (c.plan["elements"] / p[0])),
                           "traffic": load_traffic(key, fnv1a(c.fusion.source()))}
            log("%-32s %-13s %9.2f us %8.1f GB/s  %5.1f%% of peak" % (
                key, c.plan["hero"], p[0] * 1e6, c.bytes / p[0] / 1e9, 100 * c.bytes / p[0] / 1e9 / PEAK_HBM_GBS))
            del c
            torch.cuda.empty_cache()

    cpu = None
    if not a.no_cpu:
        cpu = cpu_baseline([W.transpose_exp_f32, W.transpose_bf16_021])

    line = {
        "metric": "achieved HBM GB/s (% of MI355X peak) per fusion hero; elements/s",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": round(wall * 1e3, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "transpose fusion: transpose(exp(x),{1,0}) f32[4096,4096] + "
                               "transpose(x,{0,2,1}) bf16[64,512,1024], row-major in and out",
                   "step_bytes": step_bytes, "buffer_sets": sets_used},
        "roofline": roof,
        "rooflines": {k: rooflines[k] for k in GATED if k in rooflines},
        "cpu_baseline": cpu,
        "heroes": heroes,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
