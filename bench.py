#!/usr/bin/env python
"""Throughput of the sharded mixed-precision AdamW step on one MI355X.

A step is one zf_shard_step over one batch of N resident replica gradients
(reduce-scatter sums, overflow/norm/clip, fused AdamW + cast + gather), plus
the per-unit gathers for a ZeRO-3 workload.  Under ZeRO-Offload a step is the
GPU reduction, the download of the sums, CPU-Adam on the host state and the
chunked upload of the 16-bit parameters.  For a workload with gradient
accumulation, a step is first the backward-side reduction of its
micro-batches (every bucket's reduce-scatter, accumulated into the fp32
gradient shards), then the step on the reduced shards.  Inputs are seeded synthetic
data generated on the device before the timed region; every step reuses the
same batch (the state evolves).

Prints one JSON line:
  value        algorithmic GB/s = (2N + 26) B per parameter (+ 4 for the
               ZeRO-3 unit gathers; FSDP2, backward-side and offload terms in
               algorithmic_bytes_per_param) x Psi / step time; pct_hbm_peak
               is value over 8 TB/s
  dtype        the arithmetic type (f32; the norm accumulates in f64); the
               gradient, parameter and state formats are in config
  roofline     the dominant kernel (the fused update pass, or the bucket
               launches when they move more): its algorithmic bytes per
               launch (the update pass: 26 B per parameter -- fp32 master,
               m, v in and out and the 16-bit parameter out) over its mean
               duration from HIP events recorded around it on its stream,
               against 8 TB/s.  Beside it the bytes the kernel really moves
               (design bytes: + the re-read of the replicas or of the fp32
               sums that the global-norm barrier costs), the same less the
               sums the memory-side cache window serves, and traffic =
               counted bytes per launch from the committed counter summaries
               of the same kernel code (null otherwise), and traffic_dram32 =
               the bytes of L2's 32-byte-unit requests to memory per launch
               (no calibration)
  hbm_gbs_counted
               counter bytes of every kernel of a step (bytes leaving L2)
               less the cache window's reads, over the step time; the raw
               counter figure is l2_egress_gbs_counted
  headline_2   with the default workload (73M, N = 8), the same figures for
               the second configuration the metric is quoted on (4.06B,
               N = 2), timed the same way in the same run
  graph_replay the same K steps replayed from a HIP graph of --graph-steps
               captured steps
  cpu_baseline the single-threaded CPU oracle on the whole default workload
               (a bounded slice of larger ones; rank 0, one GPU only)
--roctx adds named host ranges for rocprofv3 --marker-trace.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, vendor figure
DEFAULT_WORKLOAD = "llama-73m-n8"


def formats(w):
    """The workload's storage formats.  The path computes in binary32 (the
    reduce-scatter sums and AdamW), with the squared norm accumulated in
    binary64; gradients and parameters are stored in 16 bits."""
    from fsdp_sharded_mixed_amd import workloads as W
    name = {W.BF16: "bf16", W.F16: "f16"}
    return {"grad_dtype": name[w.grad_dtype],
            "param_dtype": "f32" if w.fp32_params else name[w.param_dtype],
            "state_dtype": "f32", "norm_accumulate": "f64"}


def backward_bytes_per_param(w):
    """Bytes of the backward-side reduction per parameter per step, over its
    n_micro micro-batches (A): every micro-batch reads the N 16-bit replicas
    and writes the fp32 shard, reading it back from the second one on; or,
    no_sync, every replica's fp32 main_grad is written (and read back from
    the second micro-batch on), then the N main_grads are read once and the
    shard written."""
    a, n = w.n_micro, w.n_ranks
    if w.accum_mode == 0:
        return a * 2 * n + (a - 1) * 4 + a * 4
    return a * 2 * n + (a - 1) * 4 * n + a * 4 * n + 4 * n + 4


def algorithmic_bytes_per_param(w):
    """Bytes the method itself moves per real parameter per applied step:
    read N 16-bit replicas, read and write fp32 master/m/v, write the 16-bit
    param; ZeRO-3 adds the unit gather (read 2 + write 2).  With the
    backward-side reduction: its bytes (backward_bytes_per_param), then the
    step reads the fp32 shard twice (norm pass, update pass)."""
    if w.backward_rs:
        b = backward_bytes_per_param(w) + 4 + 4 + 12 + 12
        if w.fp32_params:
            return b + 4 + 2
        return b + 2 + (4 if w.stage == 3 else 0)
    if w.fp32_params:
        # FSDP2: replicas in, fp32 grad shard out and back in, fp32 state in
        # and out, then each unit gather reads fp32 and writes 16-bit
        return 2 * w.n_ranks + 4 + 4 + 12 + 12 + 4 + 2
    b = 2 * w.n_ranks + 12 + 12 + 2
    if w.stage == 3:
        b += 4
    return b


def update_alg_bytes_per_param(w):
    """The method's own bytes in the fused update pass per real parameter:
    fp32 master, m and v read and written (24) and the 16-bit parameter
    written (2; none under FSDP2, whose fp32 shard is the parameter).
    When the method itself hands the update a reduced fp32 gradient shard
    (FSDP2's resident gradient shard, or the shard the backward-side
    reduction accumulated), reading it is the method's too (4).  Re-reading
    the replicas, or the fp32 sums pass 1 wrote, to get past the global-norm
    barrier is not: those are the design's bytes
    (update_kernel_bytes_per_elem)."""
    b = 24 + (0 if w.fp32_params else 2)
    if w.fp32_params or w.backward_rs:
        b += 4
    return b


def update_kernel_bytes_per_elem(w, materialized):
    """The fused update pass per (padded) element: the reduced gradient (fp32
    sums, or the N replicas again), fp32 master/m/v in and out, and the
    16-bit parameter out unless the parameters are fp32 (FSDP2)."""
    return (4 if materialized else 2 * w.n_ranks) + 12 + 12 + (0 if w.fp32_params else 2)


def backward_kernel_bytes_per_elem(w):
    """The backward-side launches of one step per (padded) element: the same
    terms as backward_bytes_per_param."""
    return backward_bytes_per_param(w)


PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = [os.path.join(ROOT, "fsdp_sharded_mixed_amd", "csrc", f)
                  for f in ("zf_step.hip", "zf_backward.hip", "zf_gather.hip", "zf_device.h",
                            "zf_internal.h", "zf_plan.cpp")]
COPY_BYTES = 1 << 30  # calibration copy: 1 GiB read + 1 GiB written


def kernel_source_hash():
    """Fingerprint of the step library's code (kernels, tiling, planner):
    the sources with comments removed and whitespace collapsed, so that a
    comment does not invalidate measured counters but any code change does."""
    import hashlib
    import re
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        with open(path) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def traffic_for(workload, kernel="zf_pass2", per="launch"):
    """Measured HBM bytes of one of the step's kernels (per launch, or summed
    over one step's launches) from the committed rocprofv3 counter summary
    (FETCH_SIZE + WRITE_SIZE, each scaled by the same counter's reading for a
    1 GiB copy), or None if there is none or the kernel sources have changed
    since it was taken."""
    path = os.path.join(PROFILES, f"zf_step_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("kernel_source_sha256_16") != kernel_source_hash() or kernel not in d:
        return None
    return d[kernel]["hbm_bytes_per_" + per]


def counted_bytes_per_step(w):
    """HBM bytes per step of every kernel of the step, from the committed
    counter summary of these kernel sources, or None."""
    path = os.path.join(PROFILES, f"zf_step_{w.name}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return sum(v["hbm_bytes_per_step"] for v in d.values()
               if isinstance(v, dict) and "hbm_bytes_per_step" in v)


def skipped_step_ms(w, dev, one_step, reps=3):
    """Median time of a step whose gradients hold a +inf (the step is
    skipped: pass 1, the reduction and the finish run, the update exits).
    Runs after the timed region; the state is left as it was except the
    dynamic loss scale, which halves per skipped step."""
    import torch
    grads = dev.micro_grads[0][0]
    p = dev.plan.units[0].O  # a real element of the first unit
    keep = grads[p].clone()
    grads[p] = float("inf")
    times = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        one_step()
        e1.record()
        torch.cuda.synchronize()
        assert dev.result().skipped == 1
        times.append(e0.elapsed_time(e1))
    grads[p] = keep
    torch.cuda.synchronize()
    return round(sorted(times)[len(times) // 2], 5)


def backward_traffic(w):
    """Measured HBM bytes of one step's backward-side launches, or None."""
    parts = [traffic_for(w.name, k, "step") for k in
             (("zf_bucket_rs_kernel",) if w.accum_mode == 0 else
              ("zf_bucket_rs_kernel", "zf_accumulate_kernel"))]
    return None if any(p is None for p in parts) else sum(parts)


def _csv_rows(directory, suffix):
    import csv
    import glob
    files = sorted(glob.glob(os.path.join(directory, "**", "*" + suffix), recursive=True))
    if not files:
        raise SystemExit(f"no *{suffix} under {directory}")
    with open(files[0]) as f:
        return list(csv.DictReader(f))


def summarize_trace(directory, out, command, bench_json=None):
    """Text summary of a rocprofv3 --kernel-trace --stats run (with the roctx
    ranges' host times when the run also had --marker-trace and --roctx),
    and, given the profiled run's stdout (bench_json), the figures of its
    bench line, whose HIP-event kernel times the trace should agree with."""
    rows = _csv_rows(directory, "kernel_stats.csv")
    lines = [f"command: {command}", "",
             f"{'kernel':<70} {'calls':>6} {'avg_us':>10} {'min_us':>10} {'max_us':>10} {'pct':>6}"]
    for r in rows:
        name = r["Name"].replace("(anonymous namespace)::", "")
        name = name if len(name) <= 70 else name[:67] + "..."
        lines.append(f"{name:<70} {int(r['Calls']):>6} {float(r['AverageNs']) / 1e3:>10.2f} "
                     f"{float(r['MinNs']) / 1e3:>10.2f} {float(r['MaxNs']) / 1e3:>10.2f} "
                     f"{float(r['Percentage']):>6.2f}")
    import glob
    # the update pass of a skipped step exits at once: its launches are
    # listed apart from the applied ones (a run with the skipped-step probe
    # has both under one kernel name)
    traces = glob.glob(os.path.join(directory, "**", "*kernel_trace.csv"), recursive=True)
    if traces:
        durs = {}
        with open(traces[0]) as f:
            import csv
            for r in csv.DictReader(f):
                if "zf_pass2" in r["Kernel_Name"]:
                    name = r["Kernel_Name"].replace("(anonymous namespace)::", "")
                    durs.setdefault(name, []).append(
                        (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        split = []
        for name, xs in sorted(durs.items()):
            med = sorted(xs)[len(xs) // 2]
            # an empty launch costs only the dispatch of its blocks: well
            # under half an applied one at every size
            full = [x for x in xs if x >= 0.5 * med]
            short = [x for x in xs if x < 0.5 * med]
            if short:
                split.append(f"{name[:70]:<70} applied {len(full):>4} x {sum(full) / len(full):>10.2f}"
                             f" us; exited at once (skipped steps) {len(short):>3} x "
                             f"{sum(short) / len(short):.2f} us")
        if split:
            lines += ["", "update-pass launches (kernel trace), applied and skipped:"] + split
    if glob.glob(os.path.join(directory, "**", "*marker_api_stats.csv"), recursive=True):
        lines += ["", "roctx ranges (host time from push to pop; the enqueue waits once the "
                      "launch queue is full, so it follows the device's pace):",
                  f"{'range':<70} {'calls':>6} {'avg_us':>10} {'min_us':>10} {'max_us':>10}"]
        for r in _csv_rows(directory, "marker_api_stats.csv"):
            lines.append(f"{r['Name']:<70} {int(r['Calls']):>6} "
                         f"{float(r['AverageNs']) / 1e3:>10.2f} {float(r['MinNs']) / 1e3:>10.2f} "
                         f"{float(r['MaxNs']) / 1e3:>10.2f}")
    if bench_json:
        with open(bench_json) as f:
            rows = [ln for ln in f if ln.startswith("{")]
        d = json.loads(rows[-1])

        def excerpt(d, label):
            roof = {k: d["roofline"].get(k) for k in
                    ("kernel", "achieved", "frac", "design_gbs", "frac_design_bytes",
                     "hbm_gbs_design_less_window", "hbm_frac_of_4r4w_probe",
                     "own_mix_probe", "frac_of_own_mix_probe", "traffic",
                     "traffic_dram32") if k in d["roofline"]}
            return [f"{label} (HIP events on the step's stream, ms):",
                    f"  kernels_ms: {json.dumps(d.get('kernels_ms', d.get('phases_ms')))}",
                    f"  roofline: {json.dumps(roof)}",
                    f"  ms_per_step: {d['ms_per_step']}  value (GB/s): {d['value']}  "
                    f"pct_hbm_peak: {d['pct_hbm_peak']}"]

        lines += [""] + excerpt(d, "bench line of the same profiled run")
        lines += [f"  stream_probe_gbs: {json.dumps(d.get('stream_probe_gbs'))}  "
                  f"device_copy_gbs: {d.get('device_copy_gbs')}"]
        if "headline_2" in d:
            lines += excerpt(d["headline_2"], f"its headline_2 ({d['headline_2']['workload']})")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_table(jsonl, out, command):
    """Markdown table of bench lines (one JSON line per workload, as the
    bench prints them) written to `out`."""
    with open(jsonl) as f:
        rows = [json.loads(ln) for ln in f if ln.startswith("{")]
    L = ["# bench.py on one MI355X: every workload (one GPU, one run)", "",
         f"command: `{command}`", "",
         "Columns: ms/step = K timed steps over K; algorithmic = the method's bytes per step "
         "(`algorithmic_bytes_per_param` x Psi) over the step time, and its share of 8 TB/s "
         "(`pct_hbm_peak`, the bench's headline figure); roofline frac = the dominant "
         "kernel's algorithmic bytes per launch over its mean duration (HIP events in the "
         "same run), over 8 TB/s; design frac = the same kernel's actual bytes (with the "
         "global-norm barrier's re-read) over 8 TB/s; HBM/probe = the update pass's actual "
         "bytes less the cache window's reads, per second, over the GPU's best "
         "4-read/4-write probe; own-mix probe = the time of a kernel that moves the update "
         "pass's 30 bytes per element with no arithmetic (its sums read from HBM) over the "
         "update pass's time, on equal element counts; counted HBM = FETCH_SIZE + "
         "WRITE_SIZE of every step kernel (committed summaries of the same code, each "
         "counter scaled by its reading for a 1 GiB copy) less the cache window's reads, per "
         "step time; L2 egress = the same without that subtraction; graph = the same K "
         "steps replayed from a HIP graph of 10 steps.", "",
         "| workload | ms/step | algorithmic GB/s (% of 8 TB/s) | params/s | roofline kernel | "
         "roofline frac (algorithmic) | design frac | HBM / 4+4 probe | own-mix probe | "
         "counted HBM GB/s (% of 8 TB/s) | L2 egress GB/s | skipped step ms | graph ms/step "
         "| probes 1+1 / 4+4 / 8+1 / update mix (replicas, sums) GB/s | phases (ms) |",
         "|" + "---|" * 15]
    for d in rows:
        r, p = d["roofline"], d.get("stream_probe_gbs", {})
        ph = d.get("kernels_ms") or d.get("phases_ms") or {}
        g = d.get("graph_replay", {}).get("ms_per_step", "—")
        counted = (f"{d['hbm_gbs_counted']:.0f} ({d['pct_hbm_peak_counted']:.1f}%)"
                   if "hbm_gbs_counted" in d else "—")
        probes = " / ".join(str(p.get(k, "—")) for k in
                            ("1r1w", "4r4w", "8r1w", "update_mix_replicas", "update_mix_sums"))
        L.append(f"| {d['config']['workload']} | {d['ms_per_step']:.4f} | {d['value']:.0f} "
                 f"({d['pct_hbm_peak']:.1f}%) | {d['params_updated_per_s']:.3g} | "
                 f"{r['kernel'].split(' (')[0]} | {r['frac']:.3f} | "
                 f"{r.get('frac_design_bytes', '—')} | {r.get('hbm_frac_of_4r4w_probe', '—')} | "
                 f"{r.get('frac_of_own_mix_probe', '—')} | {counted} | "
                 f"{d.get('l2_egress_gbs_counted', '—')} | {d.get('skipped_step_ms', '—')} | "
                 f"{g} | {probes} | " + ", ".join(f"{k} {v}" for k, v in ph.items()) + " |")
    for d in rows:
        if "cpu_baseline" in d:
            cb = d["cpu_baseline"]
            L += ["", f"CPU baseline ({d['config']['workload']}): {cb['value']} GB/s "
                      f"algorithmic, {cb['params_per_s']:.3g} params/s, {cb['s_per_step']} "
                      f"s/step, {cb['cores']} core(s): {cb['sample']}"]
    with open(out, "w") as f:
        f.write("\n".join(L) + "\n")
    print("\n".join(L))


def summarize_pmc(fetch_dir, write_dir, workload, out, commands):
    """Per-launch HBM traffic of the step's kernels from two counter runs,
    scaled by the counters' reading for the 1 GiB calibration copy."""
    from fsdp_sharded_mixed_amd import workloads as W

    def per_kernel(directory, counter):
        rows = _csv_rows(directory, "counter_collection.csv")
        vals = {}
        for r in rows:
            if r.get("Counter_Name") != counter:
                continue
            vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return vals

    def pick(vals, key):
        hits = [v for k, v in vals.items() if key in k]
        if not hits:
            raise SystemExit(f"no dispatch of {key}")
        xs = sorted(x for h in hits for x in h)
        return xs[len(xs) // 2]  # median over dispatches (KiB)

    def total(vals, key):
        xs = [x for k, v in vals.items() if key in k for x in v]
        return sum(xs), len(xs)

    fetch, write = per_kernel(fetch_dir, "FETCH_SIZE"), per_kernel(write_dir, "WRITE_SIZE")
    # the calibration copy: the bench's own 1-read/1-write probe kernel,
    # whose every dispatch reads and writes exactly PROBE_FLOATS * 4 bytes
    def median_of(vals, name):
        xs = sorted(vals[name])
        return xs[len(xs) // 2]

    copy_key = next(k for k in fetch if "stream_probe<1, 1>" in k)
    f_scale = 4 * PROBE_FLOATS / (median_of(fetch, copy_key) * 1024.0)
    w_scale = 4 * PROBE_FLOATS / (median_of(write, copy_key) * 1024.0)
    w = W.get(workload)
    res = {"workload": workload, "kernel_source_sha256_16": kernel_source_hash(),
           "calibration": {"kernel": copy_key, "bytes_each_way": 4 * PROBE_FLOATS,
                           "fetch_scale": f_scale, "write_scale": w_scale},
           "commands": commands}
    # one finish kernel per step: the step count of the run
    _, steps = total(fetch, "zf_finish")
    res["steps"] = steps
    keys = ("zf_pass1_reduced", "zf_pass1<", "zf_pass2", "zf_gather_kernel",
            "zf_gather_cast_kernel", "zf_bucket_rs_kernel", "zf_accumulate_kernel")
    for key in keys:
        try:
            fb = pick(fetch, key) * 1024.0 * f_scale
            wb = pick(write, key) * 1024.0 * w_scale
        except SystemExit:
            continue
        ft, nf = total(fetch, key)
        wt, _ = total(write, key)
        step_bytes = (ft * f_scale + wt * w_scale) * 1024.0 / max(steps, 1)
        res[key.rstrip("<")] = {
            "launches_per_step": nf / max(steps, 1), "fetch_bytes": fb, "write_bytes": wb,
            "hbm_bytes_per_launch": fb + wb, "hbm_bytes_per_step": step_bytes,
            "per_param_per_step": step_bytes / w.psi}
    with open(out, "w") as f:
        json.dump(res, f, indent=1)
    print(json.dumps(res, indent=1))


PROBE_FLOATS = 1 << 28  # 1 GiB per array

DRAM32_COUNTERS = ("TCC_EA0_RDREQ_DRAM_32B_sum", "TCC_EA0_WRREQ_WRITE_DRAM_32B_sum")


def summarize_dram32(directory, workload, out, command):
    """Per-launch bytes of the step's kernels from one counter run of L2's
    read and write requests to memory, counted in 32-byte units
    (DRAM32_COUNTERS: a 64-byte request counts 2, a 128-byte one 4), so
    bytes = 32 x count with no calibration; the run's 1 GiB probe copy is
    reported beside them as the check.  These requests are what leaves L2
    for memory: the memory-side cache may still serve some of them."""
    from fsdp_sharded_mixed_amd import workloads as W
    rows = _csv_rows(directory, "counter_collection.csv")
    vals = {}
    for r in rows:
        vals.setdefault((r["Kernel_Name"], r["Counter_Name"]), []).append(
            32.0 * float(r["Counter_Value"]))

    def med(key, counter):
        xs = sorted(x for (k, c), v in vals.items() if key in k and c == counter for x in v)
        return xs[len(xs) // 2] if xs else None

    def tot(key, counter):
        return sum(x for (k, c), v in vals.items() if key in k and c == counter for x in v)

    rd, wr = DRAM32_COUNTERS
    w = W.get(workload)
    steps = len([x for (k, c), v in vals.items() if "zf_finish" in k and c == rd for x in v])
    res = {"workload": workload, "kernel_source_sha256_16": kernel_source_hash(),
           "counters": list(DRAM32_COUNTERS), "bytes_per_count": 32, "commands": command,
           "steps": steps,
           "copy_check": {"kernel": "stream_probe<1, 1> (1 GiB read, 1 GiB written)",
                          "expected_bytes_each_way": 4 * PROBE_FLOATS,
                          "read_bytes": med("stream_probe<1, 1>", rd),
                          "write_bytes": med("stream_probe<1, 1>", wr)}}
    for key in ("zf_pass1_reduced", "zf_pass1<", "zf_pass2", "zf_gather_kernel",
                "zf_gather_cast_kernel", "zf_bucket_rs_kernel", "zf_accumulate_kernel"):
        r1, w1 = med(key, rd), med(key, wr)
        if r1 is None:
            continue
        step_bytes = (tot(key, rd) + tot(key, wr)) / max(steps, 1)
        res[key.rstrip("<")] = {"read_bytes": r1, "write_bytes": w1,
                                "bytes_per_launch": r1 + w1, "bytes_per_step": step_bytes,
                                "per_param_per_step": step_bytes / w.psi}
    with open(out, "w") as f:
        json.dump(res, f, indent=1)
    print(json.dumps(res, indent=1))


def dram32_for(workload, kernel="zf_pass2", per="launch"):
    """Bytes per launch (or per step) of a step kernel from the committed
    32-byte request counter summary of these kernel sources, or None."""
    path = os.path.join(PROFILES, f"zf_step_{workload}_dram32.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("kernel_source_sha256_16") != kernel_source_hash() or kernel not in d:
        return None
    return d[kernel]["bytes_per_" + per]


# probe shapes (quads per lane, resident blocks per CU, 0: no limit); the
# best one per access mix is this GPU's figure for that mix
PROBE_SHAPES = ((1, 0), (2, 0), (1, 3), (1, 4), (2, 3), (2, 4))


def stream_probes(reps=10):
    """GB/s of this GPU for streams in the step kernels' access pattern: a
    copy (1 read, 1 write), the update pass's mix of 4 reads and 4 writes,
    and 8 reads + 1 write (pass 1 at N = 8).  Each mix is timed with the
    fixed-shape zfi_stream_probe and with zfi_stream_probe_shaped in every
    PROBE_SHAPES shape; the best figure is reported, with its shape in
    out["shape"] ("fixed" or "q<quads>c<blocks per CU>")."""
    import torch
    from fsdp_sharded_mixed_amd import inputs as I
    bufs = [torch.ones(PROBE_FLOATS, dtype=torch.float32, device="cuda:0") for _ in range(9)]
    out, shape = {}, {}

    def gbs(run, moved):
        for _ in range(3):
            run()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            run()
        e1.record()
        torch.cuda.synchronize()
        return moved * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9

    for name, r, wr in (("1r1w", 1, 1), ("4r4w", 4, 4), ("8r1w", 8, 1)):
        src, dst = bufs[:r], bufs[r:r + wr]
        moved = (r + wr) * 4 * PROBE_FLOATS
        best, which = gbs(lambda: I.stream_probe(src, dst), moved), "fixed"
        for q, c in PROBE_SHAPES:
            g = gbs(lambda: I.stream_probe_shaped(src, dst, q, c), moved)
            if g > best:
                best, which = g, f"q{q}c{c}"
        out[name], shape[name] = round(best, 1), which
    # the update pass's own bytes (30 per element: two 16-bit replicas or
    # fp32 sums in, fp32 master/m/v in and out, the 16-bit parameter out)
    p, m, v, o = bufs[2], bufs[3], bufs[4], bufs[5]
    for name, g in (("update_mix_replicas", (bufs[0], bufs[1])), ("update_mix_sums", bufs[0])):
        best, which = 0.0, None
        for t, c in MIX_SHAPES:
            gb = gbs(lambda: I.update_mix_probe(g, p, m, v, o, PROBE_FLOATS, t, c),
                     UPDATE_MIX_BYTES * PROBE_FLOATS)
            if gb > best:
                best, which = gb, f"t{t}c{c}"
        out[name], shape[name] = round(best, 1), which
    del bufs
    torch.cuda.empty_cache()
    out["shape"] = shape
    return out


# the update-mix probe's shapes (threads per block, resident blocks per CU)
MIX_SHAPES = tuple((t, c) for t in (128, 256) for c in (0, 2, 3, 4, 6))
UPDATE_MIX_BYTES = 30


def own_mix_probe(w, materialized):
    """The stream_probes key whose bytes per element equal the update pass's
    (None where no probe has its mix: N = 3 or 4 recomputing, fp32 params)."""
    if w.fp32_params:
        return None
    if materialized or w.backward_rs:
        return "update_mix_sums"
    return "update_mix_replicas" if w.n_ranks == 2 else None


def apply_overrides(w, items):
    """Apply FIELD=VALUE overrides to a workload (typed like the field)."""
    done = {}
    for item in items:
        key, _, val = item.partition("=")
        if not hasattr(w, key) or key in ("segments", "extra"):
            raise SystemExit(f"bench.py: unknown workload field {key!r}")
        cur = getattr(w, key)
        if isinstance(cur, bool):
            new = val.lower() in ("1", "true", "yes")
        elif isinstance(cur, int) or cur is None and key in ("inject_step", "bucket_numel"):
            new = int(val)
        elif isinstance(cur, float):
            new = float(val)
        else:
            new = val
        setattr(w, key, new)
        done[key] = new
    if done:
        w.name = w.name + "+" + ",".join(f"{k}={v}" for k, v in done.items())
    return done


def host_info():
    """CPU model, logical CPUs and RAM of the host the oracle ran on."""
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    ram = None
    try:
        with open("/proc/meminfo") as f:
            for ln in f:
                if ln.startswith("MemTotal"):
                    ram = round(int(ln.split()[1]) / 2 ** 20, 1)
                    break
    except OSError:
        pass
    return {"cpu": model, "cpus": os.cpu_count(), "ram_gib": ram}


def _oracle_replicas(ws, units, psi_pad, step, scale, micro=0):
    """The N padded replicas of `step` from the oracle's own generator, as
    OI.replicas builds them, filled over all host threads (input
    generation, outside the timed region)."""
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor
    import oracle as O
    from fsdp_sharded_mixed_amd import workloads as W
    out = [np.zeros(psi_pad, np.uint16) for _ in range(ws.n_ranks)]
    piece = 1 << 22
    tasks = [(q, u, a) for q in range(ws.n_ranks) for u in units
             for a in range(0, int(u["L"]), piece)]

    def fill(t):
        q, u, a = t
        b = min(int(u["L"]), a + piece)
        o = int(u["O"])
        out[q][o + a:o + b] = O.gen16(b - a, ws.grad_dtype, ws.seed,
                                      W.grad_stream(step, q, micro), int(u["lam"]) + a,
                                      ws.sigma, scale)

    with ThreadPoolExecutor(os.cpu_count() or 1) as ex:
        list(ex.map(fill, tasks))
    return out


def cpu_baseline(w, min_seconds=10.0, max_steps=40, full_limit=150_000_000):
    """The CPU oracle as it stands, single-threaded on one pinned core.  On
    the whole workload when it has at most full_limit parameters (the
    default 73M workload: every parameter), else on its first segments up
    to ~19M parameters (for the larger Llama workloads: the embedding and
    the first decoder layers); same N, dtypes and hyperparameters, one
    resident batch, steps until min_seconds.  The inputs are generated
    before the timed region, over all host threads."""
    import oracle as O  # noqa: F401
    from fsdp_sharded_mixed_amd import workloads as W
    from tests import oracle_inputs as OI

    segs, tot = [], 0
    whole = w.psi <= full_limit
    for s in w.segments:
        segs.append(s)
        tot += s.numel
        if not whole and tot >= 18_000_000:
            break
    ws = W.Workload(**{**w.__dict__, "segments": segs})
    units, psi, psi_pad = OI.plan(ws)
    run = OI.OracleRun(ws, units, psi, psi_pad)
    if ws.backward_rs:
        grads = [_oracle_replicas(ws, units, psi_pad, 1, ws.loss_scale, micro=a)
                 for a in range(ws.n_micro)]
    else:
        grads = _oracle_replicas(ws, units, psi_pad, 1, ws.loss_scale)
    # one core, as the oracle is single-threaded by design
    try:
        saved = os.sched_getaffinity(0)
        os.sched_setaffinity(0, {min(saved)})
    except (AttributeError, OSError):
        saved = None
    try:
        steps, t0 = 0, time.perf_counter()
        while steps < max_steps and (time.perf_counter() - t0) < min_seconds:
            run.step(grads)
            steps += 1
        dt = time.perf_counter() - t0
    finally:
        if saved is not None:
            os.sched_setaffinity(0, saved)
    gbs = algorithmic_bytes_per_param(ws) * psi * steps / dt / 1e9
    what = (f"the whole {w.name} workload ({psi:,} params)" if whole else
            f"first {len(segs)} parameter tensors ({psi:,} params) of {w.name}")
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "host": host_info(),
            "params_per_s": round(psi * steps / dt, 1),
            "s_per_step": round(dt / steps, 4),
            "sample": f"{what}, N={ws.n_ranks}, {steps} steps over one batch"
                      + (f" of {ws.n_micro} micro-batches" if ws.backward_rs else "")
                      + f", {dt:.1f} s timed, single-threaded C oracle on one pinned core "
                        f"(input generation untimed)"}


def offload_line(args, w, dev, ms, wall, copy_gbs):
    """The bench line of a ZeRO-Offload workload: the step's wall time, its
    phases from the library's events (GPU reduction; the download of the
    sums; CPU-Adam with the chunked upload), and CPU-Adam alone on the same
    host arrays."""
    import torch
    from fsdp_sharded_mixed_amd import workloads as W, zf
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for row in evs:
        for e in row:
            e.record()
    torch.cuda.synchronize()
    for row in evs:
        dev.step(phase_events=[e.cuda_event for e in row])
    torch.cuda.synchronize()
    red = sum(r[0].elapsed_time(r[1]) for r in evs) / args.steps
    down = sum(r[1].elapsed_time(r[2]) for r in evs) / args.steps
    upd = sum(r[2].elapsed_time(r[3]) for r in evs) / args.steps
    res = dev.last_result
    assert res.skipped == 0
    # CPU-Adam alone over the whole padded flat, same threads
    n = dev.psi_pad
    reps = 3
    t0 = time.perf_counter()
    for _ in range(reps):
        zf.cpu_adam(dev.hp, dev.h_grad, dev.master, dev.exp_avg, dev.exp_avg_sq, res.gs,
                    res.bc1, res.bc2, params=dev.h_params, param_dtype=w.param_dtype,
                    n_threads=dev.n_threads,
                    grad_dtype=w.grad_dtype if w.offload_down16 else zf.F32)
    cpu_s = (time.perf_counter() - t0) / reps
    threads = dev.n_threads if dev.n_threads > 0 else (os.cpu_count() or 1)
    s = dev.plan.summary
    alg = algorithmic_bytes_per_param(w) * w.psi
    gbs = alg / (ms * 1e-3) / 1e9
    # pass 1 reads N 16-bit replicas and writes the sums: fp32, or rounded
    # to the gradient dtype for a 16-bit download
    p1_bytes = (2 * w.n_ranks + (2 if w.offload_down16 else 4)) * s.psi_pad
    p1_gbs = p1_bytes / (red * 1e-3) / 1e9
    return {
        "metric": "ZeRO step GB/s (algorithmic bytes) and % of HBM peak; params updated/s",
        "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded splitmix64/Irwin-Hall normal grads and master init, "
                "random-init weights)",
        "config": {"workload": w.name, "psi": w.psi, "psi_padded": s.psi_pad,
                   "virtual_ranks": w.n_ranks, "zero_stage": w.stage, **formats(w),
                   "offload": "fp32 state + CPU-Adam on the host, "
                              + ("16-bit" if w.offload_down16 else "fp32") + " sums down",
                   "cpu_adam_threads": threads, "pipeline_chunks": dev.n_chunks},
        "params_updated_per_s": round(w.psi / (ms * 1e-3), 1),
        "pct_hbm_peak": round(100 * gbs / PEAK_HBM_GBS, 2),
        "wall_ms_per_step": round(1e3 * wall / args.steps, 5),
        "device_copy_gbs": round(copy_gbs, 1),
        "phases_ms": {"gpu_reduce": round(red, 4), "download": round(down, 4),
                      "cpu_adam_and_upload": round(upd, 4)},
        "pcie_down_gbs": round((2 if w.offload_down16 else 4) * n / (down * 1e-3) / 1e9, 2),
        "cpu_adam": {"ms": round(cpu_s * 1e3, 3), "params_per_s": round(n / cpu_s, 1),
                     "host_gbs": round((28 if w.offload_down16 else 30) * n / cpu_s / 1e9, 2),
                     "threads": threads,
                     "host_cpus": os.cpu_count()},
        "roofline": {"bound": "hbm", "achieved": round(p1_gbs, 2), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(p1_gbs / PEAK_HBM_GBS, 4),
                     "traffic": traffic_for(w.name, "zf_pass1"),
                     "kernel": "zf_pass1 (reduce-scatter sums + norm partials, the offload "
                               "step's GPU kernel)", "bytes_per_launch": p1_bytes},
    }


HEADLINE_2 = "llama-4.06b-n2"


def bench_workload(w, args, probe, copy_gbs, graph=True, skip_probe=True):
    """Times one workload: K steps after W warm-up steps (the value), the
    same K steps again with the library's phase events (the per-kernel
    times and the roofline), optionally K steps replayed from a HIP graph,
    and skipped steps.  Returns (line, dev)."""
    import torch
    from fsdp_sharded_mixed_amd import runner, trace

    dev = runner.DeviceRun(w, device="cuda:0", resident_micro=True)
    dev.n_chunks, dev.n_threads = args.offload_chunks, args.offload_threads
    dev.init_state()
    if w.backward_rs:
        dev.fill_micro(1, w.loss_scale)
    else:
        dev.fill_grads(1, w.loss_scale)
    torch.cuda.synchronize()

    def one_step(phase_events=None, backward_event=None):
        if w.backward_rs:
            if backward_event is not None:
                backward_event.record()
            with trace.span("backward buckets"):
                dev.backward_all()
        with trace.span("step"):
            dev.step(phase_events=phase_events)
        with trace.span("gathers"):
            dev.gather_all()

    for _ in range(args.warmup):
        one_step()
    torch.cuda.synchronize()
    res = dev.result()
    assert res.skipped == 0, "warm-up step skipped"

    # timed region: exactly K steps
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for _ in range(args.steps):
        one_step()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = start.elapsed_time(end) / args.steps
    res = dev.result()
    assert res.skipped == 0

    if w.offload:
        line = offload_line(args, w, dev, ms, wall, copy_gbs)
        line["stream_probe_gbs"] = probe
        return line, dev

    # per-kernel durations: a second run of K steps with HIP events recorded
    # by the library between its kernels, on the step's stream
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    for row in evs:
        for e in row:
            e.record()
    torch.cuda.synchronize()
    for row in evs:
        one_step(phase_events=[e.cuda_event for e in row[1:5]], backward_event=row[0])
        row[5].record()  # after the unit gathers
    torch.cuda.synchronize()
    step_ms = [(r[0] if w.backward_rs else r[1]).elapsed_time(r[5]) for r in evs]
    per_step = sorted(step_ms)
    evs_b = [r[0] for r in evs]
    evs = [r[1:5] for r in evs]
    bw = (sum(b.elapsed_time(r[0]) for b, r in zip(evs_b, evs)) / args.steps
          if w.backward_rs else 0.0)
    p1 = sum(r[0].elapsed_time(r[1]) for r in evs) / args.steps
    fin = sum(r[1].elapsed_time(r[2]) for r in evs) / args.steps
    p2 = sum(r[2].elapsed_time(r[3]) for r in evs) / args.steps

    # the same K steps replayed from a HIP graph of G steps (the step only
    # enqueues kernels, so it captures whole; t and the loss scale advance on
    # the device from one replay to the next)
    graph_ms = None
    if graph:
        gsteps = args.graph_steps if args.steps % args.graph_steps == 0 else 1
        g = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for _ in range(gsteps):
                one_step()
        g.replay()
        torch.cuda.synchronize()
        start.record()
        for _ in range(args.steps // gsteps):
            g.replay()
        end.record()
        torch.cuda.synchronize()
        graph_ms = start.elapsed_time(end) / args.steps
        assert dev.result().skipped == 0
        del g

    s = dev.plan.summary
    materialized = s.policy != 0
    alg = algorithmic_bytes_per_param(w) * w.psi
    gbs = alg / (ms * 1e-3) / 1e9
    # sums that pass 1 leaves in the memory-side cache and the update pass
    # reads from there (not from HBM): the cached-sums window
    window = s.cached_sums_bytes if (materialized and not w.backward_rs) else 0
    upd_alg = update_alg_bytes_per_param(w) * w.psi
    upd_design = update_kernel_bytes_per_elem(w, materialized or w.backward_rs) * s.psi_pad
    upd_gbs = upd_alg / (p2 * 1e-3) / 1e9
    design_gbs = upd_design / (p2 * 1e-3) / 1e9
    hbm_gbs = (upd_design - window) / (p2 * 1e-3) / 1e9
    roof = {"bound": "hbm", "achieved": round(upd_gbs, 2), "peak": PEAK_HBM_GBS,
            "unit": "GB/s", "frac": round(upd_gbs / PEAK_HBM_GBS, 4),
            "traffic": traffic_for(w.name, "zf_pass2"),
            "traffic_dram32": dram32_for(w.name, "zf_pass2"),
            "kernel": "zf_pass2 (fused AdamW" + ("" if w.fp32_params else "+cast+gather") + ")",
            "bytes_per_launch": upd_alg,
            "bytes_basis": f"algorithmic: {update_alg_bytes_per_param(w)} B per parameter",
            "design_bytes_per_launch": upd_design,
            "design_gbs": round(design_gbs, 2),
            "frac_design_bytes": round(design_gbs / PEAK_HBM_GBS, 4),
            "cache_window_bytes": window,
            "hbm_gbs_design_less_window": round(hbm_gbs, 2)}
    kernels = {"pass1_rs_norm": round(p1, 5), "finish": round(fin, 5),
               "pass2_update": round(p2, 5)}
    if w.backward_rs:
        bw_bytes = backward_kernel_bytes_per_elem(w) * s.psi_pad
        bw_gbs = bw_bytes / (bw * 1e-3) / 1e9
        kernels["backward_buckets"] = round(bw, 5)
        kernels["backward_launches"] = (w.n_micro * s.n_groups if w.accum_mode == 0 else
                                        w.n_micro * w.n_ranks + s.n_groups)
        if bw_bytes > upd_design:
            # the backward-side reduction moves the most bytes: it is the
            # roofline row (all its launches of one step, back to back);
            # every byte it moves is the method's
            roof = {"bound": "hbm", "achieved": round(bw_gbs, 2), "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": round(bw_gbs / PEAK_HBM_GBS, 4),
                    "traffic": backward_traffic(w),
                    "kernel": ("zf_bucket_rs_kernel (every bucket of every micro-batch)"
                               if w.accum_mode == 0 else
                               "zf_accumulate_kernel + zf_bucket_rs_kernel (no_sync)"),
                    "bytes_per_step": bw_bytes, "launches_per_step":
                        kernels["backward_launches"]}
        kernels["backward_gbs"] = round(bw_gbs, 2)
    line = {
        "metric": "ZeRO step GB/s (algorithmic bytes) and % of HBM peak; params updated/s",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded splitmix64/Irwin-Hall normal grads and master init, "
                "random-init weights)",
        "config": {"workload": w.name, "psi": w.psi, "psi_padded": s.psi_pad,
                   "virtual_ranks": w.n_ranks, "zero_stage": w.stage, **formats(w),
                   "layout": ["global flat", "per-unit FlatParameter",
                              "per-parameter dim-0 (FSDP2)"][w.layout],
                   "rs_policy": ["recompute", "materialize", "fp32 grad shard"][s.policy]},
        "params_updated_per_s": round(w.psi / (ms * 1e-3), 1),
        "pct_hbm_peak": round(100 * gbs / PEAK_HBM_GBS, 2),
        "algorithmic_bytes_per_param": algorithmic_bytes_per_param(w),
        "wall_ms_per_step": round(1e3 * wall / args.steps, 5),
        "device_copy_gbs": round(copy_gbs, 1),
        "kernels_ms": kernels,
        "roofline": roof,
    }
    if graph_ms is not None:
        line["graph_replay"] = {"steps_per_graph": gsteps, "ms_per_step": round(graph_ms, 5),
                                "value": round(alg / (graph_ms * 1e-3) / 1e9, 2),
                                "params_updated_per_s": round(w.psi / (graph_ms * 1e-3), 1)}
    if args.per_step_log:
        res = dev.result()
        with open(args.per_step_log, "a") as f:
            for k, t_ms in enumerate(step_ms):
                f.write(json.dumps({"workload": w.name, "step": k, "ms": round(t_ms, 5),
                                    "n_ranks": w.n_ranks, "stage": w.stage}) + "\n")
            f.write(json.dumps({"workload": w.name, "last_result": {
                "skipped": res.skipped, "t": res.t, "loss_scale": res.scale_next,
                "norm": res.norm, "clip_coef": res.coef}}) + "\n")
    line["stream_probe_gbs"] = probe
    if roof["kernel"].startswith("zf_pass2"):
        # the update pass's HBM-side rate (its bytes less the window's cache
        # hits) against the best probe of its 4-read / 4-write mix
        roof["hbm_frac_of_4r4w_probe"] = round(hbm_gbs / probe["4r4w"], 4)
        mix = own_mix_probe(w, materialized)
        if mix is not None:
            # the same bytes per element moved by a kernel with no
            # arithmetic (its sums, if any, read from HBM): probe time over
            # the update pass's time on equal element counts
            assert update_kernel_bytes_per_elem(w, materialized or w.backward_rs) == \
                UPDATE_MIX_BYTES
            roof["own_mix_probe"] = mix
            roof["frac_of_own_mix_probe"] = round(design_gbs / probe[mix], 4)
    line["ms_per_step_median"] = round(per_step[len(per_step) // 2], 5)
    line["ms_per_step_min"] = round(per_step[0], 5)
    counted = counted_bytes_per_step(w)
    if counted is not None:
        # bytes the counters saw leave L2 per step (committed summaries of
        # these kernel sources), and the HBM share of them: less the
        # update pass's reads of the cached-sums window, which the
        # memory-side cache serves
        line["l2_egress_gbs_counted"] = round(counted / (ms * 1e-3) / 1e9, 2)
        hg = (counted - window) / (ms * 1e-3) / 1e9
        line["hbm_gbs_counted"] = round(hg, 2)
        line["pct_hbm_peak_counted"] = round(100 * hg / PEAK_HBM_GBS, 2)
        # the same against this GPU's own best copy (1 read + 1 write) probe
        line["pct_copy_probe_counted"] = round(100 * hg / probe["1r1w"], 2)
    if skip_probe:
        line["skipped_step_ms"] = skipped_step_ms(w, dev, one_step)
    if w.backward_rs:
        line["config"]["micro_batches"] = w.n_micro
        line["config"]["accumulation"] = ["reduce-scatter every micro-batch",
                                          "no_sync fp32 local, one reduce-scatter"][w.accum_mode]
        line["config"]["buckets"] = s.n_groups
    return line, dev


def headline_summary(line):
    """The second headline configuration's figures, for the main line."""
    keep = ("ms_per_step", "value", "unit", "pct_hbm_peak", "params_updated_per_s",
            "algorithmic_bytes_per_param", "hbm_gbs_counted", "pct_hbm_peak_counted",
            "pct_copy_probe_counted", "l2_egress_gbs_counted", "kernels_ms", "roofline", "skipped_step_ms",
            "ms_per_step_median", "ms_per_step_min", "steps", "warmup")
    out = {"workload": line["config"]["workload"], "config": line["config"]}
    out.update({k: line[k] for k in keep if k in line})
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    from fsdp_sharded_mixed_amd import workloads as _W
    ap.add_argument("--workload", default=None, choices=sorted(_W.ALL),
                    help=f"default {DEFAULT_WORKLOAD}, with {HEADLINE_2} as headline_2")
    ap.add_argument("--no-headline-2", action="store_true",
                    help=f"with the default workload, do not also time {HEADLINE_2}")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the second timing of the K steps replayed from a HIP graph")
    ap.add_argument("--roctx", action="store_true",
                    help="roctx ranges around backward, step and gathers (rocprofv3 "
                         "--marker-trace)")
    ap.add_argument("--graph-steps", type=int, default=10,
                    help="steps captured per graph (1 when it does not divide --steps)")
    ap.add_argument("--no-skip-probe", action="store_true",
                    help="do not time skipped steps (profiled runs: keeps every launch of "
                         "the step kernels an applied step's)")
    ap.add_argument("--set", action="append", default=[], metavar="FIELD=VALUE",
                    help="override a workload field (seed, n_ranks, stage, lr, n_micro, "
                         "max_norm, ...); the line's config records every override")
    ap.add_argument("--per-step-log", metavar="FILE",
                    help="also write one JSON line per timed step (result and time)")
    ap.add_argument("--offload-chunks", type=int, default=16,
                    help="pipeline chunks of an offload step")
    ap.add_argument("--offload-threads", type=int, default=0,
                    help="CPU-Adam threads of an offload step (0: every hardware thread)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--summarize-trace", nargs=2, metavar=("DIR", "OUT"))
    ap.add_argument("--bench-json", metavar="FILE",
                    help="with --summarize-trace: the profiled run's stdout, whose bench "
                         "line's figures are added to the summary")
    ap.add_argument("--summarize-pmc", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "OUT"))
    ap.add_argument("--summarize-dram32", nargs=2, metavar=("DIR", "OUT"),
                    help="summary of a run with --pmc " + " ".join(DRAM32_COUNTERS))
    ap.add_argument("--summarize-table", nargs=2, metavar=("JSONL", "OUT"),
                    help="markdown table of bench lines, one workload per line")
    ap.add_argument("--command", default="", help="command text recorded in a summary")
    args = ap.parse_args()
    default_run = args.workload is None and not args.set and not args.no_headline_2
    if args.per_step_log:
        open(args.per_step_log, "w").close()  # each workload appends its lines
    args.workload = args.workload or DEFAULT_WORKLOAD
    if args.summarize_trace:
        summarize_trace(*args.summarize_trace, args.command, args.bench_json)
        return
    if args.summarize_table:
        summarize_table(*args.summarize_table, args.command)
        return
    if args.summarize_dram32:
        summarize_dram32(args.summarize_dram32[0], args.workload, args.summarize_dram32[1],
                         args.command)
        return
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], args.workload,
                      args.summarize_pmc[2], args.command)
        return
    if args.gpus != 1:
        print(f"bench.py: the step runs on one GPU; --gpus {args.gpus} is not supported "
              "(N data-parallel ranks are emulated on a single device)", file=sys.stderr)
        sys.exit(2)

    import torch
    from fsdp_sharded_mixed_amd import trace, workloads as W

    if args.roctx:
        trace.enable()
    w = W.get(args.workload)
    overrides = apply_overrides(w, args.set)
    torch.cuda.set_device(0)
    print(f"bench: {w.name} Psi={w.psi:,} N={w.n_ranks} stage={w.stage}", file=sys.stderr,
          flush=True)
    # this GPU's plain device-copy bandwidth (1 GiB read + 1 GiB written),
    # the practical ceiling the step's streams are compared against
    src = torch.ones(COPY_BYTES, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3 if args.calibrate_copy else 2):
        dst.copy_(src)
    torch.cuda.synchronize()
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record()
    for _ in range(5):
        dst.copy_(src)
    c1.record()
    torch.cuda.synchronize()
    copy_gbs = 2 * COPY_BYTES * 5 / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del src, dst
    probe = stream_probes()
    line, dev = bench_workload(w, args, probe, copy_gbs, graph=not args.no_graph,
                               skip_probe=not args.no_skip_probe)
    del dev
    torch.cuda.empty_cache()
    if overrides:
        line["config"]["overrides"] = overrides
    if default_run:
        # the second configuration the metric is quoted on, timed the same way
        w2 = W.get(HEADLINE_2)
        print(f"bench: headline_2 {w2.name} Psi={w2.psi:,} N={w2.n_ranks}", file=sys.stderr,
              flush=True)
        line2, dev2 = bench_workload(w2, args, probe, copy_gbs, graph=False,
                                     skip_probe=not args.no_skip_probe)
        del dev2
        torch.cuda.empty_cache()
        line["headline_2"] = headline_summary(line2)
    if not args.no_cpu_baseline:
        cb = cpu_baseline(w)
        if "value" in line:
            cb["gpu_over_oracle"] = round(line["value"] / cb["value"], 1)
        line["cpu_baseline"] = cb
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
