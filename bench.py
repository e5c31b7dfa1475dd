#!/usr/bin/env python3
"""Absorbed-MLA decode benchmark on one MI355X.

Workload: the DeepSeek-V2/V3-shaped decode layer, h=128, d_c=512, d_rope=64,
d_qk_nope=d_v=128, batch 32, 4096 cached tokens + 1 query token per sequence
(kv_len 4097), bf16 latent cache [32, 4097, 576], fp32 accumulation, seeded
synthetic inputs. One step = one mla_decode call: query absorption + RoPE,
split-K attention over the latent cache, split combine + W_UV up-projection.

Prints one JSON line. Inputs are resident in HBM before the timed region; untimed
steps run for half a second (clock settling) before the W warmup steps. Three
copies of (cache, packed weights) are used in turn, as three layers would be,
so the 256 MB Infinity Cache cannot hold the working set between steps.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
    python bench.py --config 3|4|5          the other decode workloads
    python bench.py --workload append       the fused latent append from the hidden state
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0           # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2516.6   # dense bf16 matrix-core peak (256 CU x 2.4 GHz x 4096)
COPIES = 3
EVERY = 8  # timed steps per sampled attention-kernel event pair
SETTLE_S = 0.5  # seconds of untimed steps before the warmup steps


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class HipEvents:
    """Raw hipEvent_t pairs (the library records them around its attention kernel,
    on the stream that kernel is launched on)."""

    def __init__(self, n):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.pairs = []
        for _ in range(n):
            a, b = ctypes.c_void_p(), ctypes.c_void_p()
            assert self.hip.hipEventCreate(ctypes.byref(a)) == 0
            assert self.hip.hipEventCreate(ctypes.byref(b)) == 0
            self.pairs.append((a.value, b.value))

    def elapsed_ms(self, k):
        ms = ctypes.c_float()
        a, b = self.pairs[k]
        assert self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
        return ms.value


def algorithmic(w):
    """FLOPs and bytes the absorbed method needs per step (the cache read once,
    the weights once, queries in, outputs out)."""
    import numpy as np
    kv = w.kv_lens.astype(np.float64)
    vis = sum(float(n) - w.n_q + j + 1 for n in kv for j in range(w.n_q))
    M = w.batch * w.n_q
    flops = (2.0 * w.h * vis * (w.d_c + w.d_r) + 2.0 * w.h * vis * w.d_c
             + 2.0 * w.h * M * w.d_n * w.d_c + 2.0 * w.h * M * w.d_c * w.d_v)
    cache_bytes = float(kv.sum()) * (w.d_c + w.d_r) * 2
    weight_bytes = 2.0 * w.d_c * w.h * (w.d_n + w.d_v)
    io_bytes = M * w.h * (w.d_n + w.d_r) * 2 + M * w.h * w.d_v * 4
    if w.gated:  # the output gate's logits x · W_G, x [M, d_model] bf16, W_G [d_model, h*d_v] bf16
        flops += 2.0 * M * w.d_model * w.h * w.d_v
        weight_bytes += 2.0 * w.d_model * w.h * w.d_v
        io_bytes += 2.0 * M * w.d_model
    return flops, cache_bytes, cache_bytes + weight_bytes + io_bytes


def attention_flops(w):
    """FLOPs of the attention kernel alone: scores and the value sum over the
    visible tokens."""
    vis = sum(float(n) - w.n_q + j + 1 for n in w.kv_lens for j in range(w.n_q))
    return 2.0 * w.h * vis * (w.d_c + w.d_r) + 2.0 * w.h * vis * w.d_c


def config_desc(w):
    import numpy as np
    d = {"workload": w.name, "heads": w.h, "batch": w.batch, "query_tokens": w.n_q,
         "kv_len_max": int(w.kv_max), "kv_len_total": int(np.sum(w.kv_lens)), "d_c": w.d_c,
         "d_rope": w.d_r, "d_qk_nope": w.d_n, "d_v": w.d_v, "layer_copies_rotated": COPIES}
    if w.paged:
        d["cache"] = "paged bf16, %d-token blocks, pool %d blocks" % (w.block_size, w.pool_blocks)
    else:
        d["cache"] = "contiguous bf16 [%d, %d, %d]" % (w.batch, w.kv_max, w.row)
    if w.gated:
        d["gate_d_model"] = w.d_model
    return d


# the attention kernels, their device helpers, and the planner that sizes their launches
KERNEL_SOURCES = ("decode_bf16.hip", "common.hpp", "api.hip", "launch.hpp")
KERNEL_SOURCES_TEXT = " + ".join("mla_latent_kv_41_amd/csrc/" + f for f in KERNEL_SOURCES)


def kernel_source_hash():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(os.path.join(ROOT, "mla_latent_kv_41_amd", "csrc", f), "rb").read())
    return h.hexdigest()


def traffic_from_profile(workload):
    """HBM bytes of one step's attention launches for `workload` (a workload name)
    from the committed rocprofv3 counter runs, or None when absent or taken on a
    different kernel source."""
    p = os.path.join(ROOT, "profiles", "attention_traffic.json")
    if not os.path.exists(p):
        return None
    rec = json.load(open(p)).get("workloads", {}).get(workload)
    if rec is None or rec.get("kernel_source_sha256") != kernel_source_hash():
        return None
    return rec.get("bytes_per_launch")


def stream_read_gbps(nbytes=1 << 30, reps=10):
    """A secondary reference, never a roofline denominator: HBM read bandwidth of a
    plain stream on this GPU, measured outside the timed region as torch's row sums
    of an fp32 [nbytes / 16 KiB, 4096] matrix (it reads nbytes and writes 1/4096 of
    that; the fastest plain read among torch's reductions and GEMVs measured here),
    median of reps after warm-up."""
    import numpy as np
    import torch
    x = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda").view(-1, 4096)
    for _ in range(3):
        x.sum(1)
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        x.sum(1)
        b.record()
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b))
    del x
    return round(nbytes / (float(np.median(times)) * 1e-3) / 1e9, 1)


def _host_cores():
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count()


GRAPH_ROUNDS = 10  # rounds over the COPIES cache copies captured in one graph


def graph_step_ms(steps, n_steps):
    """Step time with the host taken out: GRAPH_ROUNDS x COPIES decode steps (the same
    rotation as the eager loop) captured into one HIP graph, replayed until about
    n_steps steps have run. Before timing, the graph is replayed three times with an
    eager step between replays, and each replay's output must equal the eager output
    bit for bit (the merge order is fixed, so the step is deterministic). Returns
    (ms per step, replays checked)."""
    import torch
    per_graph = GRAPH_ROUNDS * COPIES
    out = steps[0].out
    steps[0].decode()
    torch.cuda.synchronize()
    ref = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for k in range(per_graph):
            steps[k % COPIES].decode()
    torch.cuda.synchronize()
    for _ in range(3):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        if not torch.equal(out, ref):
            raise RuntimeError("graph replay differs from the eager step")
        steps[1 % COPIES].decode()
        torch.cuda.synchronize()
    replays = max(3, -(-n_steps // per_graph))
    g.replay()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(replays):
        g.replay()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / (replays * per_graph)
    del g
    return ms, 3


def cpu_baseline(w, t, budget_s=12.0):
    """The fp64 oracle (explicit K/V, as it stands) on whole sequences of the same
    workload until about budget_s of wall time. `value` prices the sample in the
    metric's unit (the absorbed method's algorithmic FLOPs per second, so it compares
    with the GPU's value); `executed_tflops` is the rate of the FLOPs the explicit
    form actually executes (oracle.unabsorbed_flops of the sample)."""
    import oracle
    done, t0 = 0, time.perf_counter()
    while done < w.batch and time.perf_counter() - t0 < budget_s:
        sel = [(done, i) for i in range(w.h)]
        oracle.mla_decode(h=w.h, d_c=w.d_c, d_r=w.d_r, d_n=w.d_n, d_v=w.d_v, c_kv=t["c_kv"],
                          k_r=t["k_r"], kv_lens=w.kv_lens, q_nope=t["q_nope"], q_r=t["q_r"],
                          w_uk=t["w_uk"], w_uv=t["w_uv"], x=t.get("x"), w_g=t.get("w_g"),
                          store_bf16=True, select=sel)
        done += 1
    secs = time.perf_counter() - t0
    flops, _, _ = algorithmic(_first_sequences(w, done))
    executed = oracle.unabsorbed_flops(w.h, w.d_c, w.d_n, w.d_v, w.d_r, w.kv_lens[:done], w.n_q,
                                       d_model=w.d_model if w.gated else 0)
    return {"value": flops / secs / 1e12, "unit": "TFLOP/s", "cores": oracle.threads(),
            "kind": "oracle",
            "sample": "%d of %d sequences (all %d heads), fp64 explicit-K/V oracle, %.1f s; query tokens/s %.3g"
                      % (done, w.batch, w.h, secs, done * w.n_q / secs),
            "executed_flops": float(executed), "executed_tflops": float(executed) / secs / 1e12,
            "omp_max_threads": oracle.threads(), "nproc": _host_cores()}


def cpu_baseline_absorbed(w, t, budget_s=10.0):
    """The oracle's absorbed fp64 twin (pinned to the explicit form at 1e-12) on whole
    sequences of the same workload, in order and wrapping around, until about
    budget_s: the second CPU baseline. It executes the absorbed method's own FLOPs,
    so `value` is also its executed rate."""
    import oracle
    done, t0 = 0, time.perf_counter()
    while done == 0 or time.perf_counter() - t0 < budget_s:
        b = done % w.batch
        oracle.mla_decode(h=w.h, d_c=w.d_c, d_r=w.d_r, d_n=w.d_n, d_v=w.d_v, c_kv=t["c_kv"],
                          k_r=t["k_r"], kv_lens=w.kv_lens, q_nope=t["q_nope"], q_r=t["q_r"],
                          w_uk=t["w_uk"], w_uv=t["w_uv"], x=t.get("x"), w_g=t.get("w_g"),
                          store_bf16=True, absorbed=True, select=[(b, i) for i in range(w.h)])
        done += 1
    secs = time.perf_counter() - t0
    full, rest = divmod(done, w.batch)
    flops = full * algorithmic(w)[0] + (algorithmic(_first_sequences(w, rest))[0] if rest else 0.0)
    return {"value": flops / secs / 1e12, "unit": "TFLOP/s", "cores": oracle.threads(),
            "kind": "oracle (absorbed fp64 twin)",
            "sample": "%d sequence passes over the %d sequences (all %d heads), fp64 absorbed twin, %.1f s; "
                      "query tokens/s %.3g" % (done, w.batch, w.h, secs, done * w.n_q / secs),
            "executed_flops": flops, "executed_tflops": flops / secs / 1e12,
            "omp_max_threads": oracle.threads(), "nproc": _host_cores()}


def _first_sequences(w, n):
    """The workload restricted to its first n sequences (for pricing a CPU sample)."""
    import copy
    v = copy.copy(w)
    v.batch = n
    v.kv_lens = w.kv_lens[:n]
    return v


TRACE_CMD = ("rocprofv3 --kernel-trace --stats --output-format csv -d <out>/prof_ds -o ds -- "
             "python3 bench.py --steps 20 --warmup 5 --no-cpu-baseline")
TRACE_CMD_CFG = ("rocprofv3 --kernel-trace --stats --output-format csv -d <out>/prof_c{c} -o c{c} -- "
                 "python3 bench.py --config {c} --steps 10 --warmup 3 --no-cpu-baseline")
PMC_CMD = ("rocprofv3 --pmc {c} --output-format csv -d <out>/pmc_c{cfg}/{c} -o {c} -- "
           "python3 bench.py --config {cfg} --steps 4 --warmup 2 --no-cpu-baseline --calibrate-copy")
COPY_BYTES = 512 << 20


def _bench_line(log_path):
    """The JSON line a profiled bench run printed (its last line starting with '{')."""
    line = None
    for ln in open(log_path):
        if ln.startswith("{"):
            line = ln
    if line is None:
        raise SystemExit("no bench result line in %s" % log_path)
    return json.loads(line)


def _short_kernel_name(name):
    name = name.replace("void ", "", 1)
    return name.split("(")[0] if not name.startswith("at::") else name.split(")")[0] + ")"


def summarize_append_trace(d):
    """profiles/ summary of a kernel-trace run of the fused-append bench
    (DIR/prof_append, log DIR/prof_append.log)."""
    import csv
    import glob
    line = _bench_line(os.path.join(d, "prof_append.log"))
    wl = line["config"]["workload"]
    stats = list(csv.DictReader(open(glob.glob(os.path.join(d, "prof_append", "*kernel_stats.csv"))[0])))
    per_call = sum(float(r["AverageNs"]) for r in stats
                   if "splitk_gemm_kernel" in r["Name"] or "latent_finish_kernel" in r["Name"]) / 1e3
    lines = ["# Kernel trace: fused latent append, %s (`bench.py --workload append`)" % wl, "",
             "Command (from /tmp with TMPDIR=/tmp):", "", "    " + APPEND_TRACE_CMD, "",
             "One call = splitk_gemm_kernel (both projections, split over d_model) then "
             "latent_finish_kernel (split sum, RMSNorm, RoPE, store). pack_down_kernel and the fills "
             "belong to set-up.", "",
             "| kernel | calls | average us | min us | max us | share |", "|---|---|---|---|---|---|"]
    for r in stats:
        lines.append("| `%s` | %s | %.2f | %.2f | %.2f | %.1f%% |" % (
            _short_kernel_name(r["Name"]), r["Calls"], float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
            float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
    lines += ["", "Sum of the two kernels' averages: %.2f us per call, %.1f GB/s of the %d algorithmic bytes "
              "per call. (Under the tracer the bench's own clock reads %.2f us per call: the tracer adds "
              "time to every dispatch.)" % (per_call, line["algorithmic_bytes_per_call"] / (per_call * 1e3),
                                           line["algorithmic_bytes_per_call"], line["ms_per_step"] * 1e3), ""]
    open(os.path.join(ROOT, "profiles", "%s_kernel_trace.md" % wl), "w").write("\n".join(lines))
    print("fused append trace summary written")


def _copy_calibration(vals):
    """What FETCH_SIZE and WRITE_SIZE (KiB) count for the one 512 MiB device copy of a
    counter run: the sum over its dispatches (the runtime may split the copy into
    several dispatches of the same grid), checked against the bytes it writes."""
    copy = [k for k in vals if "copyBuffer" in k[0] and k[1] == COPY_BYTES // 4096]
    if len(copy) != 1:
        raise SystemExit("calibration copy not found in the counter runs")
    cf = {c: sum(v) for c, v in vals[copy[0]].items()}
    if abs(cf["WRITE_SIZE"] * 1024 / COPY_BYTES - 1) > 0.05:
        raise SystemExit("calibration copy dispatches write %.0f KiB, not 512 MiB" % cf["WRITE_SIZE"])
    return cf


def _counter_table(d, sub):
    """{(kernel, grid): {counter: [values]}} of the FETCH_SIZE and WRITE_SIZE runs
    under DIR/sub, and the calibration factors from the 512 MiB copy."""
    import csv
    import glob
    from collections import defaultdict
    vals = defaultdict(lambda: defaultdict(list))
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        for f in glob.glob(os.path.join(d, sub, c, "*counter_collection.csv")):
            for r in csv.DictReader(open(f)):
                vals[(_short_kernel_name(r["Kernel_Name"]), int(r["Grid_Size"]))][r["Counter_Name"]].append(
                    float(r["Counter_Value"]))
    cf = _copy_calibration(vals)
    return vals, cf, COPY_BYTES / (cf["FETCH_SIZE"] * 1024), COPY_BYTES / (cf["WRITE_SIZE"] * 1024)


def summarize_append_counters(d):
    """profiles/ counter summary and append_traffic.json from one FETCH_SIZE and one
    WRITE_SIZE run of the fused-append bench (DIR/pmc_append/<C>, logs <C>.log)."""
    shas = {_bench_line(os.path.join(d, "pmc_append", c + ".log"))["append_kernel_source_sha256"]
            for c in ("FETCH_SIZE", "WRITE_SIZE")}
    if len(shas) != 1:
        raise SystemExit("counter runs used different fused-append sources: %s" % shas)
    sha = shas.pop()
    line = _bench_line(os.path.join(d, "pmc_append", "FETCH_SIZE.log"))
    wl = line["config"]["workload"]
    vals, cf, f_fac, w_fac = _counter_table(d, "pmc_append")
    per = {}
    for name in ("mla::splitk_gemm_kernel", "mla::latent_finish_kernel<unsigned short>"):
        # the product is a template over its staging depth (the append's one-chunk
        # splits take splitk_gemm_kernel<1>)
        ks = [k for k in vals if k[0] == name or k[0].startswith(name + "<")]
        if len(ks) != 1:
            raise SystemExit("%s not found once in the counter runs" % name)
        v = {c: sum(x) / len(x) for c, x in vals[ks[0]].items()}
        per[name] = (ks[0][1], len(vals[ks[0]]["FETCH_SIZE"]), v["FETCH_SIZE"], v["WRITE_SIZE"],
                     v["FETCH_SIZE"] * 1024 * f_fac, v["WRITE_SIZE"] * 1024 * w_fac)
    total = sum(p[4] + p[5] for p in per.values())
    lines = ["# HBM traffic counters: fused latent append, %s" % wl, "",
             "Commands (one counter per pass, from /tmp with TMPDIR=/tmp; `--calibrate-copy` adds one 512 MiB "
             "device-to-device copy):", ""]
    lines += ["    " + APPEND_PMC_CMD.format(c=c) for c in ("FETCH_SIZE", "WRITE_SIZE")]
    lines += ["", "Summarised with `python3 bench.py --summarize-profiles <out>`. Fused-append source sha256 "
              "(%s): `%s`" % (" + ".join("mla_latent_kv_41_amd/csrc/" + f for f in APPEND_SOURCES), sha), "",
              "| kernel | grid | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | fetch MB | write MB |",
              "|---|---|---|---|---|---|---|"]
    for n, p in per.items():
        lines.append("| `%s` | %d | %d | %.1f | %.1f | %.3f | %.3f |" % (n, p[0], p[1], p[2], p[3], p[4] / 1e6,
                                                                     p[5] / 1e6))
    lines += ["", "Calibration: the 512 MiB copy counts FETCH_SIZE %.1f KiB (factor %.4f) and WRITE_SIZE %.1f KiB "
              "(factor %.4f)." % (cf["FETCH_SIZE"], f_fac, cf["WRITE_SIZE"], w_fac), "",
              "Per call (both kernels): %.3f MB, against %d algorithmic bytes (the weights once, the hidden "
              "states, the gain, the rows written). The difference is the split partial sums, written by "
              "the product and read back by the finishing kernel." % (total / 1e6,
                                                                       line["algorithmic_bytes_per_call"]), ""]
    open(os.path.join(ROOT, "profiles", "%s_hbm_counters.md" % wl), "w").write("\n".join(lines))
    rec = {"kernels": list(per), "workload": wl, "kernel_source_sha256": sha,
           "kernel_sources": ["mla_latent_kv_41_amd/csrc/" + f for f in APPEND_SOURCES],
           "copy_calibration": {"fetch_factor": round(f_fac, 4), "write_factor": round(w_fac, 4)},
           "bytes_per_kernel": {n: int(p[4] + p[5]) for n, p in per.items()},
           "bytes_per_call": int(total)}
    json.dump(rec, open(os.path.join(ROOT, "profiles", "append_traffic.json"), "w"), indent=1)
    print("fused append counter summary written")


def summarize_profiles(d):
    """profiles/ summaries of whatever rocprofv3 output DIR holds: the fused append's
    trace and counters, the DeepSeek-shaped kernel trace (DIR/prof_ds), the other
    workloads' traces, their kernel-efficiency counters, and their HBM traffic
    counters (one FETCH_SIZE and one WRITE_SIZE run per workload, with the 512 MiB
    copy calibration) into profiles/attention_traffic.json, keyed by the attention
    kernel source hash the profiled runs printed."""
    if os.path.isdir(os.path.join(d, "prof_append")):
        summarize_append_trace(d)
    if os.path.isdir(os.path.join(d, "pmc_append")):
        summarize_append_counters(d)
    if os.path.isdir(os.path.join(d, "prof_ds")):
        summarize_ds_trace(d)
    summarize_other(d)


def summarize_ds_trace(d):
    """profiles/ summary of the DeepSeek-shaped kernel trace (DIR/prof_ds)."""
    import csv
    import glob
    prof = os.path.join(ROOT, "profiles")
    w_name = "deepseek_b32_ctx4096"
    sha = _bench_line(os.path.join(d, "prof_ds.log"))["attention_kernel_source_sha256"]

    def short(name):
        name = name.replace("void ", "", 1)
        return name.split("(")[0] if not name.startswith("at::") else name.split(")")[0] + ")"

    stats = list(csv.DictReader(open(glob.glob(os.path.join(d, "prof_ds", "*kernel_stats.csv"))[0])))
    attn = [short(r["Name"]) for r in stats if short(r["Name"]).startswith(ATTENTION_KERNELS)]
    if len(attn) != 1:
        raise SystemExit("expected one attention kernel in the DeepSeek-shaped trace, found %s" % attn)
    kname = attn[0]
    lines = ["# Kernel trace: DeepSeek-shaped decode (h=128, B=32, 4096+1 tokens)", "",
             "Command (from /tmp with TMPDIR=/tmp; the run includes the bench's clock-settling steps):",
             "", "    " + TRACE_CMD, "",
             "Per-step kernels: qprep_kernel (query absorption + RoPE, the split plan), "
             "%s (split-K attention), combine_kernel (split merge + W_UV). "
             "append_kernel, pack_kernel and the fills belong to set-up." % kname, "",
             "| kernel | calls | average us | min us | max us | share |", "|---|---|---|---|---|---|"]
    for r in stats:
        lines.append("| `%s` | %s | %.2f | %.2f | %.2f | %.1f%% |" % (
            short(r["Name"]), r["Calls"], float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
            float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
    lines += ["", "Attention kernel source sha256 (%s): `%s`" % (KERNEL_SOURCES_TEXT, sha), ""]
    open(os.path.join(prof, "decode_step_%s_kernel_trace.md" % w_name), "w").write("\n".join(lines))


def summarize_other(d):
    """Kernel traces of the other workloads (DIR/prof_c<N>, log DIR/prof_c<N>.log),
    kernel-efficiency counters (DIR/ctr_c<N>) and HBM traffic counters (DIR/pmc_c<N>)."""
    import csv
    import glob
    prof = os.path.join(ROOT, "profiles")
    short = _short_kernel_name
    for c in (3, 4, 5):
        tdir = os.path.join(d, "prof_c%d" % c)
        if not os.path.isdir(tdir):
            continue
        line = _bench_line(tdir + ".log")
        wl = line["config"]["workload"]
        stats = list(csv.DictReader(open(glob.glob(os.path.join(tdir, "*kernel_stats.csv"))[0])))
        lines = ["# Kernel trace: %s (`bench.py --config %d`)" % (wl, c), "",
                 "Command (from /tmp with TMPDIR=/tmp):", "", "    " + TRACE_CMD_CFG.format(c=c), "",
                 "Attention kernel: %s. Bench line of the traced run: %.1f TFLOP/s, %.1f us per step "
                 "(under the tracer)." % (line["roofline"]["kernel"], line["value"], line["ms_per_step"] * 1e3), "",
                 "| kernel | calls | average us | min us | max us | share |", "|---|---|---|---|---|---|"]
        for r in stats:
            lines.append("| `%s` | %s | %.2f | %.2f | %.2f | %.1f%% |" % (
                short(r["Name"]), r["Calls"], float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
                float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
        lines += ["", "Attention kernel source sha256 (%s): `%s`"
                  % (KERNEL_SOURCES_TEXT, line["attention_kernel_source_sha256"]), ""]
        open(os.path.join(prof, "decode_step_%s_kernel_trace.md" % wl), "w").write("\n".join(lines))
    for c in (2, 3, 4, 5):
        if os.path.isdir(os.path.join(d, "ctr_c%d" % c, "sq")):
            summarize_efficiency_counters(d, c)
        if os.path.isdir(os.path.join(d, "pmc_c%d" % c, "WRITE_SIZE")):
            summarize_traffic(d, c)
    print("summaries written")


def summarize_traffic(d, cfg):
    """HBM traffic of one workload's attention launches from one FETCH_SIZE and one
    WRITE_SIZE counter run (DIR/pmc_c<cfg>/<C>, logs DIR/pmc_c<cfg>/<C>.log), scaled by
    what the same counters read for the 512 MiB calibration copy of the same run:
    profiles/attention_<workload>_hbm_counters.md and the workload's entry in
    profiles/attention_traffic.json, keyed by the attention kernel source hash."""
    import csv
    import glob
    from collections import defaultdict
    prof = os.path.join(ROOT, "profiles")
    base = os.path.join(d, "pmc_c%d" % cfg)
    lines_of = {c: _bench_line(os.path.join(base, c + ".log")) for c in ("FETCH_SIZE", "WRITE_SIZE")}
    shas = {ln["attention_kernel_source_sha256"] for ln in lines_of.values()}
    if len(shas) != 1:
        raise SystemExit("counter runs used different attention kernel sources: %s" % shas)
    sha = shas.pop()
    wl = lines_of["FETCH_SIZE"]["config"]["workload"]
    vals = defaultdict(lambda: defaultdict(list))
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        for f in glob.glob(os.path.join(base, c, "*counter_collection.csv")):
            for r in csv.DictReader(open(f)):
                vals[(_short_kernel_name(r["Kernel_Name"]), int(r["Grid_Size"]))][r["Counter_Name"]].append(
                    float(r["Counter_Value"]))
    cf = _copy_calibration(vals)
    f_fac = COPY_BYTES / (cf["FETCH_SIZE"] * 1024)
    w_fac = COPY_BYTES / (cf["WRITE_SIZE"] * 1024)
    attn = sorted(k for k in vals if k[0].startswith(ATTENTION_KERNELS))
    if not attn:
        raise SystemExit("no attention kernel in the counter runs of config %d" % cfg)
    names = sorted({k[0] for k in attn})
    if len(attn) != len(names):
        raise SystemExit("an attention kernel ran with several grids: %s" % attn)
    avg = {k: {c: sum(v) / len(v) for c, v in vals[k].items()} for k in attn}
    fetch_b = sum(v["FETCH_SIZE"] for v in avg.values()) * 1024 * f_fac
    write_b = sum(v["WRITE_SIZE"] for v in avg.values()) * 1024 * w_fac
    kname = " + ".join(names)
    lines = ["# HBM traffic counters: attention launches of %s (`bench.py --config %d`)" % (wl, cfg), "",
             "Commands (one counter per pass, from /tmp with TMPDIR=/tmp; `--calibrate-copy` adds one 512 MiB "
             "device-to-device copy, dispatched as `__amd_rocclr_copyBuffer` with grid %d):" % (COPY_BYTES // 4096), ""]
    lines += ["    " + PMC_CMD.format(c=c, cfg=cfg) for c in ("FETCH_SIZE", "WRITE_SIZE")]
    lines += ["", "Summarised with `python3 bench.py --summarize-profiles <out>`.", "",
              "Attention kernel source sha256 (%s): `%s`" % (KERNEL_SOURCES_TEXT, sha), "",
              "| kernel | grid | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB |", "|---|---|---|---|---|"]
    for (n, g), cs in sorted(vals.items(), key=lambda kv: -sum(kv[1].get("FETCH_SIZE", [0])) / max(1, len(kv[1].get("FETCH_SIZE", [0])))):
        fs = cs.get("FETCH_SIZE", [float("nan")])
        ws = cs.get("WRITE_SIZE", [float("nan")])
        lines.append("| `%s` | %d | %d | %.1f | %.1f |" % (n, g, len(fs), sum(fs) / len(fs), sum(ws) / len(ws)))
    alg = lines_of["FETCH_SIZE"]["roofline"]["algorithmic_bytes_per_launch"]
    lines += ["", "Calibration: the 512 MiB copy reads and writes %d bytes; summed over its dispatches, "
              "FETCH_SIZE counts %.1f KiB (factor %.4f bytes per counted byte) and WRITE_SIZE %.1f KiB "
              "(factor %.4f)." % (
                  COPY_BYTES, cf["FETCH_SIZE"], f_fac, cf["WRITE_SIZE"], w_fac), "",
              "Attention launches of one step (%s): fetch %.1f MB, write %.1f MB, total %.1f MB, against %.1f MB "
              "algorithmic (%.2fx)." % (kname, fetch_b / 1e6, write_b / 1e6, (fetch_b + write_b) / 1e6, alg / 1e6,
                                       (fetch_b + write_b) / alg), ""]
    open(os.path.join(prof, "attention_%s_hbm_counters.md" % wl), "w").write("\n".join(lines))
    p = os.path.join(prof, "attention_traffic.json")
    doc = json.load(open(p)) if os.path.exists(p) else {}
    doc = doc if "workloads" in doc else {"workloads": {}}
    doc["workloads"][wl] = {
        "kernels": names, "kernel_source_sha256": sha,
        "kernel_sources": ["mla_latent_kv_41_amd/csrc/" + f for f in KERNEL_SOURCES],
        "fetch_size_kib_per_step": round(sum(v["FETCH_SIZE"] for v in avg.values()), 1),
        "write_size_kib_per_step": round(sum(v["WRITE_SIZE"] for v in avg.values()), 1),
        "copy_calibration": {"bytes_read": COPY_BYTES, "bytes_written": COPY_BYTES,
                             "fetch_size_kib": cf["FETCH_SIZE"], "write_size_kib": cf["WRITE_SIZE"],
                             "fetch_factor": round(f_fac, 4), "write_factor": round(w_fac, 4)},
        "fetch_bytes_per_launch": int(fetch_b), "write_bytes_per_launch": int(write_b),
        "bytes_per_launch": int(fetch_b + write_b), "algorithmic_bytes_per_launch": alg}
    json.dump(doc, open(p, "w"), indent=1)
    print("traffic counters written for %s" % wl)




ATTENTION_KERNELS = ("mla::decode_kernel", "mla::decode_roles_kernel", "mla::decode_pp_kernel", "mla::decode_mixed_kernel")
# Kernel-efficiency counter passes (one run each; rocprofv3 does not split counters
# over passes): MFMA busy share, MFMA work, LDS busy share and bank conflicts; L2.
EFF_PASSES = {"sq": "MfmaUtil LdsUtil LdsBankConflict SQ_INSTS_VALU_MFMA_MOPS_BF16 GRBM_GUI_ACTIVE",
              "tcc": "TCC_HIT_sum TCC_MISS_sum TCC_REQ_sum"}
EFF_CMD = ("rocprofv3 --pmc {counters} --output-format csv -d <out>/ctr_c{c}/{p} -o {p} -- "
           "python3 bench.py --config {c} --steps 4 --warmup 2 --no-cpu-baseline")


def summarize_efficiency_counters(d, c):
    """profiles/ summary of the kernel-efficiency counter passes of one workload
    (DIR/ctr_c<N>/{sq,tcc}, logs DIR/ctr_c<N>/<pass>.log): per per-step kernel, the
    MFMA busy share of the SIMD cycles, the bf16 MFMA work it counted, the LDS busy
    share and bank-conflict cycles per access cycle, and the L2 hit rate."""
    import csv
    import glob
    from collections import defaultdict
    vals = defaultdict(lambda: defaultdict(list))
    lines_of = {}
    for p in EFF_PASSES:
        lines_of[p] = _bench_line(os.path.join(d, "ctr_c%d" % c, p + ".log"))
        for f in glob.glob(os.path.join(d, "ctr_c%d" % c, p, "*counter_collection.csv")):
            for r in csv.DictReader(open(f)):
                vals[_short_kernel_name(r["Kernel_Name"])][r["Counter_Name"]].append(float(r["Counter_Value"]))
    line = lines_of["sq"]
    wl = line["config"]["workload"]
    per_step = [k for k in vals if k.startswith(ATTENTION_KERNELS) or k.startswith(
        ("mla::combine_kernel", "mla::qprep_kernel", "mla::splitk_gemm_kernel"))]
    avg = lambda k, n: (sum(vals[k][n]) / len(vals[k][n])) if vals[k].get(n) else float("nan")
    lines = ["# Kernel-efficiency counters: %s (`bench.py --config %d`)" % (wl, c), "",
             "Commands (one pass each, from /tmp with TMPDIR=/tmp; rocprofv3 serialises the dispatches "
             "while it counts):", ""]
    lines += ["    " + EFF_CMD.format(counters=v, c=c, p=p) for p, v in EFF_PASSES.items()]
    lines += ["", "Summarised with `python3 bench.py --summarize-profiles <out>`. Attention kernel source "
              "sha256: `%s`" % line["attention_kernel_source_sha256"], "",
              "Columns: MfmaUtil = MFMA busy cycles / (GPU busy cycles x 1024 SIMDs); MFMA GFLOP = "
              "SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 per dispatch; LdsUtil = LDS-active cycles / (GPU busy cycles x "
              "256 CUs); LdsBankConflict = bank-conflict stall cycles per conflict-free LDS cycle; L2 hit = "
              "TCC_HIT / (TCC_HIT + TCC_MISS); GPU busy = GRBM_GUI_ACTIVE cycles per dispatch.", "",
              "| kernel | dispatches | MfmaUtil % | MFMA GFLOP | LdsUtil % | LdsBankConflict | L2 hit % | GPU busy cycles |",
              "|---|---|---|---|---|---|---|---|"]
    for k in sorted(per_step):
        hit, miss = avg(k, "TCC_HIT_sum"), avg(k, "TCC_MISS_sum")
        lines.append("| `%s` | %d | %.1f | %.2f | %.1f | %.4f | %.1f | %.0f |" % (
            k, len(vals[k].get("MfmaUtil", [])), avg(k, "MfmaUtil"),
            avg(k, "SQ_INSTS_VALU_MFMA_MOPS_BF16") * 512 / 1e9, avg(k, "LdsUtil"), avg(k, "LdsBankConflict"),
            100.0 * hit / (hit + miss) if hit + miss > 0 else float("nan"), avg(k, "GRBM_GUI_ACTIVE")))
    lines += ["", "Algorithmic attention FLOPs per launch of this workload: %.2f GFLOP (the attention kernels' "
              "MFMA work above includes the precise form's second MFMA per operand pair and the padding of "
              "partial tiles)." % (line["roofline"]["algorithmic_flops_per_launch"] / 1e9), ""]
    open(os.path.join(ROOT, "profiles", "efficiency_counters_%s.md" % wl), "w").write("\n".join(lines))
    print("efficiency counters written for %s" % wl)


APPEND_COPIES = 64  # packed down-projection copies, rotated as 64 layers would be
APPEND_TRACE_CMD = ("rocprofv3 --kernel-trace --stats --output-format csv -d <out>/prof_append -o append -- "
                    "python3 bench.py --workload append --steps 400 --warmup 50 --no-cpu-baseline")
APPEND_PMC_CMD = ("rocprofv3 --pmc {c} --output-format csv -d <out>/pmc_append/{c} -o {c} -- "
                  "python3 bench.py --workload append --steps 20 --warmup 5 --no-cpu-baseline --calibrate-copy")
APPEND_SOURCES = ("gemm_bf16.hip", "project.hip", "common.hpp")  # the fused append's kernels


def append_source_hash():
    h = hashlib.sha256()
    for f in APPEND_SOURCES:
        h.update(open(os.path.join(ROOT, "mla_latent_kv_41_amd", "csrc", f), "rb").read())
    return h.hexdigest()


def append_traffic_from_profile():
    """HBM bytes per fused-append call (both kernels) from the committed counter
    runs, or None when absent or taken on different kernel sources."""
    p = os.path.join(ROOT, "profiles", "append_traffic.json")
    if not os.path.exists(p):
        return None
    d = json.load(open(p))
    return d.get("bytes_per_call") if d.get("kernel_source_sha256") == append_source_hash() else None


def append_bytes(w):
    """Bytes the fused append must move per call: both projections once, the hidden
    states and the gain in, the new cache rows out."""
    eb = 4 if w.dtype == "f32" else 2
    return (w.d_model * w.row * eb + w.rows * w.d_model * eb + w.d_c * 4 + w.batch * 4
            + w.rows * w.row * eb)


def append_cpu_baseline(w, t, budget_s=10.0):
    """The fp64 oracle of the fused append (as it stands) on the whole workload,
    repeated for about budget_s, in GB/s of the same algorithmic bytes."""
    import oracle
    n, t0 = 0, time.perf_counter()
    while n == 0 or time.perf_counter() - t0 < budget_s:
        oracle.project_latent(hidden=t["hidden"], w_dkv=t["w_dkv"], w_kr=t["w_kr"], gain=t["gain"],
                              eps=w.eps, pos=w.positions(), rope_base=w.rope_base)
        n += 1
    secs = time.perf_counter() - t0
    return {"value": round(append_bytes(w) * n / secs / 1e9, 4), "unit": "GB/s", "cores": oracle.threads(),
            "kind": "oracle",
            "sample": "the whole workload (%d rows) %d times, fp64 oracle, %.1f s; rows/s %.3g"
                      % (w.rows, n, secs, w.rows * n / secs)}


def bench_append(args):
    """The fused latent append from the hidden state (mla_project_append) on the
    DeepSeek-shaped decode step: 32 new tokens, d_model 4096, rows of 512 + 64."""
    import numpy as np
    import torch
    from mla_latent_kv_41_amd import mla, synth
    from mla_latent_kv_41_amd.harness import to_device

    w = synth.make_projection("deepseek")
    t = synth.draw_projection(w)
    log("workload %s: rows=%d d_model=%d row=%d" % (w.name, w.rows, w.d_model, w.row))
    d = mla.dims(128, w.d_c, w.d_r, 128, 128, mla.MLA_BF16, rope_base=w.rope_base)
    w_dkv, w_kr = to_device(t["w_dkv"]), to_device(t["w_kr"])
    nbytes = mla.mla_pack_down_weights(d, w.d_model)
    packs = []
    for _ in range(APPEND_COPIES):
        p = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        mla.mla_pack_down_weights(d, w.d_model, w_dkv, w_kr, p)
        packs.append(p)
    hidden, gain = to_device(t["hidden"]), to_device(t["gain"])
    pos0 = torch.from_numpy(w.pos0.astype(np.int32)).cuda()
    cache = torch.zeros((w.batch, w.t_max, w.row), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(mla.project_workspace_bytes(d, batch=w.batch, n_new=w.n_new, d_model=w.d_model,
                                                 k_splits=args.k_splits), dtype=torch.uint8, device="cuda")
    if args.calibrate_copy:
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # arguments marshalled once per weight copy: a Python-built call per step would
    # take longer than the GPU work it launches
    calls = [mla.prepare_project_append(d, cache, hidden=hidden, packed_down=p, pos0=pos0, workspace=ws,
                                        norm_gain=gain, norm_eps=w.eps, t_max=w.t_max,
                                        k_splits=args.k_splits) for p in packs]

    def call(k):
        calls[k % APPEND_COPIES]()

    t0 = time.perf_counter()
    k = 0
    while time.perf_counter() - t0 < SETTLE_S:
        for _ in range(256):
            call(k)
            k += 1
        torch.cuda.synchronize()
    for k in range(args.warmup):
        call(k)
    torch.cuda.synchronize()
    # HIP events (torch's, on torch's current stream, where the library launches)
    # around the K timed calls; the per-call average is the roofline figure. It
    # spans both kernels of a call and the gap between them.
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for k in range(args.steps):
        call(k)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    alg = append_bytes(w)
    gbps = alg / (ms * 1e-3) / 1e9
    flops = 2.0 * w.rows * w.d_model * w.row
    out = {
        "metric": "fused latent append GB/s (% of HBM peak), 32 new tokens, d_model=4096, row 512+64",
        "value": round(gbps, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; N(0,1) hidden states, N(0,1/d_model) weights, gain 1+N(0,0.01))",
        "config": {"workload": w.name, "batch": w.batch, "new_tokens": w.n_new, "d_model": w.d_model,
                   "d_c": w.d_c, "d_rope": w.d_r, "position": int(w.pos0[0]),
                   "cache": "contiguous bf16 [%d, %d, %d]" % (w.batch, w.t_max, w.row),
                   "weight_copies_rotated": APPEND_COPIES,
                   "k_splits": args.k_splits or "library's choice"},
        "algorithmic_bytes_per_call": alg,
        "tflops": round(flops / (ms * 1e-3) / 1e12, 3),
        "rows_per_s": round(w.rows / (ms * 1e-3), 1),
        "append_kernel_source_sha256": append_source_hash(),
        "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": append_traffic_from_profile(),
                     "kernel": "one mla_project_append call: splitk_gemm_kernel then latent_finish_kernel",
                     "algorithmic_bytes_per_launch": alg},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = append_cpu_baseline(w, t)
    print(json.dumps(out), flush=True)


def bench_explicit(args):
    """The absorbed decode step against the non-absorbed form (MLA tutorial page
    §3.2-§3.3) on one MI355X: the pages compare them on an A100 (DeepSeek-V2, 8K
    context, batch 16; absorbed: about 22% lower latency, 28% higher throughput). Two
    shapes: the DeepSeek-shaped decode (B=32, 4096+1) and the pages' comparison shape
    (B=16, 8192+1), h=128, d_c=512, d_rope=64. The non-absorbed step is timed two
    ways: recomputing the explicit K/V from the latent cache every step
    (mla_expand_kv + mla_decode_explicit, the training-time forward of §3.2), and over
    K/V already held in HBM (mla_decode_explicit alone, as a cache of explicit K/V
    would serve it). K/V are fp32 (17.2 GB for either shape)."""
    import numpy as np
    import torch
    from mla_latent_kv_41_amd import mla, synth
    from mla_latent_kv_41_amd.harness import GpuStep, to_device

    def timed(fn, n):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(n):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    results = []
    for name, kw in (("deepseek_b32_ctx4096", dict()), ("pages_comparison_b16_ctx8192", dict(batch=16, ctx=8192))):
        w = synth.make_workload(2, **kw)
        w.name = name
        t = synth.draw(w)
        steps = [GpuStep(w, t, poison=False) for _ in range(COPIES)]
        for st in steps[1:]:
            st.q_nope, st.q_rope, st.out, st.lse = steps[0].q_nope, steps[0].q_rope, steps[0].out, steps[0].lse
        k_idx = [0]

        def absorbed():
            steps[k_idx[0] % COPIES].decode()
            k_idx[0] += 1
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < SETTLE_S:
            absorbed()
        torch.cuda.synchronize()
        ms_abs = timed(absorbed, max(args.steps, 20))
        st = steps[0]
        k = torch.empty((w.batch, w.kv_max, w.h, 128), dtype=torch.float32, device="cuda")
        v = torch.empty_like(k)
        w_uk, w_uv = to_device(t["w_uk"]), to_device(t["w_uv"])
        ews = torch.empty(2 * w.h * 128 * w.d_c * 2 + 256, dtype=torch.uint8, device="cuda")
        out = torch.empty_like(st.out)
        lse = torch.empty_like(st.lse)

        def expand():
            mla.mla_expand_kv(st.dims, st.cache, kv_lens=st.kv_lens, max_kv_len=w.kv_max, w_uk=w_uk, w_uv=w_uv,
                              k_out=k, v_out=v, batch=w.batch, t_max=st.t_max, workspace=ews)
        expand()
        torch.cuda.synchronize()
        dws = None  # the binding sizes the explicit decode's workspace on each call

        def explicit_decode():
            nonlocal dws
            mla.mla_decode_explicit(st.dims, k, v, st.cache, kv_lens=st.kv_lens, max_kv_len=w.kv_max,
                                    q_nope=st.q_nope, q_rope=st.q_rope, out=out, lse=lse, t_max=st.t_max,
                                    kv_lens_host=st.kv_lens_host, workspace=dws)
        explicit_decode()
        torch.cuda.synchronize()
        n_ex = max(4, args.steps // 5)
        ms_dec = timed(explicit_decode, n_ex)
        ms_exp = timed(expand, n_ex)
        ms_both = timed(lambda: (expand(), explicit_decode()), n_ex)
        # the two forms agree (fp32 explicit form against the bf16 absorbed path)
        ref = st.decode().cpu().numpy().astype(np.float64)
        explicit_decode()
        got = out.cpu().numpy().astype(np.float64)
        agree = float(np.max(np.abs(got - ref)) / np.sqrt(np.mean(got ** 2)))
        kv_bytes = 2.0 * w.batch * w.kv_max * w.h * 128 * 4
        flops_abs, cache_bytes, _ = algorithmic(w)
        expand_flops = 2.0 * float(np.sum(w.kv_lens)) * w.d_c * w.h * 256
        results.append({
            "workload": name, "batch": w.batch, "kv_len": int(w.kv_max), "heads": w.h,
            "absorbed_step_ms": round(ms_abs, 5),
            "non_absorbed_recompute_step_ms": round(ms_both, 4),
            "non_absorbed_cached_kv_step_ms": round(ms_dec, 4),
            "expand_kv_ms": round(ms_exp, 4),
            "expand_kv_tflops": round(expand_flops / (ms_exp * 1e-3) / 1e12, 1),
            "explicit_decode_kv_GBps": round(kv_bytes / (ms_dec * 1e-3) / 1e9, 1),
            "absorbed_latency_vs_recompute": round(ms_abs / ms_both, 5),
            "absorbed_latency_vs_cached_kv": round(ms_abs / ms_dec, 5),
            "absorbed_throughput_gain_vs_cached_kv": round(ms_dec / ms_abs, 2),
            "cache_bytes_absorbed": cache_bytes, "kv_bytes_non_absorbed_fp32": kv_bytes,
            "forms_agree_max_abs_over_rms": agree,
        })
        log(json.dumps(results[-1]))
        del k, v, steps, st
        torch.cuda.empty_cache()
    print(json.dumps({
        "metric": "absorbed vs non-absorbed MLA decode step latency (ms), h=128, one MI355X",
        "value": results[0]["absorbed_latency_vs_cached_kv"], "unit": "absorbed / non-absorbed step time",
        "n_gpus": 1, "steps": args.steps, "higher_is_better": False, "dtype": "bf16 cache; fp32 explicit K/V",
        "data": "synthetic (seeded)", "config": {"workload": "absorbed_vs_non_absorbed"},
        "pages_claim_context": "A100, DeepSeek-V2, 8K context, batch 16: absorbed about -22% latency, +28% throughput",
        "results": results}), flush=True)


def bench_folded(args):
    """Weight-level absorption (MLA tutorial page §2.2: W_UK folded into the query's
    up-projection W_UQ, W_UV into the output projection W_O) against the runtime
    absorption the library does, on the DeepSeek-shaped layer from the query latent
    c_Q (d_q = 512, the tutorial's §4.2 choice) to the layer output (d_model = 4096):

      runtime: q_nope = c_Q · W_UQ;  mla_decode (W_UK and W_UV applied per step);
               y = out · W_O         weights per step 16.8 + 33.6 + 134.2 MB
      folded:  q_abs = c_Q · W_UQK;  mla_decode_latent;  y = o_lat · W_UVO
               weights per step 67.1 + 536.9 MB

    The projections are plain bf16 products (torch, i.e. hipBLASLt); three copies of
    every weight set rotate as three layers would, so none stays in the 256 MB
    Infinity Cache. Reports each form's step time and its parts."""
    import numpy as np
    import torch
    from mla_latent_kv_41_amd import mla, synth
    from mla_latent_kv_41_amd.harness import GpuStep

    w = synth.make_workload(2)
    t = synth.draw(w)
    d_q, d_model = 512, 4096
    steps = [GpuStep(w, t, poison=False) for _ in range(COPIES)]
    for st in steps[1:]:
        st.q_rope, st.out, st.lse = steps[0].q_rope, steps[0].out, steps[0].lse
    g = torch.Generator(device="cuda").manual_seed(4103)
    bf = torch.bfloat16
    M, H = w.batch * w.n_q, w.h
    c_q = torch.randn(M, d_q, device="cuda", generator=g).to(bf)
    rt = [(torch.randn(d_q, H * 128, device="cuda", generator=g).div_(d_q ** 0.5).to(bf),
           torch.randn(H * 128, d_model, device="cuda", generator=g).div_((H * 128) ** 0.5).to(bf))
          for _ in range(COPIES)]
    fd = [(torch.randn(d_q, H * 512, device="cuda", generator=g).div_(d_q ** 0.5).to(bf),
           torch.randn(H * 512, d_model, device="cuda", generator=g).div_((H * 512) ** 0.5).to(bf))
          for _ in range(COPIES)]
    o_lat = torch.empty(M, H, 512, dtype=torch.float32, device="cuda")
    ws_lat = [None]

    def runtime(k):
        st = steps[k % COPIES]
        w_uq, w_o = rt[k % COPIES]
        st.q_nope = (c_q @ w_uq).view(w.batch, w.n_q, H, 128)
        st.decode()
        return st.out.view(M, H * 128).to(bf) @ w_o

    def folded(k):
        st = steps[k % COPIES]
        w_uqk, w_uvo = fd[k % COPIES]
        q_abs = (c_q @ w_uqk).float().view(w.batch, w.n_q, H, 512)
        mla.mla_decode_latent(st.dims, st.cache, kv_lens=st.kv_lens, max_kv_len=w.kv_max, q_abs=q_abs,
                              q_rope=st.q_rope, o_lat=o_lat, t_max=st.t_max, kv_lens_host=st.kv_lens_host,
                              workspace=ws_lat[0])
        return o_lat.view(M, H * 512).to(bf) @ w_uvo

    def timed(fn, n):
        t0 = time.perf_counter()
        k = 0
        while time.perf_counter() - t0 < SETTLE_S:
            fn(k)
            k += 1
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for k in range(n):
            fn(k)
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    n = max(args.steps, 20)
    ms_rt = timed(runtime, n)
    ms_fd = timed(folded, n)
    ms_rt_q = timed(lambda k: c_q @ rt[k % COPIES][0], n)
    ms_rt_o = timed(lambda k: steps[0].out.view(M, H * 128).to(bf) @ rt[k % COPIES][1], n)
    ms_fd_q = timed(lambda k: (c_q @ fd[k % COPIES][0]).float(), n)
    ms_fd_o = timed(lambda k: o_lat.view(M, H * 512).to(bf) @ fd[k % COPIES][1], n)
    rt_bytes = 2.0 * (d_q * H * 128 + 2 * 512 * H * 128 + H * 128 * d_model)
    fd_bytes = 2.0 * (d_q * H * 512 + H * 512 * d_model)
    flops_abs, cache_bytes, _ = algorithmic(w)
    rt_flops = flops_abs + 2.0 * M * (d_q * H * 128 + H * 128 * d_model)
    fd_flops = flops_abs - 2.0 * H * M * 128 * 512 * 2 + 2.0 * M * (d_q * H * 512 + H * 512 * d_model)
    out = {
        "metric": "weight-level vs runtime absorption: MLA layer step (c_Q -> y) latency, DeepSeek-shaped",
        "value": round(ms_fd / ms_rt, 3), "unit": "folded / runtime step time", "n_gpus": 1, "steps": n,
        "higher_is_better": False, "dtype": "bf16", "data": "synthetic (seeded)",
        "config": {"workload": "weight_folding_deepseek_b32_ctx4096", "d_q": d_q, "d_model": d_model,
                   "weight_copies_rotated": COPIES},
        "runtime_step_ms": round(ms_rt, 5), "folded_step_ms": round(ms_fd, 5),
        "runtime_parts_ms": {"c_Q·W_UQ": round(ms_rt_q, 5), "out·W_O": round(ms_rt_o, 5)},
        "folded_parts_ms": {"c_Q·W_UQK": round(ms_fd_q, 5), "o_lat·W_UVO": round(ms_fd_o, 5)},
        "weight_bytes_per_step": {"runtime": rt_bytes, "folded": fd_bytes},
        "flops_per_step": {"runtime": rt_flops, "folded": fd_flops},
        "latent_cache_bytes": cache_bytes,
    }
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run one 512 MiB device copy first (counter calibration)")
    ap.add_argument("--config", type=int, default=2, choices=[2, 3, 4, 5],
                    help="workload: 2 DeepSeek-shaped (default, the headline), 3 paged long "
                         "context, 4 ragged with two queries, 5 gated h=64 without RoPE")
    ap.add_argument("--workload", default="decode", choices=["decode", "append", "explicit", "folded"],
                    help="decode: the decode step (default); append: the fused latent append "
                         "from the hidden state (mla_project_append); explicit: the absorbed step "
                         "against the non-absorbed form (mla_expand_kv + mla_decode_explicit); "
                         "folded: weight-level absorption (mla_decode_latent) against the runtime form")
    ap.add_argument("--k-splits", type=int, default=0,
                    help="append workload: force the d_model splits of the product (0: library)")
    ap.add_argument("--summarize-profiles", metavar="DIR",
                    help="write profiles/ summaries from rocprofv3 output under DIR "
                         "(no GPU work)")
    args = ap.parse_args()
    if args.summarize_profiles:
        summarize_profiles(args.summarize_profiles)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if args.workload == "append":
        bench_append(args)
        return
    if args.workload == "explicit":
        bench_explicit(args)
        return
    if args.workload == "folded":
        bench_folded(args)
        return

    import numpy as np
    import torch
    from mla_latent_kv_41_amd import mla, synth
    from mla_latent_kv_41_amd.harness import GpuStep

    w = synth.make_workload(args.config)
    t = synth.draw(w)
    log("workload %s: B=%d kv_len=%d h=%d row=%d" % (w.name, w.batch, w.kv_max, w.h, w.row))
    steps = [GpuStep(w, t, poison=False) for _ in range(COPIES)]
    for s in steps[1:]:
        s.q_nope, s.q_rope, s.out, s.lse = steps[0].q_nope, steps[0].q_rope, steps[0].out, steps[0].lse
    torch.cuda.synchronize()

    if args.calibrate_copy:
        src = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # The attention kernel is timed on every EVERY-th step of the timed region (at
    # least four samples): each timed launch carries its own event pair, which costs
    # the step several microseconds, so sampling keeps the step rate honest.
    every = max(1, min(EVERY, args.steps // 4))
    sampled = list(range(0, args.steps, every))
    ev = HipEvents(len(sampled))
    # Clock settling: the GPU ramps its clocks over the first fraction of a second of
    # sustained load, so untimed steps run for SETTLE_S of wall time before the W
    # warmup steps (measured: 10 warmup steps alone leave the step ~10% slower).
    t0 = time.perf_counter()
    k = 0
    while time.perf_counter() - t0 < SETTLE_S:
        for _ in range(64):
            steps[k % COPIES].decode()
            k += 1
        torch.cuda.synchronize()
    for k in range(args.warmup):
        steps[k % COPIES].decode()
    torch.cuda.synchronize()

    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for k in range(args.steps):
        if k % every == 0:
            steps[k % COPIES].decode(events=ev.pairs[k // every])
        else:
            steps[k % COPIES].decode()
    end.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    ms = total_ms / args.steps
    attn_ms = [ev.elapsed_ms(k) for k in range(len(sampled))]
    attn_avg = float(np.mean(attn_ms))

    flops, cache_bytes, alg_bytes = algorithmic(w)
    tflops = flops / (ms * 1e-3) / 1e12
    cache_gbps = cache_bytes / (ms * 1e-3) / 1e9
    tok_s = w.batch * w.n_q / (ms * 1e-3)
    attn_gbps = cache_bytes / (attn_avg * 1e-3) / 1e9
    traffic = traffic_from_profile(w.name)
    attn_flops = attention_flops(w)
    attn_tflops = attn_flops / (attn_avg * 1e-3) / 1e12
    mfma_bound = args.config == 4  # 256 score rows per tile: the matrix cores bind
    if mfma_bound:
        roof = {"bound": "mfma", "achieved": round(attn_tflops, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(attn_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                "traffic": traffic, "hbm_GBps": round(attn_gbps, 1),
                "hbm_frac": round(attn_gbps / HBM_PEAK_GBPS, 4)}
    else:
        roof = {"bound": "hbm", "achieved": round(attn_gbps, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(attn_gbps / HBM_PEAK_GBPS, 4), "traffic": traffic,
                "mfma_TFLOPs": round(attn_tflops, 1),
                "mfma_frac": round(attn_tflops / MFMA_BF16_PEAK_TFLOPS, 4)}
    roof.update({"kernel": "split-K attention over the latent cache (all attention launches of a step: the fast "
                           "form for sequences of 4096 tokens or more, the precise form below)",
                 "algorithmic_bytes_per_launch": cache_bytes, "algorithmic_flops_per_launch": attn_flops})
    out = {
        "metric": "MLA decode TFLOP/s + latent-cache GB/s (% roofline), h=128 B=32 ctx=4096",
        # other workloads (--config) report the same quantities for their own shapes
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; N(0,1) RMS-normalised latents, N(0,1/512) weights)",
        "config": config_desc(w),
        "latent_cache_GBps": round(cache_gbps, 1),
        "latent_cache_frac_of_hbm_peak": round(cache_gbps / HBM_PEAK_GBPS, 4),
        "algorithmic_GBps": round(alg_bytes / (ms * 1e-3) / 1e9, 1),
        "algorithmic_frac_of_hbm_peak": round(alg_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "tflops_frac_of_mfma_peak": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
        "tokens_per_s": round(tok_s, 1),
        "attention_kernel_ms": round(attn_avg, 5),
        "attention_kernel_samples": len(sampled),
        "attention_kernel_source_sha256": kernel_source_hash(),
        "roofline": roof,
    }
    # the same steps replayed from a HIP graph (no Python or launch overhead): the
    # difference to ms_per_step is what the host adds per step
    g_ms, g_checked = graph_step_ms(steps, args.steps)
    out["graph_ms_per_step"] = round(g_ms, 5)
    out["graph_replays_checked_bitwise"] = g_checked
    out["host_overhead_ms_per_step"] = round(ms - g_ms, 5)
    if not args.no_cpu_baseline:
        out["stream_read_GBps"] = stream_read_gbps()
        out["attention_frac_of_stream_read"] = round(attn_gbps / out["stream_read_GBps"], 4)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, t)
        out["cpu_baseline_absorbed"] = cpu_baseline_absorbed(w, t)
        out["speedup_vs_cpu"] = round(out["value"] / out["cpu_baseline"]["value"], 1)
        out["speedup_vs_cpu_absorbed"] = round(out["value"] / out["cpu_baseline_absorbed"]["value"], 1)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
