"""Phase stamps of the attention kernels.

Builds libmla with -DMLA_STAMPS (the kernels then read the shader clock at entry,
right after every step's barrier, after the last value pass and after the
epilogue's stores; see StampRec in csrc/decode_bf16.hip), runs decode steps of one
workload through that build, and prints the phases of the sampled workgroups of
the last attention launch as a markdown table.

    python -m mla_latent_kv_41_amd.stamps --build DIR            # build only (CPU)
    python -m mla_latent_kv_41_amd.stamps --lib DIR/libmla.so --config 2 [--write FILE]

    python -m mla_latent_kv_41_amd.stamps --time-only --config 2 --copies 1   # product build

Each stamp costs one scalar round trip where the wave has no LDS operation
outstanding, so the stamped kernel runs a little slower than the product build;
the table gives both kernel times. Three copies of (cache, weights) are decoded in
turn, as in the benchmark.
"""
from __future__ import annotations

import argparse
import ctypes
import os
import statistics
import subprocess
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
UNITS, WAVES, SLOTS = 64, 8, 16  # the stamp buffer's shape (kStampUnits, kStampWaves, kStampSlots)


def build_stamped(out_dir: str) -> str:
    from . import build
    os.makedirs(out_dir, exist_ok=True)
    lib = os.path.join(out_dir, "libmla.so")
    cmd = [build.HIPCC, *build.FLAGS, "-DMLA_STAMPS", *build.sources(), "-o", lib]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stderr[-3000:])
    return lib


def _events(n):
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    pairs = []
    for _ in range(n):
        a, b = ctypes.c_void_p(), ctypes.c_void_p()
        assert hip.hipEventCreate(ctypes.byref(a)) == 0 and hip.hipEventCreate(ctypes.byref(b)) == 0
        pairs.append((a.value, b.value))

    def elapsed(p):
        ms = ctypes.c_float()
        assert hip.hipEventElapsedTime(ctypes.byref(ms), p[0], p[1]) == 0
        return ms.value
    return hip, pairs, elapsed


def run(config: int, steps: int, num_splits: int = 0, copies: int = 3):
    """Decode steps through the loaded (stamped) library; returns the stamp buffer of
    the last step and the attention times (ms) of the timed steps. `copies` copies
    of (cache, weights) are decoded in turn."""
    import numpy as np
    import torch
    from . import mla, synth
    from .harness import GpuStep
    L = mla.lib()
    stamped = hasattr(L, "mla_stamps_buffer")
    w = synth.make_workload(config)
    t = synth.draw(w)
    # by default three copies of (cache, weights) in turn, as the benchmark does, so
    # the memory-side cache cannot hold the working set; one copy lets it
    steps_on = [GpuStep(w, t, poison=False) for _ in range(copies)]
    for c in steps_on[1:]:
        c.q_nope, c.q_rope, c.out, c.lse = steps_on[0].q_nope, steps_on[0].q_rope, steps_on[0].out, steps_on[0].lse
    hip, pairs, elapsed = _events(steps)
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < 0.5:  # clock ramp
        for k in range(32):
            steps_on[k % copies].decode(num_splits=num_splits)
        torch.cuda.synchronize()
    for k in range(steps):
        steps_on[k % copies].decode(num_splits=num_splits, events=pairs[k])
    torch.cuda.synchronize()
    attn = [elapsed(p) for p in pairs]
    if not stamped:
        return w, None, attn
    ptr, nbytes = ctypes.c_void_p(), ctypes.c_size_t()
    L.mla_stamps_buffer.restype = ctypes.c_int32
    L.mla_stamps_buffer.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.POINTER(ctypes.c_size_t)]
    assert L.mla_stamps_buffer(ctypes.byref(ptr), ctypes.byref(nbytes)) == 0
    assert nbytes.value == UNITS * WAVES * SLOTS * 8
    host = np.zeros(UNITS * WAVES * SLOTS, np.uint64)
    hip.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
    assert hip.hipMemcpy(host.ctypes.data, ptr.value, nbytes.value, 2) == 0  # device to host
    return w, host.reshape(UNITS, WAVES, SLOTS), attn


def table(w, st, attn, product_ms=None):
    """Markdown lines: per role, the mean over sampled workgroups of each phase."""
    import numpy as np
    valid = [(u, v) for u in range(UNITS) for v in range(WAVES) if st[u, v, 8] > st[u, v, 0] > 0]
    if not valid:
        raise RuntimeError("no stamps recorded")
    kernel_ms = statistics.median(attn)
    total = np.median([float(st[u, v, 8] - st[u, v, 0]) for u, v in valid])
    ghz = total / (kernel_ms * 1e6)  # the sampled workgroups span about the whole launch
    # role-split form: waves 0-1 score, waves 2-3 hold the values; 128-row form: every
    # wave does both; eight-wave form: waves 0-3 score, waves 4-7 hold the values
    roles = {"waves 0-1": (0, 1), "waves 2-3": (2, 3), "waves 4-7": (4, 5, 6, 7)}
    lines = ["| phase (cycles, mean over sampled workgroups) | " + " | ".join(roles) + " |",
             "|---|" + "---|" * len(roles)]
    rows = [("entry to the first step's barrier (Q, first tiles)", lambda s: s[1] - s[0]),
            ("steps (barriers passed)", lambda s: s[3]),
            ("one step (barrier to barrier), mean", lambda s: s[4] / max(1, s[3] - 1)),
            ("one step, shortest", lambda s: s[5]),
            ("one step, longest", lambda s: s[6]),
            ("barrier to mark 0, mean per step (eight-wave form: scores done / loads issued)",
             lambda s: s[9] / max(1, s[3])),
            ("barrier to mark 1, mean per step (eight-wave form: P written / value MFMAs issued)",
             lambda s: s[10] / max(1, s[3] - 1)),
            ("barrier to mark 2, mean per step (eight-wave form: next tile landed)",
             lambda s: s[11] / max(1, s[3] - 1)),
            ("last barrier to the end of the last value pass", lambda s: s[7] - s[2]),
            ("epilogue (partial rows stored and complete)", lambda s: s[8] - s[7]),
            ("entry to stores complete", lambda s: s[8] - s[0])]
    for name, f in rows:
        cells = []
        for ws in roles.values():
            vals = [float(f(st[u, v].astype(np.float64))) for u, v in valid if v in ws]
            cells.append("%.0f" % statistics.mean(vals) if vals else "-")
        lines.append("| %s | %s |" % (name, " | ".join(cells)))
    lines += ["", "Attention launch (HIP events, median of %d): %.2f us instrumented%s; the stamps' clock "
              "runs at about %.2f GHz (entry-to-completion cycles of the sampled workgroups over that time); "
              "%d sampled (workgroup, wave) records." % (
                  len(attn), kernel_ms * 1e3,
                  "" if product_ms is None else ", %.2f us in the product build" % (product_ms * 1e3), ghz,
                  len(valid))]
    return lines


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--build", metavar="DIR", help="build the instrumented library into DIR and exit")
    ap.add_argument("--lib", metavar="PATH", help="an instrumented libmla.so (from --build)")
    ap.add_argument("--config", type=int, default=2, choices=[2, 3, 4, 5])
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--num-splits", type=int, default=0,
                    help="force token ranges per sequence (e.g. 8 on the DeepSeek shape: the 128-row form)")
    ap.add_argument("--write", metavar="FILE", help="also write the table, with this command, to FILE")
    ap.add_argument("--time-only", action="store_true",
                    help="print the median attention time (ms) of the loaded library and exit")
    ap.add_argument("--copies", type=int, default=3,
                    help="with --time-only: copies of (cache, weights) decoded in turn (1 lets the "
                         "memory-side cache hold one copy's working set)")
    args = ap.parse_args()
    if args.build:
        print(build_stamped(args.build))
        return
    if args.time_only:
        if args.copies < 1:
            ap.error("--copies must be at least 1")
        _, _, attn = run(args.config, args.steps, args.num_splits, args.copies)
        print("attention_ms %.6f" % statistics.median(attn))
        return
    if not args.lib:
        ap.error("--lib or --build is required")
    # the product build's time on the same GPU, from a process of its own
    env = dict(os.environ)
    env.pop("MLA_LIB_PATH", None)
    res = subprocess.run([sys.executable, "-m", "mla_latent_kv_41_amd.stamps", "--time-only", "--config",
                          str(args.config), "--steps", str(args.steps), "--num-splits", str(args.num_splits)],
                         capture_output=True, text=True, env=env, cwd=os.path.dirname(HERE))
    product_ms = None
    for line in res.stdout.splitlines():
        if line.startswith("attention_ms "):
            product_ms = float(line.split()[1])
    os.environ["MLA_LIB_PATH"] = os.path.abspath(args.lib)  # before the binding loads a library
    w, st, attn = run(args.config, args.steps, args.num_splits)
    if st is None:
        raise RuntimeError("%s is not an instrumented build (no mla_stamps_buffer)" % args.lib)
    lines = ["# Attention phases: %s (instrumented build)" % w.name, "",
             "Command: `python3 -m mla_latent_kv_41_amd.stamps --build <dir>` (CPU), then",
             "`python3 -m mla_latent_kv_41_amd.stamps --lib <dir>/libmla.so --config %d --steps %d%s`." % (
                 args.config, args.steps, " --num-splits %d" % args.num_splits if args.num_splits else ""), "",
             "Workgroups whose unit is below %d record their waves' stamps; the table is of the last of "
             "the timed steps." % UNITS, ""] + table(w, st, attn, product_ms) + [""]
    text = "\n".join(lines)
    print(text)
    if args.write:
        with open(args.write, "w") as f:
            f.write(text)


if __name__ == "__main__":
    sys.exit(main())
