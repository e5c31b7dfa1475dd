"""Per-CU rates of the units the attention kernels lean on (LDS reads, the two bf16
MFMA shapes, plain vector loads, direct-to-LDS loads), from the microbenchmark in
probe/rates.hip.

    python -m mla_latent_kv_41_amd.rates --build          # compile on the CPU
    python -m mla_latent_kv_41_amd.rates [--write FILE]   # run it on the GPU

The binary is built in-tree next to its source. Each line gives the rate of the
slowest wave of a 256-workgroup launch (one workgroup per CU), in bytes or FLOPs
per shader-clock cycle per CU.
"""
from __future__ import annotations

import argparse
import os
import subprocess
import sys

from . import build as _build

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "probe", "rates.hip")
BIN = os.path.join(HERE, "probe", "rates")


def build_probe(out: str = BIN) -> str:
    flags = [f for f in _build.FLAGS if f not in ("-fPIC", "-shared")]
    tmp = out + ".tmp%d" % os.getpid()
    res = subprocess.run([_build.HIPCC, *flags, SRC, "-o", tmp], capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stderr[-4000:])
    os.replace(tmp, out)
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--build", action="store_true", help="compile the microbenchmark and exit")
    ap.add_argument("--write", metavar="FILE", help="also write the output, with this command, to FILE")
    args = ap.parse_args()
    if args.build:
        print(build_probe())
        return 0
    if not os.path.exists(BIN):
        raise SystemExit("%s is not built: run python -m mla_latent_kv_41_amd.rates --build" % BIN)
    res = subprocess.run([BIN], capture_output=True, text=True)
    sys.stdout.write(res.stdout)
    sys.stderr.write(res.stderr)
    if res.returncode != 0:
        return res.returncode
    if args.write:
        with open(args.write, "w") as f:
            f.write("# Per-CU unit rates (microbenchmark)\n\n"
                    "Command: `python3 -m mla_latent_kv_41_amd.rates --build` (CPU), then\n"
                    "`python3 -m mla_latent_kv_41_amd.rates --write <file>`.\n\n"
                    "Source: mla_latent_kv_41_amd/probe/rates.hip. One workgroup per CU (256), "
                    "rates from the slowest wave, per shader-clock cycle per CU.\n\n```\n"
                    + res.stdout + "```\n")
    return 0


if __name__ == "__main__":
    sys.exit(main())
