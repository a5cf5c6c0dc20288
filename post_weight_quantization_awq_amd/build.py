"""Build libawq.so (HIP, gfx950) in-tree: one hipcc -c per source, then link.

Usage: python -m post_weight_quantization_awq_amd.build [--jobs N]
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libawq.so")
# the VALU issue-rate probe behind the search kernel's ALU peak (bench.py
# --workload valu_issue_probe): a library of its own, not part of libawq
PROBE_SRCS = [os.path.join(PKG, "probe", "valu_issue.hip"), os.path.join(PKG, "probe", "stream_read.hip")]
PROBE_LIB = os.path.join(PKG, "libawq_probe.so")
ARCH = os.environ.get("AWQ_OFFLOAD_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # no contraction of separate mul/add into FMA: the quantization arithmetic
    # is written with explicit fmaf where an FMA is intended
    "-ffp-contract=off",
    # keep the compiler from forming packed fp32 ops (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src)[:-4] + ".o")
    cmd = [HIPCC, *CFLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in (r.stderr or "").splitlines()
                     if "packed-fp32-ops" not in l)  # host pass does not know the feature
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{errs}")
    if errs.strip():
        sys.stderr.write(errs + "\n")
    return obj


def build(jobs: int = 8) -> str:
    if shutil.which(HIPCC) is None and not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=max(1, min(jobs, len(srcs)))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    r = subprocess.run([HIPCC, "-shared", f"--offload-arch={ARCH}", "-o", tmp, *objs],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    build_probe()
    return LIB


def build_probe() -> str:
    tmp = PROBE_LIB + ".tmp"
    r = subprocess.run([HIPCC, *CFLAGS, "-shared", *PROBE_SRCS, "-o", tmp], capture_output=True, text=True)
    if r.returncode != 0:
        errs = "\n".join(l for l in (r.stderr or "").splitlines() if "packed-fp32-ops" not in l)
        raise RuntimeError(f"hipcc failed on {PROBE_SRCS}:\n{errs}")
    os.replace(tmp, PROBE_LIB)
    return PROBE_LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=8)
    a = ap.parse_args()
    print(build(a.jobs))
