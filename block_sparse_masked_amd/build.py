"""Build the gfx950 shared library ``libflexattn.so`` in-tree with hipcc.

Usage: ``python -m block_sparse_masked_amd.build [--jobs N] [--debug]``.
Every HIP source is compiled for gfx950 only, with packed-FP32 instruction
selection disabled (plain fp32 VALU code only).
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libflexattn.so")
# matrix-core throughput probe, a library of its own that only bench.py loads
PROBE_SRC = "probe_mfma.hip"
PROBE_LIB = os.path.join(HERE, "libfaprobe.so")

SOURCES = ["api.cpp", "block_mask.hip", "fwd_bf16.hip", "fwd_f32.hip"]
# bwd_bf16.hip is compiled once per 16-bit element type (0: bf16, 1: fp16)
BWD_ELEMS = (0, 1)
# fwd_bf16_inst.hip is compiled once per kernel slice (head dim, paged K/V,
# fp16 elements), so the slices build in parallel
SLICES = [(d, paged, f16) for d in (64, 128, 256) for paged, f16 in ((0, 0), (1, 0), (0, 1), (1, 1))]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libflexattn.so)")


def common_flags(debug: bool):
    flags = ["-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", CSRC, "-I", INCLUDE,
             "-Wall", "-Wno-unused-function",
             # plain fp32 VALU code: no packed-fp32 instruction selection
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
    flags += ["-O1", "-g"] if debug else ["-O3"]
    return flags


def compile_one(src: str, debug: bool, extra, defines=(), obj_name=None) -> str:
    obj = os.path.join(BUILD, obj_name or os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") or src.endswith(".cpp") else []
    cmd = ([hipcc()] + common_flags(debug) + list(extra) + [f"-D{d}" for d in defines] + lang
           + ["-c", os.path.join(CSRC, src), "-o", obj])
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(line for line in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in line)
    if res.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{' '.join(cmd)}\n{out}")
    if out.strip():
        sys.stderr.write(out + "\n")
    return obj


def _jobs():
    """(source, defines, object name) of every object of the library."""
    jobs = [(s, (), None) for s in SOURCES]
    for d, paged, f16 in SLICES:
        jobs.append(("fwd_bf16_inst.hip", (f"FA_D={d}", f"FA_PAGED={paged}", f"FA_F16={f16}"),
                     f"fwd_bf16_inst_d{d}_p{paged}_h{f16}.o"))
    for f16 in BWD_ELEMS:
        jobs.append(("bwd_bf16.hip", (f"FA_BWD_F16={f16}",), f"bwd_bf16_h{f16}.o"))
    # the longest compiles first
    return sorted(jobs, key=lambda j: j[0] not in ("fwd_bf16_inst.hip", "bwd_bf16.hip"))


def build(jobs: int = 8, debug: bool = False, extra=()) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(lambda j: compile_one(j[0], debug, extra, j[1], j[2]), _jobs()))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"linking failed:\n{' '.join(cmd)}\n{res.stdout}{res.stderr}")
    os.replace(tmp, LIB)
    build_probe(debug)
    return LIB


def build_probe(debug: bool = False) -> str:
    """libfaprobe.so: the benchmark's matrix-core throughput probe."""
    os.makedirs(BUILD, exist_ok=True)
    obj = compile_one(PROBE_SRC, debug, ())
    tmp = PROBE_LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"linking failed:\n{' '.join(cmd)}\n{res.stdout}{res.stderr}")
    os.replace(tmp, PROBE_LIB)
    return PROBE_LIB


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--jobs", type=int, default=8)
    ap.add_argument("--debug", action="store_true")
    ap.add_argument("--save-temps", action="store_true",
                    help="keep the gfx950 assembly of our own kernels under _build/")
    args = ap.parse_args(argv)
    extra = []
    if args.save_temps:
        extra = ["-save-temps=obj"]
    print(build(args.jobs, args.debug, extra))


if __name__ == "__main__":
    main()
