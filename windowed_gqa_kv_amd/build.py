"""Build libgqa_mi355x.so from csrc/ with hipcc for gfx950.

Usage: python -m windowed_gqa_kv_amd.build [--jobs N] [--verbose]

Each .hip file is compiled to an object in _build/ (repository root) in
parallel, then linked into windowed_gqa_kv_amd/libgqa_mi355x.so.  Always
recompiles: the caller asks for a build, it gets one.
"""

from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libgqa_mi355x.so")

ARCH = "gfx950"
CXXFLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    f"--offload-arch={ARCH}",
    "-Wall", "-Wno-unused-function",
    # no packed-fp32 VALU ops anywhere
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


# Per-source flags: MFMA results in VGPRs.  Both kernels keep their output
# accumulators in VGPRs across tiles / units (the lazy rescale multiplies
# them on the vector ALU); with the MFMA results in AGPRs the compiler copied
# them to AGPRs around every P V step (the decode: 32 copies and their wait
# states per unit at head size 128; the head-size-256 prefill: 500-650 copies
# each way in a kernel body, and its additive-mask instances spilled).  gfx950
# MFMAs read and write VGPRs directly; AGPRs are still used where a kernel
# needs more than 256 registers (the head-size-256 prefill).
FILE_FLAGS = {
    "decode_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "prefill_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libgqa_mi355x)")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(cc, src, verbose):
    obj = os.path.join(BUILD, os.path.basename(src)[:-4] + ".o")
    cmd = [cc, *CXXFLAGS, *FILE_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in l)  # host pass does not know the feature
    return src, obj, r.returncode, msgs


def build(jobs: int | None = None, verbose: bool = False) -> str:
    cc = hipcc()
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    objs = []
    errors = []
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        for src, obj, rc, msgs in ex.map(lambda s: _compile(cc, s, verbose), srcs):
            if msgs.strip():
                print(msgs, file=sys.stderr)
            if rc != 0:
                errors.append(src)
            objs.append(obj)
    if errors:
        raise RuntimeError("hipcc failed for: " + ", ".join(os.path.basename(e) for e in errors))
    tmp = LIB + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("--verbose", action="store_true")
    args = ap.parse_args(argv)
    print(build(args.jobs, args.verbose))


if __name__ == "__main__":
    main()
