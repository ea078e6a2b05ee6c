"""Build libmxq.so (the HIP library behind include/mxq.h) for gfx950, in-tree.

    python -m mxfp4_microscaling_quantization_mxq_amd.build
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmxq.so")
# measurement kernels (on-box ceilings), a library of their own that only
# the benchmark loads
CEILING_SRC = os.path.join(PKG, "ceiling", "ceilings.hip")
CEILING_LIB = os.path.join(PKG, "libmxq_ceiling.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -packed-fp32-ops: no v_pk_{add,mul,fma}_f32 in generated code.
# -ffp-contract=off: every fp32 operation rounds once, as the quantizers assume.
CFLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fvisibility=hidden", "-Wall", "-Wno-unused-function",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    procs = []
    objs = []
    ceiling_tmp = CEILING_LIB + ".tmp"
    procs.append((CEILING_SRC, subprocess.Popen([HIPCC, *CFLAGS, "-shared", CEILING_SRC, "-o", ceiling_tmp],
                                                stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    for src in sources():
        obj = os.path.join(BUILD, os.path.basename(src) + ".o")
        objs.append(obj)
        cmd = [HIPCC, *CFLAGS, "-I", os.path.join(ROOT, "include"), "-c", src, "-o", obj]
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = False
    for src, p in procs:
        out, _ = p.communicate()
        text = "\n".join(
            ln for ln in out.decode(errors="replace").splitlines() if "not a recognized feature" not in ln
        )
        if p.returncode != 0:
            failed = True
            sys.stderr.write(f"hipcc failed on {src}:\n{text}\n")
        elif verbose and text.strip():
            sys.stderr.write(text + "\n")
    if failed:
        raise RuntimeError("HIP compilation failed")
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    os.replace(ceiling_tmp, CEILING_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
