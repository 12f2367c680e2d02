"""Build libbd.so (the gfx950 HIP kernels + C ABI) in-tree with hipcc.

    python -m block_diffusion_decoding_amd.build

Every .hip file under csrc/ is compiled for gfx950 into _build/, then linked
into block_diffusion_decoding_amd/libbd.so.  Packed fp32 instructions are
disabled for every file (-packed-fp32-ops).  BD_DEFINES (environment) adds
-D options that override the kernels' tuning constants.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
ROOT = os.path.dirname(PKG)
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libbd.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-result",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I" + os.path.join(ROOT, "include")]
# tuning constants of the kernels (e.g. "-DBD_LM_WIDE_PF=3"); only -D options are taken
FLAGS += [f for f in os.environ.get("BD_DEFINES", "").split() if f.startswith("-D")]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature; that warning is noise
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{err}")
    return err


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
    objs = [os.path.join(BUILD, f[:-4] + ".o") for f in srcs]

    def compile_one(i):
        return _run([HIPCC, *FLAGS, "-c", os.path.join(CSRC, srcs[i]), "-o", objs[i]])

    with ThreadPoolExecutor(min(8, len(srcs))) as ex:
        logs = list(ex.map(compile_one, range(len(srcs))))
    tmp = LIB + ".tmp"
    logs.append(_run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]))
    os.replace(tmp, LIB)
    if verbose:
        for l in logs:
            if l.strip():
                print(l, file=sys.stderr)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
