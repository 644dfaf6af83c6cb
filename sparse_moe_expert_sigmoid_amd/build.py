"""Build the HIP library (gfx950) in-tree.

    python -m sparse_moe_expert_sigmoid_amd.build

Compiles every csrc/*.hip (device code, hipcc; cross-compiles without a GPU)
and csrc/*.cc (host-only argument checks, the host compiler through hipcc)
into libmoe_mi355x.so beside this file.  Packed fp32 VALU ops are disabled
for the device code.  Always recompiles.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libmoe_mi355x.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

DEVICE_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
                "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra"]


def _compile(src: str, obj: str, verbose: bool) -> None:
    if src.endswith(".cc"):
        cmd = [HIPCC, *HOST_FLAGS, "-c", src, "-o", obj]
    else:
        cmd = [HIPCC, *DEVICE_FLAGS, "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)


def build(verbose: bool = False) -> str:
    srcs = sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")) +
                  glob.glob(os.path.join(HERE, "csrc", "*.cc")))
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = []
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        futs = []
        for s in srcs:
            o = os.path.join(objdir, os.path.basename(s) + ".o")
            objs.append(o)
            futs.append(ex.submit(_compile, s, o, verbose))
        for f in futs:
            f.result()
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
