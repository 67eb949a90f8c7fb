"""Builds libkda.so (the C-ABI library) for gfx950 with hipcc.

Usage: python -m kda_chunked_amd.build [-v]
Every HIP source is compiled for --offload-arch=gfx950 only, with packed FP32
instructions disabled, into kda_chunked_amd/libkda.so.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJ = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libkda.so")

SOURCES = ["kda_api.cpp", "kda_prep.hip", "kda_scan.hip", "kda_bwd_intra.hip",
           "kda_noalloc.hip", "conv_silu.hip", "kda_walk.hip", "attn.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def _compile(src: str, verbose: bool, extra=(), objdir=OBJ) -> str:
    out = os.path.join(objdir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", out]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed on {src}")
    noise = "warning: unknown target feature"  # host pass ignores the GPU-only feature flag
    msg = "\n".join(x for x in (r.stdout + r.stderr).splitlines() if x and noise not in x
                    and "packed-fp32-ops" not in x)
    if msg.strip() and verbose:
        sys.stderr.write(msg + "\n")
    return out


def build(verbose: bool = False, extra=(), out: str = LIB, objdir: str = OBJ) -> str:
    """Compile and link the library. `extra` adds compiler flags (for example
    -DKDA_SPLIT_KS=SPLIT_B to change a product's split terms); `out` and
    `objdir` place a variant build elsewhere."""
    os.makedirs(objdir, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), 8)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, extra, objdir), SOURCES))
    tmp = out + f".tmp{os.getpid()}"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
