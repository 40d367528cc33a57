"""Build libdsmoe.so (HIP, gfx950) in-tree.

Every HIP source under csrc/ is compiled by hipcc for gfx950 into _build/, then linked into
deepseek_gate_expert_amd/libdsmoe.so.  Flags: -O3, no floating-point contraction (the router
and gate reproduce a documented fp32 operation order), packed-fp32 instructions disabled.
"""
from __future__ import annotations

import glob
import hashlib
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libdsmoe.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function", "-I", os.path.join(ROOT, "include")]


STAMP = LIB + ".sha256"


def sources() -> list:
    """Every file the library is built from: the HIP sources, their headers and the C ABI header."""
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.hpp")) +
                  glob.glob(os.path.join(ROOT, "include", "*.h")))


def source_digest() -> str:
    """sha256 over the build flags and the contents of every source, in name order."""
    h = hashlib.sha256(" ".join(os.path.basename(f) if os.path.isabs(f) else f for f in FLAGS).encode())
    for f in sources():
        h.update(os.path.relpath(f, ROOT).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def is_current() -> bool:
    """True when libdsmoe.so exists and was built from the sources as they are now."""
    try:
        with open(STAMP) as fh:
            return os.path.exists(LIB) and fh.read().strip() == source_digest()
    except OSError:
        return False


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC] + FLAGS + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link libdsmoe.so.  Always recompiles."""
    os.makedirs(BUILD, exist_ok=True)
    digest = source_digest()
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    jobs = max(1, min(len(srcs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4))))
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    with open(STAMP, "w") as fh:
        fh.write(digest + "\n")
    if verbose:
        print(f"built {LIB}", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
