"""Build libkq.so for gfx950 in-tree: ``python -m gguf_quant_matmul_amd.build``.

Compiles every ``csrc/*.hip`` with hipcc (one process per file, in parallel)
and links them into ``gguf_quant_matmul_amd/libkq.so``.
"""

from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libkq.so")
ARCH = os.environ.get("KQ_OFFLOAD_ARCH", "gfx950")

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

FLAGS = [
    "-O3",
    "-std=c++17",
    "-fPIC",
    f"--offload-arch={ARCH}",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    # no packed-fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(line for line in (res.stdout + res.stderr).splitlines() if "packed-fp32-ops" not in line)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{out}")
    if verbose and out.strip():
        print(out)
    return obj


def _stale(src: str) -> bool:
    """True if src's object is missing or older than src or any header of csrc/."""
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    if not os.path.exists(obj):
        return True
    newest = max([os.path.getmtime(src)] + [os.path.getmtime(h) for h in glob.glob(os.path.join(CSRC, "*.h"))])
    return os.path.getmtime(obj) < newest


def build(verbose: bool = False, incremental: bool = False) -> str:
    """Compile every source and link libkq.so; with incremental=True only the
    sources whose object is older than the source or a header are compiled."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    todo = [s for s in srcs if _stale(s)] if incremental else srcs
    workers = max(1, min(len(todo), int(os.environ.get("MAX_JOBS", "8")), 16))
    with cf.ThreadPoolExecutor(max_workers=workers) as ex:
        list(ex.map(lambda s: _compile(s, verbose), todo))
    objs = [os.path.join(BUILD, os.path.basename(s) + ".o") for s in srcs]
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True, incremental="--incremental" in sys.argv)
    sys.exit(0)
