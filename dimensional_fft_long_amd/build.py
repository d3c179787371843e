"""Build the gfx950 shared library ``libhyenand.so`` in-tree with hipcc.

Every HIP translation unit is compiled with packed-FP32 instruction selection
disabled (``-Xclang -target-feature -Xclang -packed-fp32-ops``).  The kernel
units (``csrc/k_*.hip``) compile in parallel.

    python -m dimensional_fft_long_amd.build [--incremental]

``--incremental`` recompiles only the units whose object is older than the
unit or one of the headers it included (hipcc dependency files); the default
compiles everything.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libhyenand.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# Kernel translation units (one per group of chains, compiled in parallel) and
# the C ABI.
SOURCES = sorted(f for f in os.listdir(CSRC) if f.startswith("k_") and f.endswith(".hip")) + ["api.cpp"]
FLAGS = ["-std=c++20", "-O3", f"--offload-arch={ARCH}", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include")]


def _obj(src: str) -> str:
    return os.path.join(BUILD, os.path.splitext(src)[0] + ".o")


def _up_to_date(src: str) -> bool:
    """True if the unit's object is newer than every file its dependency list names."""
    obj, dep = _obj(src), _obj(src)[:-2] + ".d"
    if not (os.path.exists(obj) and os.path.exists(dep)):
        return False
    t = os.path.getmtime(obj)
    text = open(dep).read().replace("\\\n", " ")
    files = [f for f in text.split(":", 1)[-1].split() if f]
    return all(os.path.exists(f) and os.path.getmtime(f) <= t for f in files)


def _compile(src: str) -> str:
    out = _obj(src)
    cmd = [HIPCC] + FLAGS + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", out,
                             "-MD", "-MF", out[:-2] + ".d"]
    t0 = time.time()
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    if os.environ.get("HYENAND_BUILD_TIMES"):
        print(f"  {src}: {time.time() - t0:.1f} s", file=sys.stderr)
    return out


def build(verbose: bool = True, incremental: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    todo = [s for s in SOURCES if not (incremental and _up_to_date(s))]
    with cf.ThreadPoolExecutor(max_workers=max(1, min(len(todo), os.cpu_count() or 1))) as ex:
        list(ex.map(_compile, todo))
    objs = [_obj(s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}"] + objs + ["-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} ({len(todo)} of {len(SOURCES)} units compiled)", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build(incremental="--incremental" in sys.argv[1:])
