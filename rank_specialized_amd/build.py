"""Build the HIP library in-tree: rank_specialized_amd/librank_specialized.so.

    python -m rank_specialized_amd.build          # gfx950, -O3

Every source is compiled with hipcc for gfx950 only, with packed-FP32
instructions disabled, then linked into one shared library.  The benchmark's
bandwidth references (a plain copy and a plain read) go into a library of
their own, libstream_ref.so, apart from the LoRA library.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
OUT = os.path.join(HERE, "librank_specialized.so")
REF_OUT = os.path.join(HERE, "libstream_ref.so")
REF_SOURCES = ["stream_ref.hip"]
BUILD_DIR = os.path.join(HERE, "_build")
ARCH = os.environ.get("LORA_OFFLOAD_ARCH", "gfx950")

SOURCES = ["api.hip", "pack.hip", "segment.hip", "group.hip", "shrink.hip", "expand.hip", "decode.hip", "jd.hip", "rsvd.hip", "multi.hip", "fused.hip", "validate.cpp", "ranks.cpp"]

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
          f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}"]
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-munsafe-fp-atomics"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm install expected under /opt/rocm)")


def _compile(src: str, extra) -> str:
    obj = os.path.join(BUILD_DIR, src + ".o")
    path = os.path.join(CSRC, src)
    if src.endswith(".hip"):
        cmd = [hipcc(), *COMMON, *DEVICE, *extra, "-c", path, "-o", obj]
    else:
        cmd = [hipcc(), *COMMON, "-x", "c++", *extra, "-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, out: str) -> None:
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = False, extra=()) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = SOURCES + REF_SOURCES
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, list(extra)), srcs))
    _link(objs[: len(SOURCES)], OUT)
    _link(objs[len(SOURCES):], REF_OUT)
    if verbose:
        print(f"built {OUT}")
        print(f"built {REF_OUT}")
    return OUT


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
