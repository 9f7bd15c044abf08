"""Build the HIP libraries in-tree with hipcc for gfx950.

    python -m bit_flashattention_hifa4_amd.build

produces ``libhifa4.so`` (the attention library, C ABI in include/hifa4.h) and
``libhifa4_probes.so`` (instruction probes, include/hifa4_probes.h) next to
this file.  Objects go to ``_build/`` at the repository root.
"""
from __future__ import annotations

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

LIB = os.path.join(PKG, "libhifa4.so")
PROBES_LIB = os.path.join(PKG, "libhifa4_probes.so")

LIB_SOURCES = ["api.cpp", "quantize.hip", "attn_mxfp4.hip", "attn_bf16.hip", "scratch.hip"]
PROBE_SOURCES = ["probes.hip"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP libraries cannot be built")


def flags() -> list[str]:
    return [
        "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
        # packed fp32 VALU forms are kept out of the generated code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # IEEE fp32 division (the key smoothing divides)
        "-fhip-fp32-correctly-rounded-divide-sqrt",
        # Code placement.  The interleaved prefill step's loop ran at speeds
        # that depended on where its instructions sat relative to 16-byte
        # boundaries (69 to 82 us on a Qwen3-8B-shaped d = 128 layer for the
        # same instructions).  Branch targets that are never fallen into start
        # on a 16-byte boundary, and every loop header on a 64-byte one; the
        # loop itself then places its body (see the prefill kernel),
        # independent of the code before it.
        "-mllvm", "-align-all-nofallthru-blocks=4",
        "-falign-loops=64",
        "-Wall", "-Wno-unused-function",
        "-I", INCLUDE, "-I", CSRC,
    ]


def _existing(sources):
    return [s for s in sources if os.path.exists(os.path.join(CSRC, s))]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc()] + flags() + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed on %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return obj


def _link(objs: list[str], out: str) -> None:
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, out)


def build(verbose: bool = False) -> list[str]:
    """Compile every HIP source and link both libraries (always rebuilds)."""
    os.makedirs(BUILD, exist_ok=True)
    lib_src = _existing(LIB_SOURCES)
    probe_src = _existing(PROBE_SOURCES)
    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = dict(zip(lib_src + probe_src, ex.map(_compile, lib_src + probe_src)))
    _link([objs[s] for s in lib_src], LIB)
    _link([objs[s] for s in probe_src], PROBES_LIB)
    if verbose:
        print("built", LIB, PROBES_LIB)
    return [LIB, PROBES_LIB]


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
