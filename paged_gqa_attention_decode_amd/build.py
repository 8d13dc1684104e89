"""Build libpaged_attn.so, and its checked variant libpaged_attn_checked.so, from csrc/*.hip
with hipcc for gfx950; and libpaged_attn_probes.so, the measurement kernels of bench.py
(csrc/probes.hip), which is not part of the attention library.

    python -m paged_gqa_attention_decode_amd.build

Each translation unit compiles separately (in parallel) to an object under _build/ (the
checked variant, with -DPAGED_ATTN_CHECKED, under _build_checked/), then hipcc links the
shared library next to this file.  Packed-FP32 instructions are disabled
(-target-feature -packed-fp32-ops); all arithmetic is ordinary f32.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libpaged_attn.so")
BUILD_CHECKED = os.path.join(HERE, "_build_checked")
LIB_CHECKED = os.path.join(HERE, "libpaged_attn_checked.so")
LIB_PROBES = os.path.join(HERE, "libpaged_attn_probes.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
SOURCES = ["api.hip", "decode.hip", "combine.hip", "prefill.hip", "kv_write.hip",
           "kv_write_rope.hip", "noalloc.hip"]
FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _compile(src: str, extra=(), build_dir=None) -> str:
    obj = os.path.join(build_dir or BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + FLAGS + list(extra) + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, extra_flags=(), checked: bool = False) -> str:
    """Compile every source and link libpaged_attn.so (or, with checked=True,
    libpaged_attn_checked.so); returns its path."""
    build_dir, lib = (BUILD_CHECKED, LIB_CHECKED) if checked else (BUILD, LIB)
    flags = tuple(extra_flags) + (("-DPAGED_ATTN_CHECKED",) if checked else ())
    os.makedirs(build_dir, exist_ok=True)
    jobs = min(len(SOURCES), max(1, (os.cpu_count() or 4)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, flags, build_dir), SOURCES))
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


def build_probes(verbose: bool = False) -> str:
    """libpaged_attn_probes.so from csrc/probes.hip (one translation unit, linked directly)."""
    tmp = LIB_PROBES + ".tmp%d" % os.getpid()
    cmd = [HIPCC] + FLAGS + ["-shared", os.path.join(CSRC, "probes.hip"), "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for probes.hip:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB_PROBES)
    if verbose:
        print(f"built {LIB_PROBES}")
    return LIB_PROBES


def build_all(verbose: bool = False):
    """The libraries, the product, its checked variant and the probes, built concurrently."""
    with cf.ThreadPoolExecutor(3) as ex:
        product = ex.submit(build, verbose)
        checked = ex.submit(build, verbose, (), True)
        probes = ex.submit(build_probes, verbose)
        return product.result(), checked.result(), probes.result()


if __name__ == "__main__":
    build_all(verbose=True)
    sys.exit(0)
