"""Builds libfattn.so (and the benchmark's probe library) in-tree with hipcc for gfx950.

    python io_aware_tiled_amd/build.py [-v]       # compile every source, link the libraries

It is a standalone script (it does not import the package, which needs the library to exist).

Objects go to io_aware_tiled_amd/_build/; the attention library to io_aware_tiled_amd/libfattn.so,
the measurement probes (matrix-core and HBM-read rates, used by bench.py only) to
io_aware_tiled_amd/libfattn_probe.so.
"""

from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_PATH = os.path.join(HERE, "libfattn.so")

SOURCES = ["api.cpp", "prefill_bf16.hip", "prefill_f32.hip", "decode_bf16.hip", "backward_bf16.hip",
           "noalloc.hip"]
PROBE_SOURCES = ["probe.hip"]
PROBE_LIB_PATH = os.path.join(HERE, "libfattn_probe.so")

ARCH = "gfx950"
COMMON = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # only what include/fattn.h declares is exported (the header switches visibility back on)
    "-fvisibility=hidden",
    "-Wall",
    "-Wno-unused-command-line-argument",
    # packed fp32 VALU forms are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE,
    "-I", CSRC,
]


def hipcc() -> str:
    return os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)


def _compile(sources, verbose, jobs):
    objs, cmds = [], []
    for src in sources:
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmds.append([hipcc()] + COMMON + lang + ["-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    with concurrent.futures.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        for f in [ex.submit(_run, c, verbose) for c in cmds]:
            f.result()
    return objs


def _link(objs, path, verbose):
    tmp = path + ".tmp"
    # --no-undefined: a kernel whose host-side launch stub was not emitted fails here, not at load
    _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,--no-undefined", "-o", tmp]
         + objs, verbose)
    os.replace(tmp, path)


def build(verbose: bool = False, jobs: int = 4) -> str:
    """Compile all sources and link libfattn.so and libfattn_probe.so; returns libfattn's path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = _compile(SOURCES + PROBE_SOURCES, verbose, jobs)
    _link(objs[:len(SOURCES)], LIB_PATH, verbose)
    _link(objs[len(SOURCES):], PROBE_LIB_PATH, verbose)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
