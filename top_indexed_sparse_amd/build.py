"""Build libtopidx.so (all HIP kernels + the C ABI) for gfx950 with hipcc, in the package dir.

    python -m top_indexed_sparse_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libtopidx.so")
SOURCES = ["api.hip", "indexer.hip", "topk.hip", "attn.hip", "append.hip", "blocks.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for c in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libtopidx)")


# Per-file code-generation options.  The scorer's matrix products write ordinary vector
# registers (its epilogue reads every result at once; results in accumulator registers would
# each be copied out first); the attention kernel keeps its accumulators where the compiler
# puts them.
FILE_FLAGS = {"indexer.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _common() -> list[str]:
    return [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
            "-fvisibility=hidden",
            # packed fp32 VALU forms are kept out of the generated code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def compile_command(src: str, obj: str) -> list[str]:
    """One source file to an object holding its host code and gfx950 code object."""
    return _common() + FILE_FLAGS.get(src, []) + ["-c", "-o", obj, os.path.join(CSRC, src)]


def link_command(objs: list[str], out: str) -> list[str]:
    return [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", out] + objs


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "packed-fp32-ops"  # the host pass does not know the device-only feature
    msgs = [l for l in (r.stdout + r.stderr).splitlines() if l.strip() and noise not in l]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))


def build_library(verbose: bool = False) -> str:
    """Compile every source (in parallel, one hipcc per file) and link libtopidx.so."""
    from concurrent.futures import ThreadPoolExecutor
    import tempfile
    with tempfile.TemporaryDirectory(prefix="topidx_build_") as d:
        objs = [os.path.join(d, os.path.splitext(s)[0] + ".o") for s in SOURCES]
        with ThreadPoolExecutor(max_workers=min(len(SOURCES), 8)) as ex:
            list(ex.map(lambda a: _run(compile_command(*a), verbose), zip(SOURCES, objs)))
        tmp = LIB + ".tmp"
        _run(link_command(objs, tmp), verbose)
        os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_library(verbose="-v" in sys.argv))
