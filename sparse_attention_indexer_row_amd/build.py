"""Builds the HIP selection library for gfx950 in-tree.

``python -m sparse_attention_indexer_row_amd.build`` compiles
``csrc/*.hip`` and ``csrc/*.cpp`` into ``libtopk_select.so`` next to this
file.  hipcc cross-compiles, so this works on a machine without a GPU.
Each source is compiled to an object of its own, in parallel, and the
objects are linked into the library (no relocatable device code: every
kernel is launched from the file that defines it).
"""

from __future__ import annotations

import concurrent.futures
import glob
import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB_PATH = os.path.join(HERE, "libtopk_select.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-result",
    # keep the compiler from forming packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def _jobs() -> int:
    try:
        n = int(os.environ.get("MAX_JOBS", "0"))
    except ValueError:
        n = 0
    return max(1, min(n or (os.cpu_count() or 1), 16))


def build(out: str = LIB_PATH, extra: list[str] | None = None, verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    srcs = sources()
    with tempfile.TemporaryDirectory(prefix="topk_build_") as tmpdir:
        objs = [os.path.join(tmpdir, os.path.basename(s) + ".o") for s in srcs]

        def compile_one(pair):
            src, obj = pair
            cmd = [hipcc, *HIPCC_FLAGS, *(extra or []), "-x", "hip", "-c", src, "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            subprocess.run(cmd, check=True)

        with concurrent.futures.ThreadPoolExecutor(max_workers=_jobs()) as ex:
            for f in [ex.submit(compile_one, p) for p in zip(srcs, objs)]:
                f.result()
        tmp = out + ".tmp"
        cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
