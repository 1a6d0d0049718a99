"""Build libhisa.so in-tree with hipcc for gfx950.

    python -m long_context_sparse_hisa_amd.build

Every HIP source is compiled to an object of its own (in parallel), then
the objects are linked into the shared library.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libhisa.so")

COMPILE_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
    # no packed-fp32 instructions in any kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]
LINK_FLAGS = ["-shared", "-fPIC", "--offload-arch=gfx950"]


def sources():
    return sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))


def _filter(text):
    return "\n".join(l for l in text.splitlines() if "packed-fp32-ops' is not a recognized feature" not in l)


def build(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "hipcc")
    srcs = sources()
    with tempfile.TemporaryDirectory(prefix="hisa_build_") as tmpdir:
        objs = [os.path.join(tmpdir, os.path.basename(s) + ".o") for s in srcs]

        def compile_one(pair):
            src, obj = pair
            cmd = [hipcc] + COMPILE_FLAGS + ["-I", os.path.join(ROOT, "include"), "-c", src, "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            res = subprocess.run(cmd, capture_output=True, text=True)
            return src, res.returncode, _filter(res.stdout + res.stderr)

        jobs = max(1, min(len(srcs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4))))
        with ThreadPoolExecutor(jobs) as ex:
            results = list(ex.map(compile_one, zip(srcs, objs)))
        failed = [(s, out) for s, rc, out in results if rc != 0]
        if failed:
            raise RuntimeError("hipcc failed:\n" + "\n".join("%s:\n%s" % f for f in failed))
        if verbose:
            for s, _, out in results:
                if out.strip():
                    print(out)
        tmp = LIB + ".tmp%d" % os.getpid()
        cmd = [hipcc] + LINK_FLAGS + ["-o", tmp] + objs
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError("link failed:\n" + _filter(res.stdout + res.stderr))
        os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
