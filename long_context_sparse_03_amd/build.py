"""Build libcsa.so (the gfx950 kernels and the C ABI) in-tree with hipcc.

Every source compiles to its own object in parallel (each kernel is launched
from the file that defines it, so no relocatable device code is needed), and
the objects are linked into one shared library."""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libcsa.so")
SOURCES = ["abi.hip", "compress.hip", "append.hip", "index.hip", "topk.hip", "attention.hip", "prefix.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # keep the compiler from forming packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]


def _clean(stderr: str) -> str:
    return "\n".join(l for l in stderr.splitlines() if "packed-fp32-ops" not in l)


def build(verbose: bool = False) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    with tempfile.TemporaryDirectory(prefix="csa_build_") as tmpd:
        def compile_one(src):
            obj = os.path.join(tmpd, os.path.basename(src) + ".o")
            cmd = [HIPCC] + FLAGS + ["-I", os.path.join(ROOT, "include"), "-c", src, "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            return obj, subprocess.run(cmd, capture_output=True, text=True)

        jobs = min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
        with ThreadPoolExecutor(jobs) as ex:
            results = list(ex.map(compile_one, srcs))
        errs = [(o, r) for o, r in results if r.returncode != 0]
        if errs:
            raise RuntimeError("hipcc failed:\n" + "\n".join(_clean(r.stderr) for _, r in errs))
        if verbose:
            for _, r in results:
                if _clean(r.stderr).strip():
                    print(_clean(r.stderr), file=sys.stderr)
        tmp = LIB + ".tmp%d" % os.getpid()
        cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + [o for o, _ in results] + ["-o", tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError("hipcc link failed:\n" + _clean(res.stderr))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
