"""Build librdt.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

Objects go to _build/ at the repository root; the shared library lands next
to this file, where the binding loads it.  Every call recompiles.
"""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "librdt.so")
BUILD = os.path.join(ROOT, "_build")
SOURCES = ["runtime.cpp", "gemm.hip", "gemm_big.hip", "gemm_skinny.hip", "attention.hip", "rowwise.hip",
           "backward.hip", "optimizer.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include")]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the packed-fp32 feature flag; drop that note
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    return r.returncode, out


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(BUILD, src + ".o")
        cmd = [HIPCC] + FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]
        if src.endswith(".cpp"):
            cmd = [HIPCC] + FLAGS + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
        rc, out = _run(cmd)
        return src, obj, rc, out

    with ThreadPoolExecutor(len(SOURCES)) as ex:
        results = list(ex.map(compile_one, SOURCES))
    for src, obj, rc, out in results:
        if out.strip() and (verbose or rc):
            print(f"[{src}]\n{out}", file=sys.stderr)
        if rc:
            raise RuntimeError(f"hipcc failed on {src}")
    tmp = OUT + ".tmp"
    rc, out = _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Wl,--no-undefined", "-o", tmp]
                   + [r[1] for r in results])
    if rc:
        print(out, file=sys.stderr)
        raise RuntimeError("link of librdt.so failed")
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
