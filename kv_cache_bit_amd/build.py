"""Build libnsnq.so (HIP, gfx950) in-tree with hipcc.

    python -m kv_cache_bit_amd.build

Each source compiles to an object of its own, in parallel; the objects are
then linked into the shared library.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libnsnq.so")
OBJ_DIR = os.path.join(HERE, "_build")

# -packed-fp32-ops: keep the compiler from emitting v_pk_{add,mul,fma}_f32.
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results straight into VGPRs: the argmin reads every accumulator
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-function",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _clean(stderr: str) -> str:
    # hipcc's host pass does not know the packed-fp32 feature and says so; drop that line
    return "\n".join(l for l in stderr.splitlines() if "packed-fp32-ops" not in l)


def build(verbose: bool = False, jobs: int | None = None) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    os.makedirs(OBJ_DIR, exist_ok=True)
    srcs = sources()
    objs = [os.path.join(OBJ_DIR, os.path.basename(s)[:-4] + ".o") for s in srcs]

    def compile_one(pair):
        src, obj = pair
        cmd = [hipcc, *HIPCC_FLAGS, "-c", "-o", obj, src]
        if verbose:
            print(" ".join(cmd), flush=True)
        return src, subprocess.run(cmd, capture_output=True, text=True)

    jobs = jobs or min(len(srcs), os.cpu_count() or 1, 8)
    with ThreadPoolExecutor(max_workers=jobs) as pool:
        results = list(pool.map(compile_one, zip(srcs, objs)))
    failed = [(src, res) for src, res in results if res.returncode != 0]
    if failed:
        raise RuntimeError("hipcc failed:\n" + "\n".join(f"{src}:\n{_clean(res.stderr)}" for src, res in failed))
    if verbose:
        for src, res in results:
            if _clean(res.stderr).strip():
                print(_clean(res.stderr), file=sys.stderr)
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + _clean(res.stderr))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
