"""Build of the gfx950 HIP library ``libmgs.so`` (in-tree, next to this file).

The library is compiled with hipcc for gfx950 only, with FP contraction off (the recompute path
regenerates the forward's quantized activation bit for bit, so a functor must round the same way in
every kernel that inlines it) and with packed FP32 instructions disabled.
"""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_PATH = os.path.join(HERE, "libmgs.so")
SOURCES = ["mgs_api.hip", "act_quant.hip", "gemm_mx.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-function",
]


def _run(cmd):
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in res.stdout.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError("command failed: %s\n%s" % (" ".join(cmd), out))
    return out


def build(verbose=False):
    """Compile every HIP source and link libmgs.so; returns the library path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = [os.path.join(BUILD_DIR, s.replace(".hip", ".o")) for s in SOURCES]

    def compile_one(i):
        return _run([HIPCC, *FLAGS, "-c", os.path.join(CSRC, SOURCES[i]), "-o", objs[i]])

    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        logs = list(ex.map(compile_one, range(len(SOURCES))))
    tmp = LIB_PATH + ".tmp"
    logs.append(_run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]))
    os.replace(tmp, LIB_PATH)
    if verbose:
        for l in logs:
            if l.strip():
                print(l)
        print("built", LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
