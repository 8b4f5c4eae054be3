"""Build the HIP library ``libkivi.so`` in-tree for gfx950 with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libkivi.so")
SOURCES = ["kivi_api.cpp", "kivi_append.hip", "kivi_decode.hip", "kivi_prefill.hip", "kivi_fp8.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # keep the compiler from emitting packed fp32 math
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def build(verbose: bool = False, jobs: int = 0) -> str:
    """Compile every source (in parallel, `jobs` processes; 0 = one per source, at most
    8) and link libkivi.so."""
    from concurrent.futures import ThreadPoolExecutor
    os.makedirs(os.path.join(HERE, "_build"), exist_ok=True)
    cmds, objs = [], []
    for src in SOURCES:
        obj = os.path.join(HERE, "_build", os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmds.append([HIPCC, *FLAGS, "-I", os.path.join(ROOT, "include"), "-I", CSRC, *lang,
                     "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    if verbose:
        for cmd in cmds:
            print(" ".join(cmd), flush=True)
    with ThreadPoolExecutor(jobs or min(8, len(cmds))) as ex:
        for f in [ex.submit(subprocess.check_call, cmd) for cmd in cmds]:
            f.result()
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
