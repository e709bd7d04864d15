"""Build libkda.so (the HIP kernels + C ABI) in-tree for gfx950 with hipcc.

    python -m gated_delta_rule_18_amd.build [-v]

Every HIP source is compiled with packed-fp32 instruction selection disabled
(the -packed-fp32-ops target feature); hipcc's host pass warns that it does
not know the feature, which is harmless.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libkda.so")
BUILD_DIR = os.path.join(ROOT, "_build")
ARCH = "gfx950"

SOURCES = ["kda_prefill_ws.hip", "kda_decode.hip", "kda_prep.hip", "kda_gate.hip",
           "kda_bwd.hip", "kda_validate.hip", "kda_api.cpp"]
COMMON = ["-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}", "-I", CSRC, "-I", INCLUDE,
          "-Wall", "-Wno-unused-command-line-argument",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.sep not in cand or os.path.exists(cand)):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src, verbose):
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else ["-x", "hip"]
    cmd = [_hipcc(), *COMMON, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(line for line in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msgs}")
    if msgs.strip() and verbose:
        print(msgs)
    return obj


def build(verbose=False):
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
