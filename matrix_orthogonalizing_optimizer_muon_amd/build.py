"""Builds libmuon_mi355x.so in-tree for gfx950 (hipcc cross-compiles; no GPU needed).

Usage: python -m matrix_orthogonalizing_optimizer_muon_amd.build  [--verbose]
"""
import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
LIB_NAME = "libmuon_mi355x.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)

ARCH = "gfx950"
HIP_FLAGS = ["-O3", f"--offload-arch={ARCH}", "-std=c++17", "-fPIC",
             # packed fp32 instructions are kept out of every kernel
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-command-line-argument", f"-I{INCLUDE}", f"-I{CSRC}"]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", f"-I{INCLUDE}", f"-I{CSRC}"]


def _hipcc():
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"build step failed: {' '.join(cmd[:2])} ... ({r.returncode})")
    return r


def build(verbose: bool = False) -> str:
    hipcc = _hipcc()
    with tempfile.TemporaryDirectory(prefix="muon_build_") as tmp:
        objs = []
        for src, kind in (("kernels.hip", "hip"), ("probe.hip", "hip"), ("noalloc.hip", "hip"), ("abi.cpp", "hip"),
                          ("plan.cpp", "host"), ("assign.cpp", "host")):
            obj = os.path.join(tmp, src + ".o")
            path = os.path.join(CSRC, src)
            if kind == "hip":
                cmd = [hipcc, *HIP_FLAGS, "-x", "hip", "-c", path, "-o", obj]
            else:
                cmd = ["g++", *HOST_FLAGS, "-c", path, "-o", obj]
            _run(cmd, verbose)
            objs.append(obj)
        out_tmp = os.path.join(tmp, LIB_NAME)
        _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", out_tmp], verbose)
        shutil.copyfile(out_tmp, LIB_PATH + ".tmp")
        os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
