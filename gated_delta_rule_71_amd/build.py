"""Build libgdr.so (gfx950) in-tree with hipcc.

Every source is compiled for gfx950 only, with packed fp32 instructions turned
off (-Xclang -target-feature -Xclang -packed-fp32-ops), then linked into one
shared library next to this file.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(HERE, "libgdr.so")
SOURCES = ["gdr_api.cpp", "prefill.hip", "prefill64.hip", "decode.hip", "conv_norm.hip",
           "backward.hip", "segments.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libgdr.so")


def compile_flags():
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", INCLUDE, "-I", CSRC]


def build(out_path: str = LIB_PATH, verbose: bool = False) -> str:
    cc = hipcc()
    with tempfile.TemporaryDirectory(prefix="gdr_build_") as tmp:
        procs = []
        objs = []
        for src in SOURCES:
            obj = os.path.join(tmp, src + ".o")
            objs.append(obj)
            cmd = [cc, *compile_flags(), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                                stderr=subprocess.STDOUT, text=True)))
        failed = []
        for src, pr in procs:
            out, _ = pr.communicate()
            if out and (verbose or pr.returncode):
                print(out, file=sys.stderr)
            if pr.returncode:
                failed.append(src)
        if failed:
            raise RuntimeError(f"hipcc failed for {failed}")
        tmp_out = out_path + ".tmp"
        link = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp_out]
        subprocess.run(link, check=True)
        os.replace(tmp_out, out_path)
    return out_path


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
