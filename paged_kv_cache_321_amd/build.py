"""Build libpa.so in-tree with hipcc for gfx950.

Usage: ``python -m paged_kv_cache_321_amd.build`` (always recompiles).
The library lands next to this file; it is what the binding loads.
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
LIB_PATH = os.path.join(HERE, "libpa.so")
ARCH = "gfx950"

SOURCES = ["pa_api.cpp", "pa_cache.hip", "pa_decode.hip", "pa_decode_valu.hip", "pa_multi_query.hip",
           "pa_decode_mfma.hip", "pa_noalloc.hip"]

# Packed-fp32 VALU ops are switched off for all device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# The multi-query kernel keeps its MFMA accumulators in ordinary VGPRs: with
# the accumulation registers the compiler copies them out and back around
# every loop iteration.
SOURCE_FLAGS = {"pa_multi_query.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}
COMMON_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
                "-I", INCLUDE, "-I", CSRC]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libpa.so)")


def _run(cmd):
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if proc.returncode != 0:
        raise RuntimeError("build step failed:\n" + " ".join(cmd) + "\n" + proc.stdout)
    return proc.stdout


def _compile_cmd(cc: str, src: str, obj: str):
    cmd = [cc, *COMMON_FLAGS]
    if src.endswith(".hip"):
        cmd += ["-x", "hip", *DEVICE_FLAGS, *SOURCE_FLAGS.get(src, [])]
    return cmd + ["-c", os.path.join(CSRC, src), "-o", obj]


def build_library(verbose: bool = False) -> str:
    """Compile every source (in parallel) and link libpa.so (atomically replaced)."""
    cc = hipcc()
    with tempfile.TemporaryDirectory(prefix="pa_build_") as tmp:
        objs = [os.path.join(tmp, src + ".o") for src in SOURCES]
        procs = [(src, subprocess.Popen(_compile_cmd(cc, src, obj), stdout=subprocess.PIPE,
                                        stderr=subprocess.STDOUT, text=True))
                 for src, obj in zip(SOURCES, objs)]
        failed = []
        for src, proc in procs:
            out, _ = proc.communicate()
            if proc.returncode != 0:
                failed.append(f"{src}:\n{out}")
            elif verbose and out.strip():
                print(out)
        if failed:
            raise RuntimeError("build failed:\n" + "\n".join(failed))
        tmp_lib = os.path.join(tmp, "libpa.so")
        _run([cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp_lib])
        staged = LIB_PATH + ".tmp"
        shutil.copyfile(tmp_lib, staged)
        os.replace(staged, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    path = build_library(verbose="-v" in sys.argv)
    print(path)
