"""Builds libgdn.so in-tree with hipcc for gfx950.

    python -m linear_attention_recurrence_delta_amd.build

Always recompiles. The library lands next to this file, where the binding
loads it from.
"""
import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBRARY = os.path.join(HERE, "libgdn.so")
SOURCES = ["gdn_api.cpp", "gdn_prefill.hip", "gdn_decode.hip", "gdn_backward.hip", "gdn_noalloc.hip"]
ARCH = "gfx950"

# Packed-fp32 instructions are disabled for all device code. MFMA results
# are kept in ordinary VGPRs (the accumulation-register form makes the
# compiler shuffle accumulator arrays through v_accvgpr moves every loop).
# The atomic optimizer is off: the gradient kernel's LDS atomics are issued
# by one lane per already-reduced row, and the optimizer would wrap each in
# a wave-wide scan.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-mllvm", "-amdgpu-mfma-vgpr-form",
                "-mllvm", "-amdgpu-atomic-optimizer-strategy=None"]


def hipcc():
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found")
    return path


def build_library(verbose=False):
    """Compile every source and link libgdn.so; returns its path."""
    with tempfile.TemporaryDirectory(prefix="gdn_build_") as tmp:
        objs = []
        procs = []
        for src in SOURCES:
            obj = os.path.join(tmp, src + ".o")
            cmd = [hipcc(), "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
                   "-Wall", "-Wno-unused-command-line-argument",
                   "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj]
            if src.endswith(".hip"):
                cmd[1:1] = ["-x", "hip"] + DEVICE_FLAGS
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                                stderr=subprocess.STDOUT, text=True)))
            objs.append(obj)
        failed = []
        for src, p in procs:
            out, _ = p.communicate()
            if out and (verbose or p.returncode):
                print(out, file=sys.stderr)
            if p.returncode:
                failed.append(src)
        if failed:
            raise RuntimeError("hipcc failed for " + ", ".join(failed))
        tmp_lib = LIBRARY + ".tmp"
        cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp_lib] + objs
        subprocess.run(cmd, check=True)
        os.replace(tmp_lib, LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    print(build_library(verbose="-v" in sys.argv))
