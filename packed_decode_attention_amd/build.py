"""Build the HIP library libtq.so in-tree for gfx950.

    python -m packed_decode_attention_amd.build            # or: python packed_decode_attention_amd/build.py

hipcc cross-compiles the device code for gfx950 without a GPU present.  Packed-fp32 VALU
instructions are disabled for all device code (-packed-fp32-ops).  The decode kernels take
finite inputs by contract and are built with -fno-honor-nans, which lets the running-maximum
reductions fold into single DPP max instructions.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libtq.so")
ARCH = os.environ.get("TQ_OFFLOAD_ARCH", "gfx950")

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
DEVICE_FLAGS = ["-O3", "-fPIC", "-std=c++17", "-fno-strict-aliasing", f"--offload-arch={ARCH}",
                "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-Wall", "-Wno-unused-function"]
HOST_FLAGS = ["-O2", "-fPIC", "-std=c++17", "-Wall"]

SOURCES = [
    # MFMA results straight into VGPRs (no accumulation-register round trip; the quantizer's
    # products are one-shot, never accumulated across instructions)
    ("tq_quantize.hip", "device", ["-fno-honor-nans", "-mllvm", "-amdgpu-mfma-vgpr-form=1"]),
    ("tq_decode.hip", "device", ["-fno-honor-nans"]),
    ("tq_decode_block.hip", "device", ["-fno-honor-nans"]),
    ("tq_probe.hip", "device", []),  # diagnostics (include/tq_probe.h)
    ("tq_api.cpp", "host", []),
    ("tq_codebook.cpp", "host", []),
]


def _run(cmd):
    print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    objs, procs = [], []
    for src, kind, extra in SOURCES:  # compile every source in parallel
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        path = os.path.join(CSRC, src)
        if kind == "device":
            cmd = [HIPCC, *DEVICE_FLAGS, *extra, "-c", path, "-o", obj]
        else:
            cmd = ["g++", *HOST_FLAGS, *extra, "-c", path, "-o", obj]
        print(" ".join(cmd), flush=True)
        procs.append((cmd, subprocess.Popen(cmd)))
        objs.append(obj)
    for cmd, p in procs:
        if p.wait() != 0:
            raise subprocess.CalledProcessError(p.returncode, cmd)
    tmp = LIB + ".tmp"
    _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
