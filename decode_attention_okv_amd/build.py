"""Build libokv.so (HIP, gfx950) in-tree with hipcc.

    python -m decode_attention_okv_amd.build

Every call compiles from scratch into ``decode_attention_okv_amd/_build`` and links
``decode_attention_okv_amd/libokv.so``.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libokv.so")
ARCH = "gfx950"

COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # no packed-FP32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wno-unused-command-line-argument",
]

SOURCES = [
    # (source, extra flags)
    ("okv_write.hip", ["-ffp-contract=off"]),   # bit-exact float32 write path
    # MFMA results in VGPRs: the kernels read every accumulator with VALU right away
    ("okv_decode_head.hip", ["-mllvm", "-amdgpu-mfma-vgpr-form"]),
    ("okv_decode_mfma.hip", ["-mllvm", "-amdgpu-mfma-vgpr-form"]),
    ("okv_reduce.hip", []),
    # products are fused only where the source writes fmaf (hi + lo splits stay exact)
    ("okv_prefill.hip", ["-ffp-contract=off", "-mllvm", "-amdgpu-mfma-vgpr-form"]),
    ("okv_calib.hip", []),
    ("okv_probe.hip", []),
    ("okv_host.cpp", ["-x", "hip"]),
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False) -> str:
    """Compile every source (in parallel, one hipcc per file) and link libokv.so."""
    from concurrent.futures import ThreadPoolExecutor
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    cmds, objs = [], []
    for src, extra in SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        cmds.append([cc, *COMMON, *extra, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)

    def run(cmd):
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)

    workers = max(1, min(len(cmds), int(os.environ.get("MAX_JOBS", "6"))))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        for f in [ex.submit(run, c) for c in cmds]:
            f.result()
    tmp = LIB + ".tmp"
    cmd = [cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


def dump_isa(out_dir: str) -> None:
    """Write the gfx950 assembly of the kernels (for reading only)."""
    os.makedirs(out_dir, exist_ok=True)
    cc = hipcc()
    for src, extra in SOURCES[:4]:
        out = os.path.join(out_dir, os.path.splitext(src)[0] + ".s")
        subprocess.run([cc, *COMMON, *extra, "--cuda-device-only", "-S",
                        os.path.join(CSRC, src), "-o", out], check=True)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
