"""Build libfa.so (the gfx950 HIP kernels and the C ABI) in-tree with hipcc.

Usage: python -m exact_io_aware_14_amd.build [--save-temps]

The library lands next to this file (exact_io_aware_14_amd/libfa.so), where
the Python binding loads it from. Every source is compiled for gfx950 only.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libfa.so")

SOURCES = ["fa_api.hip", "fa_fwd.hip", "fa_fwd_w.hip", "fa_bwd.hip", "fa_bwd_w.hip", "fa_fp8.hip"]

# Per-source flags, for the d = 256 kernels only (the others are as fast or
# faster without them): the backward keeps its accumulators in place only
# under LLVM's "max-memory-clause" machine scheduler (with the default one the
# register allocator rotates them through other registers every tile), and
# the forward runs faster with MFMA results in VGPRs where they fit.
EXTRA_FLAGS = {"fa_bwd_w.hip": ["-mllvm", "-amdgpu-sched-strategy=max-memory-clause"],
               "fa_fwd_w.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-ffp-contract=fast",
    # no packed-FP32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I", INCLUDE,
    "-I", CSRC,
]


def _run(cmd):
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature
    lines = [ln for ln in proc.stdout.splitlines() if "packed-fp32-ops" not in ln]
    return proc.returncode, "\n".join(lines)


def build(save_temps: bool = False, verbose: bool = True) -> str:
    if not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        objs.append(obj)
        cmd = [HIPCC, *FLAGS, *EXTRA_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
        if save_temps:
            os.makedirs(os.path.join(BUILD, "temps"), exist_ok=True)
            cmd += ["--save-temps"]
        cmds.append((src, cmd))

    cwd = os.getcwd()
    if save_temps:
        os.chdir(os.path.join(BUILD, "temps"))
    try:
        with cf.ThreadPoolExecutor(max_workers=len(cmds)) as ex:
            results = list(ex.map(lambda sc: (sc[0], _run(sc[1])), cmds))
    finally:
        os.chdir(cwd)
    failed = False
    for src, (rc, out) in results:
        if out.strip() and verbose:
            print(f"[{src}]\n{out}")
        if rc != 0:
            failed = True
    if failed:
        raise RuntimeError("hipcc failed")
    tmp = LIB + ".tmp"
    rc, out = _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs])
    if rc != 0:
        raise RuntimeError("link failed:\n" + out)
    shutil.move(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(save_temps="--save-temps" in sys.argv)
