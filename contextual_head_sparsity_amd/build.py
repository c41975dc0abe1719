"""Build the SHA decode library (libsha.so) in-tree for gfx950 with hipcc.

    python -m contextual_head_sparsity_amd.build

Every call compiles from source (no staleness check) and replaces the
library atomically.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libsha.so")
PROBE_LIB = os.path.join(PKG, "libsha_probe.so")
EXAMPLE = os.path.join(PKG, "examples", "decode_c")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
ARCH = "gfx950"

# Packed-fp32 VALU ops are disabled for all device code; hipcc's host pass
# warns that it does not know the feature, which is harmless.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"-I{INCLUDE}", f"-I{CSRC}", "-Wall",
          "-Wno-unused-command-line-argument"]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the SHA library)")


def _run(cmd):
    print("+", " ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def build(verbose: bool = True) -> str:
    hipcc = _hipcc()
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs, cmds = [], []
    for src in ("sha_kernels.hip", "sha_gqa_mfma.hip", "sha_mlp.hip", "sha_router.hip",
                "sha_noalloc.hip"):
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        cmds.append([hipcc, "-c", f"--offload-arch={ARCH}", *COMMON, *DEVICE_FLAGS,
                     os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    for src in ("sha_api.cpp", "sha_step.cpp"):
        obj = os.path.join(objdir, src.replace(".cpp", ".o"))
        cmds.append([hipcc, "-c", *COMMON, os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    # The translation units are independent: compile them side by side.
    jobs = max(1, min(len(cmds), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    with concurrent.futures.ThreadPoolExecutor(jobs) as pool:
        for f in [pool.submit(_run, c) for c in cmds]:
            f.result()
    tmp = LIB + ".tmp"
    _run([hipcc, "-shared", f"--offload-arch={ARCH}", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    # The benchmark's read-bandwidth probe: a library of its own.
    tmp = PROBE_LIB + ".tmp"
    _run([hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *COMMON, *DEVICE_FLAGS,
          os.path.join(PKG, "probe", "sha_probe.hip"), "-o", tmp])
    os.replace(tmp, PROBE_LIB)
    # The plain-C example of the ABI, linked against the library just built.
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        raise RuntimeError("no C compiler for the C-ABI example")
    tmp = EXAMPLE + ".tmp"
    _run([cc, "-std=c11", "-O2", "-Wall", "-Wextra", f"-I{INCLUDE}", f"-I{ROCM}/include",
          "-D__HIP_PLATFORM_AMD__", EXAMPLE + ".c", f"-L{PKG}", "-lsha", f"-L{ROCM}/lib",
          "-lamdhip64", "-lm", "-Wl,-rpath,$ORIGIN/..", f"-Wl,-rpath,{ROCM}/lib", "-o", tmp])
    os.replace(tmp, EXAMPLE)
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
