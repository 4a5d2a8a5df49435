"""Build libfm.so (the gfx950 HIP kernels and the C ABI of include/fm.h) in-tree.

Usage: ``python -m block_diffusion_drafter_all_amd.build`` or ``build()``.
hipcc cross-compiles for gfx950, so this runs on machines without a GPU.
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
REPO_DIR = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
BUILD_DIR = os.path.join(PKG_DIR, "_build")
LIB_DIR = os.path.join(PKG_DIR, "_lib")
LIB_PATH = os.path.join(LIB_DIR, "libfm.so")
SOURCES = ("abi.cpp", "context_rows.hip", "cross_attention.hip", "dit.hip", "self_attention.hip", "write_kv.hip")
# The benchmark's memory-system probes (include/fm_probe.h), a library of their own.
PROBE_LIB_PATH = os.path.join(LIB_DIR, "libfm_probe.so")
PROBE_SOURCES = ("probe.hip",)
ARCH = "gfx950"

# Packed fp32 instructions are disabled: the compiler must not form
# v_pk_{add,mul,fma}_f32 from ordinary float code.
COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-fPIC",
    "-std=c++17",
    "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(REPO_DIR, "include"),
]


# Per-source flags.  The attention kernels keep their MFMA accumulators in
# VGPRs: in the AGPR form the compiler copied every accumulator back to VGPRs
# on every K/V tile (for the rescale and store paths), 32 to 128 VALU moves a
# tile; in the VGPR form those copies are gone and nothing spills.
SOURCE_FLAGS = {"cross_attention.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libfm)")


def _compile(hipcc: str, src: str, extra: list[str]) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc, *COMMON_FLAGS, *SOURCE_FLAGS.get(os.path.basename(src), []), *extra, "-c", os.path.join(CSRC, src),
           "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def _link(hipcc: str, objs: list[str], path: str) -> None:
    tmp = path + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, path)


def build(extra_flags: list[str] | None = None, verbose: bool = False) -> str:
    """Compile every source and link libfm.so and libfm_probe.so; returns
    libfm.so's path.  Always rebuilds."""
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    os.makedirs(LIB_DIR, exist_ok=True)
    extra = list(extra_flags or [])
    every = SOURCES + PROBE_SOURCES
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(every)) as ex:
        objs = dict(zip(every, ex.map(lambda s: _compile(hipcc, s, extra), every)))
    _link(hipcc, [objs[s] for s in SOURCES], LIB_PATH)
    _link(hipcc, [objs[s] for s in PROBE_SOURCES], PROBE_LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH} and {PROBE_LIB_PATH}")
    return LIB_PATH


if __name__ == "__main__":
    build(extra_flags=sys.argv[1:], verbose=True)
