"""Build libditattn.so (gfx950) from csrc/ with hipcc.

Each source is compiled to an object under _build/ (in parallel), then linked
into attention_non_causal_amd/libditattn.so.  Run as a module or call build().

build(debug_barriers=True) builds the race-check variant libditattn_debugsync.so
from the same sources with -DDIT_DEBUG_BARRIERS (see debug_sync in
csrc/common.hpp); only tests load it.  build_probe() builds libditprobe.so, the
matrix-core throughput and vector-issue probes that `bench.py --mfma-ceiling`
and `bench.py --valu-issue` run (probe/).
"""
from __future__ import annotations

import concurrent.futures as cf
import ctypes
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build", "ditattn")
LIB_NAME = "libditattn.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
DEBUG_BUILD_DIR = os.path.join(ROOT, "_build", "ditattn_debugsync")
DEBUG_LIB_PATH = os.path.join(PKG, "libditattn_debugsync.so")
PROBE_SRCS = [os.path.join(PKG, "probe", f) for f in ("mfma_ceiling.hip", "valu_issue.hip")]
PROBE_LIB_PATH = os.path.join(PKG, "libditprobe.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libditattn)")


def sources() -> list[str]:
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith((".hip", ".cpp")))


COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    # keep the compiler from forming packed fp32 VALU ops (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


# Per-source flags.  fwd_bf16.hip keeps O in accumulation registers through
# asm MFMAs and wants every compiler-generated MFMA (the S^T products, read by
# vector instructions) in the VGPR form; without NaN semantics its running
# maxima compile to v_max3_f32 with no canonicalising instructions (a NaN
# input gives a NaN result either way).
FILE_FLAGS = {
    "fwd_bf16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1", "-fno-honor-nans"],
    "fwd_fp8.hip": ["-fno-honor-nans"],
}


def _compile(src: str, build_dir: str = BUILD_DIR, extra: tuple = ()) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = ([hipcc()] + COMMON_FLAGS + FILE_FLAGS.get(os.path.basename(src), []) + list(extra)
           + ["-c", src, "-o", obj])
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, debug_barriers: bool = False) -> str:
    build_dir = DEBUG_BUILD_DIR if debug_barriers else BUILD_DIR
    lib_path = DEBUG_LIB_PATH if debug_barriers else LIB_PATH
    extra = ("-DDIT_DEBUG_BARRIERS",) if debug_barriers else ()
    os.makedirs(build_dir, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s_: _compile(s_, build_dir, extra), srcs))
    tmp = lib_path + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    # resolve every symbol now: a kernel whose host stub was not emitted shows
    # up here as an undefined symbol instead of at the first load on a GPU host
    ctypes.CDLL(tmp, mode=os.RTLD_NOW | os.RTLD_LOCAL)
    os.replace(tmp, lib_path)
    if verbose:
        print(f"built {lib_path}")
    return lib_path


def build_probe(verbose: bool = False) -> str:
    tmp = PROBE_LIB_PATH + ".tmp"
    cmd = [hipcc()] + COMMON_FLAGS + ["-shared"] + PROBE_SRCS + ["-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"probe build failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    ctypes.CDLL(tmp, mode=os.RTLD_NOW | os.RTLD_LOCAL)
    os.replace(tmp, PROBE_LIB_PATH)
    if verbose:
        print(f"built {PROBE_LIB_PATH}")
    return PROBE_LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
    build(verbose=True, debug_barriers=True)
    build_probe(verbose=True)
    sys.exit(0)
