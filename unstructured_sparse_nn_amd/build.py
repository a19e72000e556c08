"""Build the HIP library (libsnack.so) for gfx950 with hipcc, in-tree.

Every source under csrc/ is compiled to an object in parallel, then linked
into ``unstructured_sparse_nn_amd/libsnack.so``.  Packed fp32 instructions
are disabled for all device code (``-target-feature -packed-fp32-ops``).
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libsnack.so")
# longest compiles first (they start first in the worker pool)
SOURCES = ["wave_spmm_bf16.hip", "wave_spmm_f32.hip", "wave_fused.hip", "wave_sddmm_bf16.hip",
           "wave_sddmm_f32.hip", "spmm.hip", "prune_bitmap.hip", "api.hip", "prims.hip",
           "prepare.hip", "prune.hip", "aux.hip", "fixed.hip", "wave.hip", "noalloc.hip", "calib.hip"]
ARCH = "gfx950"  # the MI355X (CDNA4); no other target is built

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
          "-Wno-unused-function", "-Wno-unused-command-line-argument", "-fvisibility=hidden",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          f"-I{os.path.join(HERE, '..', 'include')}"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *CFLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs, "-lhiprtc"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)


# The debug build: the same library with SNACK_DEBUG_CHECKS defined in
# api.hip, whose product entry points then check every plan array and COO
# index on the device (within the arrays' sizes) before launching, and
# return SNACK_E_PLAN_CORRUPT instead of reading out of bounds.  Selected
# at import time with SNACK_LIBRARY=<path of libsnack_debug.so>.
DEBUG_LIB = os.path.join(HERE, "libsnack_debug.so")


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = min(len(SOURCES) + 1, int(os.environ.get("MAX_JOBS", "8")))

    def debug_api():
        obj = os.path.join(BUILD, "api_debug.o")
        cmd = [HIPCC, *CFLAGS, "-DSNACK_DEBUG_CHECKS", "-c", os.path.join(CSRC, "api.hip"),
               "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for api.hip (debug checks):\n{r.stderr}")
        return obj

    with ThreadPoolExecutor(jobs) as ex:
        dbg = ex.submit(debug_api)
        objs = list(ex.map(_compile, SOURCES))
        dbg_obj = dbg.result()
    _link(objs, LIB)
    _link([dbg_obj if os.path.basename(o) == "api.o" else o for o in objs], DEBUG_LIB)
    if verbose:
        print(f"built {LIB} and {DEBUG_LIB}", file=sys.stderr)
    return LIB


# Sources whose host code is more than kernel launches: argument checks and
# plan layout, the fixed-pattern code generator, the static workspace, the
# calibration entry point.
HOST_HEAVY = ["api.hip", "fixed.hip", "noalloc.hip", "calib.hip"]


def build_host_sanitized(out_dir: str) -> str:
    """libsnack.so in out_dir with the host code of HOST_HEAVY built with
    AddressSanitizer and UndefinedBehaviorSanitizer (-Xarch_host: device code
    unchanged) and the other objects taken from the regular build in _build,
    for running the host-side ABI tests under the sanitizers.  Needs a
    regular build first."""
    os.makedirs(out_dir, exist_ok=True)
    san = []
    for f in ("-fsanitize=address,undefined", "-fno-sanitize-recover=all",
              "-fno-omit-frame-pointer", "-g"):
        san += ["-Xarch_host", f]

    def one(src):
        obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
        r = subprocess.run([HIPCC, *CFLAGS, *san, "-c", os.path.join(CSRC, src), "-o", obj],
                           capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc (sanitized host) failed for {src}:\n{r.stderr}")
        return obj

    with ThreadPoolExecutor(len(HOST_HEAVY)) as ex:
        objs = list(ex.map(one, HOST_HEAVY))
    for src in SOURCES:
        if src not in HOST_HEAVY:
            obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
            if not os.path.exists(obj):
                raise FileNotFoundError(obj)
            objs.append(obj)
    lib = os.path.join(out_dir, "libsnack.so")
    r = subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Xarch_host",
                        "-fsanitize=address,undefined", "-o", lib, *objs, "-lhiprtc"],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link (sanitized host) failed:\n{r.stderr}")
    return lib


if __name__ == "__main__":
    build(verbose=True)
