"""The debug build (libsnack_debug.so, SNACK_DEBUG_CHECKS): same ABI as the
library, and on the GPU a device check of the plan before every product."""
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
PKG = os.path.join(ROOT, "unstructured_sparse_nn_amd")
DEBUG_LIB = os.path.join(PKG, "libsnack_debug.so")


def _exports(path):
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True,
                         check=True).stdout
    return sorted(line.split()[-1] for line in out.splitlines()
                  if line.split() and line.split()[-1].startswith("snack_"))


def test_debug_library_exports_the_same_abi():
    assert os.path.exists(DEBUG_LIB), "build the HIP library first (__graft_entry__.build())"
    assert _exports(DEBUG_LIB) == _exports(os.path.join(PKG, "libsnack.so"))
    import ctypes
    lib = ctypes.CDLL(DEBUG_LIB)
    lib.snack_status_str.restype = ctypes.c_char_p
    lib.snack_status_str.argtypes = [ctypes.c_int32]
    assert b"debug build" in lib.snack_status_str(-13)


@pytest.mark.gpu
def test_debug_build_checks_plans_before_products():
    env = dict(os.environ, SNACK_LIBRARY=DEBUG_LIB)
    r = subprocess.run([sys.executable, "-u", os.path.join(HERE, "_debug_checks_child.py")],
                       env=env, capture_output=True, text=True, timeout=110)
    print(r.stdout[-3000:])
    assert r.returncode == 0, r.stderr[-3000:]
    assert "DEBUG CHECKS OK" in r.stdout
