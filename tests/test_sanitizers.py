"""CPU runs under AddressSanitizer + UndefinedBehaviorSanitizer, in child
processes (no recovery: the first report aborts the child and fails the
test):
  * the oracle's pins, against a sanitized build of oracle.c;
  * the host-side ABI tests, against the HIP library with the host code of
    its host-heavy sources (argument checks, plan layout, code generator)
    built with the sanitizers.
Python itself is not instrumented, so only this code is checked; leak
checking is off (the interpreter and the HIP runtime hold allocations until
exit)."""
import importlib.util
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime(name):
    out = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True)
    path = out.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.slow
def test_oracle_pins_under_address_and_undefined_sanitizers():
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("gcc sanitizer runtimes not found")
    sys.path.insert(0, ROOT)
    import oracle
    oracle.build(force=True, sanitize=True)
    env = dict(os.environ, SNACK_ORACLE_SANITIZE="1", LD_PRELOAD=f"{asan}:{ubsan}",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    # python itself is not instrumented: only the oracle's own code is checked
    # (leak checking would report the interpreter's allocations)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py"), "-k",
                        "not graph and not config_sizes"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "passed" in r.stdout


def _clang_asan_runtime():
    """The ROCm clang's AddressSanitizer runtime (it holds the
    UndefinedBehaviorSanitizer handlers too): the library is built by that
    compiler, so its runtime, not gcc's, must be preloaded."""
    for d in ("/opt/rocm/llvm/lib/clang",):
        if not os.path.isdir(d):
            continue
        for ver in sorted(os.listdir(d), reverse=True):
            for sub in ("lib/linux/libclang_rt.asan-x86_64.so",
                        "lib/x86_64-unknown-linux-gnu/libclang_rt.asan.so"):
                p = os.path.join(d, ver, sub)
                if os.path.exists(p):
                    return p
    return None


@pytest.mark.slow
def test_host_abi_under_address_and_undefined_sanitizers(tmp_path):
    rt = _clang_asan_runtime()
    if not rt:
        pytest.skip("clang sanitizer runtime not found")
    spec = importlib.util.spec_from_file_location(
        "_snack_build", os.path.join(ROOT, "unstructured_sparse_nn_amd", "build.py"))
    hb = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(hb)
    # a scratch copy of the tree whose package holds the sanitized library
    tree = tmp_path / "tree"
    pkg = tree / "unstructured_sparse_nn_amd"
    pkg.mkdir(parents=True)
    for f in os.listdir(os.path.join(ROOT, "unstructured_sparse_nn_amd")):
        if f.endswith(".py"):
            shutil.copy(os.path.join(ROOT, "unstructured_sparse_nn_amd", f), pkg / f)
    try:
        hb.build_host_sanitized(str(tmp_path / "obj"))
    except FileNotFoundError as e:
        pytest.skip(f"the regular build's objects are missing ({e}): build the library first")
    shutil.copy(tmp_path / "obj" / "libsnack.so", pkg / "libsnack.so")
    for d in ("include", "tests", "oracle", "synth"):
        shutil.copytree(os.path.join(ROOT, d), tree / d,
                        ignore=shutil.ignore_patterns("__pycache__", "*.so"))
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "tests/test_abi_host.py", "-k", "not library_allocates_nothing"],
                       cwd=tree, env=env, capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "passed" in r.stdout
