"""CPU sanitizer runs (no GPU): the oracle and the host side of the GPU library under AddressSanitizer and
UndefinedBehaviorSanitizer.

Each runs in a child process with the sanitizer runtime preloaded first (ahead of anything already
preloaded), because the Python interpreter itself is not instrumented:

* the oracle built by gcc with -fsanitize=address,undefined, under the oracle pins and the thread-count
  test (gcc's runtime);
* libsmla.so with its host pass built by hipcc with -fsanitize=address,undefined (clang's runtime), under
  the C-ABI tests: plan logic, struct layout and every host-side argument check.

Errors abort the child (-fno-sanitize-recover=all); leak checking is off (the interpreter's own
allocations would be reported).
"""
import os
import subprocess
import sys

import pytest

import oracle
from sparse_mla_decode_smla_amd import build as gpu_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = os.path.join(ROOT, "tests")


def _runtime(cmd):
    path = subprocess.run(cmd, capture_output=True, text=True).stdout.strip()
    return path if path and os.path.exists(path) else None


def _run_child(code, preload, tmp_path):
    env = dict(os.environ)
    env["LD_PRELOAD"] = preload + (":" + env["LD_PRELOAD"] if env.get("LD_PRELOAD") else "")
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["PYTHONDONTWRITEBYTECODE"] = "1"
    r = subprocess.run([sys.executable, "-c", code], env=env, cwd=ROOT, capture_output=True, text=True,
                       timeout=1200)
    tail = (r.stdout[-4000:] + "\n" + r.stderr[-4000:])
    assert r.returncode == 0, f"sanitized run failed (rc {r.returncode}):\n{tail}"
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error:" not in r.stderr, tail
    return r


def test_oracle_under_asan_ubsan(tmp_path):
    asan = _runtime(["gcc", "-print-file-name=libasan.so"])
    if asan is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    lib = oracle.build(force=True, out_path=str(tmp_path / "liboracle_asan.so"), sanitize=True)
    code = (f"import sys; sys.path[:0] = [{ROOT!r}, {TESTS!r}]\n"
            "import oracle, pytest\n"
            f"oracle._default = oracle.Oracle({lib!r})\n"
            "sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', 'tests/test_oracle_pins.py', "
            "'tests/test_oracle_threads.py']))\n")
    r = _run_child(code, asan, tmp_path)
    assert " passed" in r.stdout


def test_library_host_side_under_asan_ubsan(tmp_path):
    rt = _runtime(["/opt/rocm/llvm/bin/clang", "-print-file-name=libclang_rt.asan-x86_64.so"])
    if rt is None:
        pytest.skip("clang's AddressSanitizer runtime is not installed")
    lib = gpu_build.build_host_sanitized(str(tmp_path / "libsmla_asan.so"))
    code = (f"import sys; sys.path[:0] = [{ROOT!r}, {TESTS!r}]\n"
            "from sparse_mla_decode_smla_amd import binding\n"
            f"binding.LIB_PATH = {lib!r}\n"
            "import pytest\n"
            "sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', 'tests/test_abi.py']))\n")
    r = _run_child(code, rt, tmp_path)
    assert " passed" in r.stdout
