"""Host AddressSanitizer and UndefinedBehaviorSanitizer runs, on the CPU.

The oracle is rebuilt with gcc -fsanitize=address,undefined and its pins
run against it; the library is rebuilt with both sanitizers on its host
code only (hipcc -Xarch_host; the device code is not instrumented) and
the host-side tests of the C ABI and of the debug checks run against it.
Each run happens in a child process with the sanitizer runtime preloaded
(the Python interpreter is not instrumented); any report aborts it, and
a nonzero exit fails the test.  Leak detection is off: the interpreter
and the HIP runtime keep allocations until exit."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = os.path.join(ROOT, "tests")

pytestmark = pytest.mark.slow

_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1:verify_asan_link_order=0",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _child(preload, code, timeout=900):
    env = dict(os.environ, LD_PRELOAD=preload, **_ENV)
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True,
                       text=True, timeout=timeout, cwd=ROOT)
    assert r.returncode == 0, (r.stdout[-4000:] + "\n" + r.stderr[-4000:])
    return r.stdout


def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    so = str(tmp_path / "liboracle_sanitized.so")
    subprocess.check_call(
        ["gcc", "-O1", "-g", "-std=c99", "-fPIC", "-shared", "-fopenmp",
         "-ffp-contract=off", "-fno-omit-frame-pointer",
         "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
         os.path.join(ROOT, "oracle", "eagletree_ref.c"), "-o", so, "-lm"])
    libasan = subprocess.check_output(["gcc", "-print-file-name=libasan.so"],
                                      text=True).strip()
    out = _child(libasan, f"""
import sys
sys.path[:0] = [{ROOT!r}, {TESTS!r}]
import oracle
oracle._SO = {so!r}
import pytest
rc = pytest.main(['-q', '-x', '-p', 'no:cacheprovider', {os.path.join(TESTS, 'test_oracle_pins.py')!r}])
assert oracle.lib()._name == {so!r}
sys.exit(rc)
""")
    assert " passed" in out


def test_host_layer_under_asan_and_ubsan(tmp_path):
    sys.path.insert(0, ROOT)
    from dynamic_draft_tree_amd import build as lib_build
    so = str(tmp_path / "libeagletree_sanitized.so")
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    flags = [f for f in lib_build.HIPCC_FLAGS if f != "-O3"]
    subprocess.run(
        [hipcc, *flags, "-O1", "-g",
         "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
         "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
         "-shared-libsan", *lib_build.sources(), "-o", so],
        check=True, capture_output=True)
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc)), "..", "llvm", "bin", "clang")
    if not os.path.exists(clang):
        clang = "/opt/rocm/llvm/bin/clang"
    rt = subprocess.check_output([clang, "-print-file-name=libclang_rt.asan-x86_64.so"],
                                 text=True).strip()
    out = _child(rt, f"""
import sys
sys.path[:0] = [{ROOT!r}, {TESTS!r}]
from dynamic_draft_tree_amd import binding
binding.LIB_PATH = {so!r}
import pytest
rc = pytest.main(['-q', '-x', '-p', 'no:cacheprovider', '-m', 'not gpu',
                  {os.path.join(TESTS, 'test_abi_host.py')!r},
                  {os.path.join(TESTS, 'test_debug_checks.py')!r}])
assert binding.lib()._name == {so!r}
sys.exit(rc)
""")
    assert " passed" in out
