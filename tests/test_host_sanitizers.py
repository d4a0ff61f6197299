"""CPU tests: the library's host code (argument checks, workspace planning,
packed-batch parsing, device lookup) under AddressSanitizer and
UndefinedBehaviorSanitizer.

The debug build (``build.build_host_sanitized``) instruments the host pass of
the host sources only; the C-ABI tests then run against it in a child process
with the sanitizer runtime preloaded. A planted heap overflow and a planted
signed overflow, built the same way, check that the set-up reports errors.
"""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(
    not (shutil.which("hipcc") or os.path.exists("/opt/rocm/bin/hipcc")), reason="hipcc not available")


@pytest.fixture(scope="module")
def san():
    from block_sparse_long_gating_amd import build
    lib = build.build_host_sanitized()
    env = dict(os.environ, LD_PRELOAD=build.asan_runtime(), MOBA_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    return build, lib, env


def run(env, *args, timeout=600):
    return subprocess.run([sys.executable, *args], cwd=ROOT, env=env, capture_output=True, text=True,
                          timeout=timeout)


def test_abi_suite_under_host_sanitizers(san):
    _, lib, env = san
    undefined = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True).stdout
    assert "__asan_" in undefined and "__ubsan_" in undefined
    r = run(env, "-c", "import block_sparse_long_gating_amd as m; print(m.library_path())")
    assert r.returncode == 0 and r.stdout.strip() == lib, r.stderr[-2000:]
    r = run(env, "-m", "pytest", "tests/test_abi.py", "-q", "-x", "-p", "no:cacheprovider")
    report = r.stdout[-3000:] + r.stderr[-3000:]
    assert r.returncode == 0, report
    assert "AddressSanitizer" not in r.stderr and "runtime error:" not in r.stderr, report


PLANTED = r"""
#include <cstdint>
#include <cstdlib>
extern "C" int heap_overflow(int n) {
  int* p = static_cast<int*>(std::malloc(n * sizeof(int)));
  for (int i = 0; i <= n; ++i) p[i] = i;
  const int r = p[n / 2];
  std::free(p);
  return r;
}
extern "C" int signed_overflow(int x) { return x + INT32_MAX; }
"""


@pytest.mark.parametrize("fn,arg,marker", [("heap_overflow", 8, "heap-buffer-overflow"),
                                           ("signed_overflow", 5, "runtime error")])
def test_planted_host_errors_are_reported(san, tmp_path, fn, arg, marker):
    build, _, env = san
    src = tmp_path / "planted.cpp"
    src.write_text(PLANTED)
    so = tmp_path / "libplanted.so"
    cmd = [build.hipcc(), "-O1", "-fPIC", "-shared", *build.SAN_FLAGS, "-shared-libsan", str(src), "-o", str(so)]
    subprocess.run(cmd, check=True, capture_output=True)
    r = run(env, "-c", f"import ctypes; print(ctypes.CDLL({str(so)!r}).{fn}({arg}))")
    assert r.returncode != 0
    assert marker in r.stderr, r.stderr[-2000:]
