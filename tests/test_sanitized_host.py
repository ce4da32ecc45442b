"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

- The pool bookkeeping and the C ABI (csrc/pool.cpp, csrc/capi.cpp) are
  built by the host compiler with both sanitizers into a host-only library
  (kernel launchers stubbed, tests/sanitize/kernel_stubs.cpp), and
  tests/test_capi_host.py -- golden fixtures, seeded random operation
  sequences bit-exact against the oracle simulator, argument validation --
  runs against it.
- tests/sanitize/index_check.cpp walks the kernels' page-table indexing (the
  constexpr helpers of csrc/index.h that the kernels call) over rings of 1-8
  pages and larger, windows 1..C and lengths across page and ring
  boundaries, under the same sanitizers.  A copy of index.h that wraps the
  ring index once per step (the one-page-ring mistake) must fail it.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "hybrid_sliding_window_hswa_amd", "csrc")
SAN = os.path.join(ROOT, "tests", "sanitize")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
FLAGS = ["-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
         "-fno-omit-frame-pointer"]

pytestmark = pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")


def _run(cmd, **kw):
    return subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, **kw)


def _asan_env():
    env = dict(os.environ)
    asan = _run(["g++", "-print-file-name=libasan.so"]).stdout.strip()
    env["LD_PRELOAD"] = asan
    env["ASAN_OPTIONS"] = "detect_leaks=0"          # the Python interpreter's own
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    return env


def _index_check(tmp_path, include_dir):
    exe = str(tmp_path / "index_check")
    r = _run(["g++", *FLAGS, "-Wall", "-I", include_dir,
              os.path.join(SAN, "index_check.cpp"), "-o", exe])
    assert r.returncode == 0, r.stdout
    return _run([exe], timeout=300)


def test_sanitizers_are_live(tmp_path):
    """The flags catch a planted heap overflow (the toolchain check)."""
    src = tmp_path / "oob.cpp"
    src.write_text("int main(int c, char**) { int* a = new int[4]; int r = a[3 + c]; "
                   "delete[] a; return r; }\n")
    exe = str(tmp_path / "oob")
    assert _run(["g++", *FLAGS, str(src), "-o", exe]).returncode == 0
    r = _run([exe])
    assert r.returncode != 0
    assert "heap-buffer-overflow" in r.stdout or "runtime error" in r.stdout


def test_kernel_index_arithmetic(tmp_path):
    r = _index_check(tmp_path, CSRC)
    assert r.returncode == 0, r.stdout[-3000:]
    assert "index checks passed" in r.stdout


def test_index_check_catches_a_single_ring_wrap(tmp_path):
    """With one wrap per 32-key step a one-page ring steps past its row."""
    src = open(os.path.join(CSRC, "index.h")).read()
    twice = "    if (e >= npr) e -= npr;\n    if (e >= npr) e -= npr;\n"
    assert src.count(twice) == 1
    (tmp_path / "index.h").write_text(src.replace(twice, "    if (e >= npr) e -= npr;\n"))
    r = _index_check(tmp_path, str(tmp_path))
    assert r.returncode != 0 and "FAILED" in r.stdout and "prefill" in r.stdout


def test_c_abi_host_tests_under_sanitizers(tmp_path):
    lib = str(tmp_path / "libhswa_host_san.so")
    r = _run(["g++", *FLAGS, "-fPIC", "-shared", "-Wall", "-D__HIP_PLATFORM_AMD__",
              f"-I{ROCM}/include", "-I", CSRC, os.path.join(CSRC, "pool.cpp"),
              os.path.join(CSRC, "capi.cpp"), os.path.join(SAN, "kernel_stubs.cpp"),
              f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib", "-o", lib])
    assert r.returncode == 0, r.stdout
    env = _asan_env()
    env["HSWA_TEST_LIBRARY"] = lib
    # the sanitized build is the one the binding loads
    probe = _run([sys.executable, "-c",
                  "import sys; sys.path.insert(0, 'tests'); import conftest; "
                  "import hybrid_sliding_window_hswa_amd as H; H.library(); "
                  "print([l for l in open('/proc/self/maps') if 'libhswa' in l][0].split()[-1])"],
                 cwd=ROOT, env=env, timeout=120)
    assert probe.returncode == 0 and probe.stdout.strip().endswith("libhswa_host_san.so"), \
        probe.stdout
    r = _run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
              os.path.join("tests", "test_capi_host.py")], cwd=ROOT, env=env, timeout=600)
    assert r.returncode == 0, r.stdout[-4000:]
    assert "AddressSanitizer" not in r.stdout and "runtime error" not in r.stdout
