"""Sanitizer runs on the CPU: the oracle and the host side of the library
built with AddressSanitizer and UndefinedBehaviorSanitizer.

* The C oracle is compiled with gcc -fsanitize=address,undefined (errors
  abort), and every oracle pin (tests/test_oracle_*.py) runs against it in a
  subprocess that preloads gcc's ASan runtime.
* libmgs.so is rebuilt with its host code instrumented (each -fsanitize
  flag after -Xarch_host, so the gfx950 device code is built as usual), and
  the C ABI's host-side tests (tests/test_abi_host.py: argument checks, the
  workspace size query, exported symbols) run against it with clang's ASan
  runtime preloaded. Those calls return before any GPU work, so no GPU is
  needed.
A sanitizer report fails the subprocess and therefore the test.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def san_env(tmp_path):
    """Sanitizer settings: stop at the first report, write reports to files
    under tmp_path (pytest's output capture would swallow them)."""
    return {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:exitcode=23:log_path=%s" % (tmp_path / "asan"),
            "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1:exitcode=24:log_path=%s"
                             % (tmp_path / "ubsan")}


def reports(tmp_path):
    return "".join(open(p).read()[-4000:] for p in sorted(glob.glob(str(tmp_path / "*san.*"))))


def _gcc_asan_runtime():
    p = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def _clang_asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    rt = _gcc_asan_runtime()
    if rt is None:
        pytest.skip("gcc's ASan runtime is not installed")
    so = tmp_path / "liboracle_san.so"
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
                    "-fno-fast-math", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-fno-omit-frame-pointer", "-o", str(so), os.path.join(ROOT, "oracle", "mgs_oracle.c"),
                    "-lm"], check=True)
    env = dict(os.environ, MGS_ORACLE_LIB=str(so), LD_PRELOAD=rt, **san_env(tmp_path))
    tests = sorted(glob.glob(os.path.join(ROOT, "tests", "test_oracle_*.py")))
    tests = [t for t in tests if not t.endswith(("test_oracle_mutants.py", "test_oracle_pool.py"))]
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider"] + tests,
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=1200)
    assert r.returncode == 0, reports(tmp_path) + r.stdout[-3000:] + r.stderr[-3000:]
    assert "passed" in r.stdout


def test_library_host_code_under_asan_and_ubsan(tmp_path):
    rt = _clang_asan_runtime()
    if rt is None:
        pytest.skip("clang's ASan runtime is not installed")
    from group_scaling_fp8_amd import build as B
    so = tmp_path / "libmgs_san.so"
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    r = subprocess.run([hipcc] + B.HIPCC_FLAGS + san + ["-I", B.INCLUDE, "-I", B.CSRC, "-o", str(so)]
                       + B.sources(), capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    runner = ("import sys; sys.path.insert(0, %r); import group_scaling_fp8_amd._lib as L; "
              "L._LIB_PATH = %r; import pytest; "
              "sys.exit(pytest.main(['-x', '-q', '-p', 'no:cacheprovider', '-k', 'not python_binding', %r]))"
              % (ROOT, str(so), os.path.join(ROOT, "tests", "test_abi_host.py")))
    env = dict(os.environ, LD_PRELOAD=rt, **san_env(tmp_path))
    r = subprocess.run([sys.executable, "-c", runner], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=600)
    assert r.returncode == 0, reports(tmp_path) + r.stdout[-3000:] + r.stderr[-3000:]
    assert "passed" in r.stdout
