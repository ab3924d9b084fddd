"""Host code under AddressSanitizer and UBSan (CPU tier).

Three builds, each exercised in a subprocess under its own sanitizer runtime
(gcc's and clang's cannot share a process):
- the oracle and the input generator (plain C, gcc) run the oracle's pin tests
  and the generator's tests;
- the C ABI's host side (argument checks, the decode split planner and the
  launch wrappers of api.hip, built by hipcc with host-only sanitizers) runs the
  ABI tests, which reach every entry point's checks without a GPU.
A first test confirms that the gcc setup reports a planted heap overflow, so a
clean run means something.
"""
import os
import subprocess
import sys
import textwrap

import pytest

import oracle
import synth
from parameterized_local_linear_amd import build as hip_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _gcc_runtime():
    libs = [subprocess.run(["gcc", f"-print-file-name={n}"], capture_output=True, text=True,
                           check=True).stdout.strip() for n in ("libasan.so", "libubsan.so")]
    return ":".join(libs)


def _env(preload, **extra):
    env = dict(os.environ, LD_PRELOAD=preload, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    env.update(extra)
    return env


def test_gcc_sanitizer_setup_reports_a_planted_overflow(tmp_path):
    src = tmp_path / "bad.c"
    src.write_text("#include <stdlib.h>\nint bad(int n){int *p=malloc(4*n);int s=p[n];free(p);"
                   "return s;}\n")
    lib = tmp_path / "libbad.so"
    subprocess.run(["gcc", "-O0", "-g", "-fsanitize=address,undefined", "-fPIC", "-shared",
                    str(src), "-o", str(lib)], check=True)
    code = f"import ctypes; ctypes.CDLL({str(lib)!r}).bad(4)"
    r = subprocess.run([sys.executable, "-c", code], env=_env(_gcc_runtime()),
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr


def test_oracle_and_generator_under_asan_ubsan():
    oracle.build(sanitize=True)
    synth.build(sanitize=True)
    check = textwrap.dedent("""
        import sys, pytest, oracle, synth
        assert oracle._LIB_PATH.endswith("_san.so") and synth._LIB_PATH.endswith("_san.so")
        sys.exit(pytest.main(["-q", "-p", "no:cacheprovider", "-m", "not gpu"] + sys.argv[1:]))
    """)
    tests = ["test_oracle_pins.py", "test_oracle_backward_pins.py", "test_oracle_window_pins.py",
             "test_oracle_block_pins.py", "test_oracle_varlen.py", "test_synth.py"]
    r = subprocess.run([sys.executable, "-c", check] + [os.path.join(ROOT, "tests", t) for t in tests],
                       env=_env(_gcc_runtime(), PLX_SANITIZED_HOST_LIBS="1",
                                PYTHONPATH=ROOT + os.pathsep + os.path.join(ROOT, "tests")),
                       capture_output=True, text=True, timeout=900, cwd=ROOT)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr


def test_abi_host_checks_under_asan_ubsan():
    lib = hip_build.build_host_sanitized()
    check = textwrap.dedent(f"""
        import sys, pytest
        import parameterized_local_linear_amd as plx
        plx.LIB_PATH = {lib!r}
        sys.exit(pytest.main(["-q", "-p", "no:cacheprovider", "-m", "not gpu", sys.argv[1]]))
    """)
    r = subprocess.run([sys.executable, "-c", check, os.path.join(ROOT, "tests", "test_abi.py")],
                       env=_env(hip_build.asan_runtime(),
                                PYTHONPATH=ROOT + os.pathsep + os.path.join(ROOT, "tests")),
                       capture_output=True, text=True, timeout=600, cwd=ROOT)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
