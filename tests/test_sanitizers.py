"""AddressSanitizer + UBSan builds of the host code (CPU only).

Two builds, each loaded into its own Python process with the matching ASan
runtime preloaded, run the CPU tests that exercise them:
  - libpw's host sources (argument checks, page-table and workspace handling,
    launch sequencing up to the first HIP call, the greedy planner), built by
    hipcc with the sanitizers on the host side only, under tests/test_abi.py
    and tests/test_planner.py;
  - the oracle (gcc), under tests/test_oracle_pins.py and the planner pins.
Any ASan report or UBSan diagnostic aborts the child process, which fails the
test. The builds go to a temporary directory, never into the tree.
"""
import importlib.util
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _builder():
    spec = importlib.util.spec_from_file_location("_pw_build_san", os.path.join(ROOT, "any_precision_bit_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _run(args, env, timeout=600):
    res = subprocess.run([sys.executable] + args, cwd=ROOT, env=env, capture_output=True, text=True,
                         timeout=timeout)
    assert res.returncode == 0, (res.stdout[-4000:] + "\n" + res.stderr[-6000:])
    return res.stdout


def _instrumented(lib):
    out = subprocess.run(["nm", "-D", lib], capture_output=True, text=True, check=True).stdout
    return "__asan_report" in out and "__ubsan_handle" in out


def test_host_abi_under_asan_ubsan(tmp_path):
    b = _builder()
    lib = b.build_sanitized(str(tmp_path))
    assert _instrumented(lib)
    env = dict(os.environ, LD_PRELOAD=b.asan_runtime(), PW_LIBRARY=lib, **SAN_ENV)
    # the sanitized library (and the ASan runtime) is what the binding loaded
    _run(["-c", "import any_precision_bit_amd.binding as B; m = open('/proc/self/maps').read(); "
          "assert B.LIB_PATH.endswith('libpw_san.so') and 'libpw_san.so' in m and 'libclang_rt.asan' in m"],
         env)
    out = _run(["-m", "pytest", "tests/test_abi.py", "tests/test_planner.py", "-q", "-m", "not gpu",
                "-p", "no:cacheprovider"], env)
    assert " passed" in out


def test_oracle_under_asan_ubsan(tmp_path):
    import oracle

    lib = oracle.build_sanitized(str(tmp_path))
    assert _instrumented(lib)
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True,
                          check=True).stdout.strip()
    if not os.path.isabs(asan):
        pytest.skip("gcc's libasan.so not found")
    env = dict(os.environ, LD_PRELOAD=asan, ORACLE_LIBRARY=lib, **SAN_ENV)
    _run(["-c", "import oracle; oracle.lib(); m = open('/proc/self/maps').read(); "
          "assert 'liboracle_san.so' in m and 'libasan' in m"], env)
    out = _run(["-m", "pytest", "tests/test_oracle_pins.py", "tests/test_planner.py", "-q", "-m", "not gpu",
                "-p", "no:cacheprovider"], env)
    assert " passed" in out
