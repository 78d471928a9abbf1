"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer: the
C-ABI layer of the library (argument validation, workspace sizing, dispatch)
and the C oracle are rebuilt with both sanitizers, and the CPU test files run
against those builds in a child process with the sanitizer runtime preloaded.
A sanitizer report ends the child with a failure.  (GPU code is not
instrumented: only the host side of the library is rebuilt.)"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CPU_TESTS = ["tests/test_abi.py", "tests/test_oracle_pins.py", "tests/test_oracle_quant_pins.py",
             "tests/test_oracle_linear_pins.py", "tests/test_synth.py"]


def test_cpu_suite_under_sanitizers(tmp_path):
    sys.path.insert(0, ROOT)
    from compressed_sparse_kv_csa_amd import build as B
    import oracle
    rt = B.sanitizer_runtime()
    if not rt:
        pytest.skip("no clang AddressSanitizer runtime in this toolchain")
    lib = B.build_sanitized(str(tmp_path))
    olib = oracle.build_sanitized(str(tmp_path))
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": rt,
        "ASAN_OPTIONS": "detect_leaks=0:detect_odr_violation=0:abort_on_error=1",
        "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1",
        "DSV4_LIB": lib,
        "DSV4_ORACLE_LIB": olib,
    })
    probe = ("import os, compressed_sparse_kv_csa_amd as K, oracle as O; K.lib(); O._L(); "
             "m = open('/proc/self/maps').read(); "
             "assert os.environ['DSV4_LIB'] in m and os.environ['DSV4_ORACLE_LIB'] in m, 'sanitizer builds not loaded'")
    subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, check=True, timeout=600)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu"] + CPU_TESTS,
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    print(r.stdout[-2000:])
    print(r.stderr[-4000:])
    assert r.returncode == 0, "CPU tests failed under the sanitizers"
