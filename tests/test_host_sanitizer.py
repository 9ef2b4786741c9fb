"""The C ABI's host code (argument checks, workspace carving, dispatch) under AddressSanitizer and
UndefinedBehaviorSanitizer: the CPU ABI checks run again, in a child process, against a library whose host pass
is instrumented. Any invalid memory access or undefined behaviour aborts the child. CPU only."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_checks_pass_under_host_sanitizers():
    if subprocess.run(["which", "hipcc"], capture_output=True).returncode != 0:
        pytest.skip("hipcc is not installed")
    from activation_sparse_ffn_predictor_amd import build_sanitized as bs
    lib = bs.build()
    env = bs.sanitizer_env()
    probe = ("from activation_sparse_ffn_predictor_amd import _lib; _lib.lib(); "
             "m = open('/proc/self/maps').read(); "
             "assert 'libclang_rt.asan' in m and 'libsffn_san.so' in m, 'sanitized library not loaded'")
    r = subprocess.run([sys.executable, "-c", probe], env=env, cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert "passed" in r.stdout and "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr
    assert os.path.exists(lib)
