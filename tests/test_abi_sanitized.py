"""The host side of the C ABI (argument validation, launch planning, error
reporting) under AddressSanitizer and UndefinedBehaviorSanitizer: the CPU ABI
tests run again, in a child process, against libpf_asan.so (the library built
with both sanitizers on its host code) with the ASan runtime preloaded. Any
sanitizer report fails the child, and so this test. No GPU is used."""
import glob
import importlib.util
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "bounded_kv_cache_pf_amd")


def _build_module():
    spec = importlib.util.spec_from_file_location("_pf_build_san", os.path.join(PKG, "build.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    return b


def test_host_abi_under_address_and_ub_sanitizers():
    b = _build_module()
    runtime = b.asan_runtime()
    if not runtime:
        pytest.skip("the compiler's AddressSanitizer runtime is not installed")
    sources = glob.glob(os.path.join(PKG, "csrc", "*")) + glob.glob(os.path.join(ROOT, "include", "*.h"))
    if not os.path.exists(b.ASAN_LIB) or os.path.getmtime(b.ASAN_LIB) < max(os.path.getmtime(s) for s in sources):
        b.build(sanitize=True)
    env = dict(os.environ, LD_PRELOAD=runtime, PF_LIBRARY=b.ASAN_LIB,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    # the sanitizer runtime is live in the child and the sanitized library is the one loaded
    probe = ("import ctypes, bounded_kv_cache_pf_amd as pf; "
             "assert hasattr(ctypes.CDLL(None), '__asan_report_load1'); "
             "assert pf.LIB_PATH.endswith('libpf_asan.so'); print('sanitized')")
    r = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and "sanitized" in r.stdout, r.stdout + r.stderr
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-3000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-3000:]
