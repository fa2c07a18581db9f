"""The host side of the C ABI (argument validation, alias checks, workspace
planning) under AddressSanitizer and UndefinedBehaviorSanitizer.

tests/test_abi.py runs again in a child process against the host-sanitized
build of the same sources (orthogonal_equivalence_amd/_build/san, made by
`python -m orthogonal_equivalence_amd.build --sanitize`; the GPU code in it
is compiled as usual), with the sanitizer runtime preloaded into the
uninstrumented Python. A sanitizer report fails the child and this test.
CPU only, like test_abi.py.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _stale(lib: str) -> bool:
    if not os.path.exists(lib):
        return True
    srcs = glob.glob(os.path.join(ROOT, "orthogonal_equivalence_amd", "csrc", "*")) + \
        glob.glob(os.path.join(ROOT, "include", "*.h"))
    return max(os.path.getmtime(s) for s in srcs) > os.path.getmtime(lib)


def test_abi_under_host_sanitizers():
    import torch
    if torch.cuda.is_available():
        pytest.skip("host-validation tests use fake device addresses; run them without a GPU")
    from orthogonal_equivalence_amd import build as B
    try:
        B.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available to build the sanitized library")
    if _stale(B.SAN_LIB):
        B.build(sanitize=True)
    env = dict(os.environ)
    env.update(POETX_LIBRARY=B.SAN_LIB, LD_PRELOAD=B.sanitizer_runtime(),
               ASAN_OPTIONS="detect_leaks=0:detect_odr_violation=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    # the child really loads the sanitized build
    probe = subprocess.run(
        [sys.executable, "-c",
         "import orthogonal_equivalence_amd.poetx as P, sys; "
         "sys.exit(0 if 'libpoetx_san.so' in open('/proc/self/maps').read() else 3)"],
        cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert probe.returncode == 0, probe.stdout[-2000:] + probe.stderr[-2000:]
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout[-4000:] + r.stderr[-4000:]
    assert r.returncode == 0, out
    assert "passed" in r.stdout and "AddressSanitizer" not in out and "runtime error" not in out, out
