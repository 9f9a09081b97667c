"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The library's host sources (argument validation, pool handles and descriptors, workspace carving,
the allocation-free entry point's per-device table) are rebuilt with the host pass instrumented
(``python -m decode_attention_paged_split_amd.build --sanitize``), and the ABI tests run against
that build in a child process with the sanitizer runtime preloaded: an out-of-bounds access, a
use after free or an undefined operation in any of their paths ends the child with a report."""
import os
import shutil
import subprocess
import sys

import pytest

from decode_attention_paged_split_amd import build as kbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def sanitized():
    if not (shutil.which("hipcc") or os.path.exists("/opt/rocm/bin/hipcc")):
        pytest.skip("hipcc not available")
    return kbuild.build_sanitized(verbose=False), kbuild.asan_runtime()


def _child(lib, rt, args):
    env = dict(os.environ)
    env.update(KVQ_LIB=lib, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:exitcode=86",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    return subprocess.run([sys.executable] + args, cwd=ROOT, env=env, capture_output=True, text=True,
                          timeout=600)


def test_sanitizer_is_live_in_the_child(sanitized):
    lib, rt = sanitized
    r = _child(lib, rt, ["-c", "import ctypes, decode_attention_paged_split_amd as k; L = k.lib(); "
                               "ctypes.CDLL(None).__asan_init; "
                               "print([l.split()[-1] for l in open('/proc/self/maps') if 'libkvq' in l][0])"])
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip().endswith("libkvq_san.so"), r.stdout


def test_abi_tests_pass_under_the_sanitizers(sanitized):
    lib, rt = sanitized
    r = _child(lib, rt, ["-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
                         os.path.join("tests", "test_abi.py")])
    out = r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in r.stdout, out[-2000:]
