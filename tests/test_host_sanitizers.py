"""The host side of the library under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only).

The library is rebuilt with its host code sanitized (device code unchanged)
and the host-only ABI tests run against it in a child process that preloads
the sanitizer runtime: the descriptor checks, the split policy and split
rule, workspace layout, plan keys, and every argument error of run /
partials / merge / the no-allocation call.  Those cases return before any
kernel launch, so the real launchers are linked but never reached.  Any
sanitizer report, or a failing case, fails this test."""

import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


@pytest.mark.skipif(not os.path.exists("/opt/rocm/bin/hipcc") or _asan_runtime() is None,
                    reason="needs hipcc and the clang sanitizer runtime")
def test_abi_cases_under_host_sanitizers():
    sys.path.insert(0, ROOT)
    from split_kv_paged_page_amd.build import build_hostcheck
    lib = build_hostcheck()
    env = dict(os.environ)
    env.update(LD_PRELOAD=_asan_runtime(), SPLITKV_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    # -s: a sanitizer report goes to file descriptor 2, which pytest's capture
    # would swallow when the report ends the process
    cmd = [sys.executable, "-m", "pytest", "-q", "-s", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
           os.path.join(ROOT, "tests", "test_abi.py")]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in r.stdout and " failed" not in r.stdout, r.stdout[-2000:]
