"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

The library's host-side sources (argument checks, planning, workspace sizing, the
allocation-free entry's fit, the block-table and combine launchers) are built with both
sanitizers on the host side only; tests/hostsan/launch_stub.hip stands in for the
split-KV launcher, whose kernels no CPU test reaches.  tests/test_abi.py then runs
against that build in a child process with the sanitizer runtime preloaded, so an
out-of-bounds access, a use after free or undefined behaviour in any host path those
tests drive aborts the child and fails this test."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
STUB = os.path.join(ROOT, "tests", "hostsan", "launch_stub.hip")


def test_abi_tests_clean_under_host_sanitizers(tmp_path):
    from speculative_decoding_verify_02_amd import build as build_mod
    try:
        build_mod.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not found")
    runtime = build_mod.sanitizer_runtime()
    if runtime is None:
        pytest.skip("no shared AddressSanitizer runtime next to hipcc's clang")
    lib = str(tmp_path / "libverify_attn_hostsan.so")
    build_mod.build_host_sanitized(lib, [STUB])
    # the build carries the instrumentation: ASan's checks and UBSan's handlers
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report_load" in syms and "__ubsan_handle" in syms

    # reports go to files (the child's pytest captures its own stderr)
    logs = tmp_path / "reports"
    logs.mkdir()
    env = dict(os.environ, LD_PRELOAD=runtime, VERIFY_ATTN_LIB=lib,
               ASAN_OPTIONS=f"detect_leaks=0:exitcode=86:log_path={logs}/asan",
               UBSAN_OPTIONS=f"print_stacktrace=1:halt_on_error=1:exitcode=87:log_path={logs}/ubsan")
    res = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"),
                          "-q", "-m", "not gpu", "-p", "no:cacheprovider"],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = res.stdout + res.stderr
    reports = "".join(f.read_text() for f in sorted(logs.iterdir()))
    assert not reports, reports[-4000:]
    assert res.returncode == 0, out[-4000:]
    assert " passed" in out and "failed" not in out, out[-2000:]
