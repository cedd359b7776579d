"""The C ABI's host code under AddressSanitizer: argument validation of every
entry point, create calls that fail after allocating their handle and release
it, and destroy of a null handle.  The library is rebuilt with the sanitizer
on its host code only (libflint_moe_asan.so; device code unchanged) and
exercised in a child process with the sanitizer runtime preloaded, so that a
heap overflow, use after free or double free in that code aborts the child
with a report.  These paths allocate no device memory, so they run without a
GPU (the sanitizer runtime's device-memory interceptor needs XNACK, which these
GPUs run without; partial releases on the device are checked by a GPU test).
"""
import os
import subprocess
import sys

import pytest

from int4_expert_ffn_amd import build as B

HERE = os.path.dirname(os.path.abspath(__file__))
SCRIPT = os.path.join(HERE, "asan_paths.py")


def _asan_env():
    runtime = B.asan_runtime()
    if not (os.path.isabs(runtime) and os.path.exists(runtime)):
        pytest.skip("the compiler's AddressSanitizer runtime is not installed")
    if not os.path.exists(B.LIB_ASAN):
        pytest.skip("libflint_moe_asan.so is not built (python -m int4_expert_ffn_amd.build --asan)")
    env = dict(os.environ)
    # the sanitizer runtime must come first; anything already preloaded stays
    env["LD_PRELOAD"] = ":".join(p for p in (runtime, os.environ.get("LD_PRELOAD", "")) if p)
    # leaks: the interpreter and the HIP runtime keep memory until exit by design;
    # new/delete pairing is checked in this library's code only by reading it,
    # since third-party runtime libraries loaded in the same process are not under test
    env["ASAN_OPTIONS"] = "detect_leaks=0:alloc_dealloc_mismatch=0:verify_asan_link_order=0:abort_on_error=1"
    env["FLINT_MOE_LIBRARY"] = B.LIB_ASAN
    env["HIP_VISIBLE_DEVICES"] = "-1"   # no device, also where one is installed
    env.pop("FLINT_MOE_FAIL_ALLOC", None)
    return env


def _run(args, timeout):
    r = subprocess.run([sys.executable, SCRIPT] + args, env=_asan_env(), capture_output=True, text=True,
                       timeout=timeout)
    report = r.stdout[-3000:] + r.stderr[-6000:]
    assert "AddressSanitizer" not in r.stderr, report
    assert r.returncode == 0 and "asan paths done" in r.stdout, report
    return r


def test_asan_build_instruments_host_code():
    if not os.path.exists(B.LIB_ASAN):
        pytest.skip("libflint_moe_asan.so is not built")
    syms = subprocess.run(["nm", "-D", "--undefined-only", B.LIB_ASAN], capture_output=True, text=True).stdout
    assert "__asan_report_load" in syms or "__asan_report_store" in syms
    assert "__asan_init" in syms


def test_host_paths_under_asan_without_device():
    r = _run([], timeout=600)
    assert r.stdout.count("ok ") == 7
