"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

Two drivers in tests/sanitize/ are built with gcc/g++ into a temporary
directory and run: host_san.cpp drives the library's argument checks, tile and
grid planning and trace formatting (csrc/attn_host.h, the same header
attn_api.cpp compiles) with fake pointers that must never be dereferenced;
oracle_san.c drives every routine of the fp64 oracle and of the precision
model on small ragged shapes and the argument errors.  Either driver fails on
the first sanitizer report (-fno-sanitize-recover) or on a failed expectation.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-g", "-O1", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]


def run(cmd, **kw):
    return subprocess.run(cmd, capture_output=True, text=True, timeout=300, **kw)


def env():
    e = dict(os.environ)
    # leak checks on; tolerate a preloaded library ahead of the runtime
    e["ASAN_OPTIONS"] = "detect_leaks=1:verify_asan_link_order=0:abort_on_error=0"
    e["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    e["OMP_NUM_THREADS"] = "2"
    return e


def build_and_run(tmp_path, compiler, sources, extra):
    if shutil.which(compiler) is None:
        pytest.skip(f"{compiler} not found")
    exe = str(tmp_path / "driver")
    b = run([compiler] + SAN + extra + [os.path.join(ROOT, s) for s in sources] + ["-o", exe, "-lm"])
    assert b.returncode == 0, b.stderr
    r = run([exe], env=env())
    assert r.returncode == 0, r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr
    return r.stdout


def test_host_checks_under_sanitizers(tmp_path):
    out = build_and_run(tmp_path, "g++", ["tests/sanitize/host_san.cpp"],
                        ["-std=c++17", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"),
                         "-I", os.path.join(ROOT, "tiled_online_softmax_fwd_amd", "csrc")])
    assert "all host checks passed" in out


def test_oracle_under_sanitizers(tmp_path):
    out = build_and_run(tmp_path, "gcc", ["oracle/oracle.c", "oracle/emulate.c", "tests/sanitize/oracle_san.c"],
                        ["-std=c11", "-Wall", "-Wextra", "-fopenmp", "-ffp-contract=off", "-fno-fast-math"])
    assert "all oracle checks passed" in out
