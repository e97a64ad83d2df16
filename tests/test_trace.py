"""ATTN_TRACE on the host (no GPU): with the variable set, an entry point that
returns before any launch (argument rejected, or nothing to do) writes one
"attn: " line naming itself and its status; without it, nothing.  The planned
kernel lines of calls that launch are checked on the GPU (test_gpu_trace.py)
and, for their formatting, by the sanitizer build of the host checks."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

PROG = r"""
import ctypes, sys
sys.path.insert(0, sys.argv[1])
import tiled_online_softmax_fwd_amd as A
L = A.lib()
P = lambda a: ctypes.c_void_p(a)
# head size 96: rejected before any HIP call
r1 = L.attn_fwd(P(0x10000), P(0x20000), P(0x30000), P(0x40000), None, 1, 2, 8, 96, ctypes.c_float(0.125), 0, None,
                A.BF16, None)
# no rows: nothing to launch
r2 = L.attn_fwd(None, None, None, None, None, 0, 2, 8, 128, ctypes.c_float(0.125), 0, None, A.BF16, None)
# decode without a workspace: rejected with the size it needs (one chunk of the
# 64 keys for each of 2 heads: 2 x (128 + 1) floats)
r3 = L.attn_decode_fwd(P(0x10000), P(0x20000), P(0x30000), P(0x40000), None, 1, 2, 1, 64, 128,
                       ctypes.c_float(0.125), 1, None, A.BF16, None, None, ctypes.c_size_t(0), 0)
print(r1, r2, r3)
"""


def run(trace):
    env = dict(os.environ)
    env.pop("ATTN_TRACE", None)
    if trace is not None:
        env["ATTN_TRACE"] = trace
    r = subprocess.run([sys.executable, "-c", PROG, ROOT], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stderr
    return r.stdout.split(), [l for l in r.stderr.splitlines() if l.startswith("attn: ")]


def test_trace_lines_for_calls_that_launch_nothing():
    codes, lines = run("1")
    assert codes == ["3", "0", "10"]
    assert lines == ["attn: attn_fwd returned ATTN_ERR_HEAD_DIM: head size d=96, supported: 64, 128",
                     "attn: attn_fwd nothing to launch (empty)",
                     "attn: attn_decode_fwd returned ATTN_ERR_WORKSPACE: workspace needs 1032 bytes, 16-byte aligned"]


def test_trace_off_by_default_and_with_zero():
    for val in (None, "", "0"):
        codes, lines = run(val)
        assert codes == ["3", "0", "10"]
        assert lines == []
