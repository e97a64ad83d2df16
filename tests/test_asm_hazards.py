"""CPU: static check of the generated instruction-scheduled blocks (waits for
LDS reads, wait states after matrix, vector and transcendental ops, VCC and
permlane inputs, M0 before LDS DMA), by the dataflow analysis of
tests/asm_check.py over each block's control flow, loops included.

The analysis is also run on copies of the blocks with a fault planted (a wait
or a no-op removed), which it must report: a checker that cannot fail would
prove nothing.
"""
import os
import re

import pytest

from tests import asm_check as ac

CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "tiled_online_softmax_fwd_amd", "csrc")
HEADERS = ["fwd_pipe_asm.h", "bwd_dq_pipe_asm.h", "bwd_dkdv_pipe_asm.h"]


def blocks():
    out = []
    for h in HEADERS:
        with open(os.path.join(CSRC, h)) as f:
            for name, lines in ac.macros(f.read()).items():
                out.append((h, name, lines))
    return out


def test_every_header_has_both_blocks():
    names = {(h, n) for h, n, _ in blocks()}
    assert len(names) == 6, names


@pytest.mark.parametrize("h,name,lines", blocks(), ids=lambda x: x if isinstance(x, str) else "")
def test_block_has_no_hazard(h, name, lines):
    errors = ac.check(lines, name)
    assert not errors, "\n".join(errors[:20])


def _first(lines, pred, start=0):
    for i in range(start, len(lines)):
        if pred(lines[i]):
            return i
    raise AssertionError("no such line")


def _loop_start(lines):
    return _first(lines, lambda ln: ln == "4:")


@pytest.mark.parametrize("h", HEADERS)
def test_planted_faults_are_reported(h):
    """Each fault below makes a real block wrong; the check must say so."""
    with open(os.path.join(CSRC, h)) as f:
        lines = next(iter(ac.macros(f.read()).values()))
    assert not ac.check(lines)
    body = _loop_start(lines)

    # an LDS read used without its wait: drop the first partial lgkmcnt wait
    # in the loop (a wait that retires some, not all, reads)
    i = _first(lines, lambda ln: re.fullmatch(r"s_waitcnt lgkmcnt\([1-9]\d*\)", ln) is not None, body)
    assert ac.check(lines[:i] + lines[i + 1:]), "missing LDS wait not reported"

    # the wait states after the block's last matrix ops: drop the final no-ops
    j = len(lines) - 1
    while lines[j].startswith("s_nop"):
        j -= 1
    assert j < len(lines) - 1
    assert ac.check(lines[:j + 1]), "matrix results read too early after the block not reported"

    # M0 written right before an LDS DMA
    k = _first(lines, lambda ln: ln.startswith("global_load_lds"), body)
    assert lines[k - 1] == "s_nop 0"
    assert ac.check(lines[:k - 1] + lines[k:]), "M0 -> LDS DMA hazard not reported"

    # a vector op right behind the matrix op whose result it reads: move the
    # first vector op that reads a matrix result up behind that matrix op
    mf = [n for n, ln in enumerate(lines) if ln.startswith("v_mfma") and n > body]
    planted = False
    for m in mf:
        dst = ac.Ins(lines[m]).writes
        for n in range(m + 1, min(m + 200, len(lines))):
            ins = ac.Ins(lines[n])
            if ins.kind in ("valu", "trans") and ins.reads & dst and not lines[n].startswith("s_"):
                moved = lines[:m + 1] + [lines[n]] + lines[m + 1:n] + lines[n + 1:]
                assert ac.check(moved), "vector read of a fresh matrix result not reported"
                planted = True
                break
            if ac.Ins(lines[n]).kind == "mfma" and ac.Ins(lines[n]).writes & dst:
                break
        if planted:
            break
    assert planted, "no vector consumer of a matrix result found to plant the fault"
