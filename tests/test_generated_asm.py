"""The instruction-scheduled loops are generated: the committed headers must be
what their generators write (a hand edit of a header, or a generator change
not rerun, fails here)."""
import os
import subprocess
import sys

import pytest

CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "tiled_online_softmax_fwd_amd", "csrc")


@pytest.mark.parametrize("gen", ["gen_fwd_pipe.py", "gen_bwd_dq_pipe.py", "gen_bwd_dkdv_pipe.py"])
def test_header_matches_generator(gen):
    r = subprocess.run([sys.executable, os.path.join(CSRC, gen), "--check"], capture_output=True, text=True)
    assert r.returncode == 0, f"{gen}: header differs from the generator's output; rerun it"
