"""The HT round trip driven through the C ABI by a plain C99 program (no
Python on its side): route, handle, FP8 dispatch, identity expert, combine.
Its inputs make every step exact, so it checks the output against the input
bit for bit, plus the receive count, the device error word and rejected
calls; it prints one line and exits 0 on success."""
import os
import subprocess

import pytest

from gpu_util import need_gpu, say

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLIENT = os.path.join(ROOT, "tests", "c_client", "ep_c_client")


def test_c_client_round_trip():
    need_gpu()
    if not os.path.exists(CLIENT):
        pytest.fail("tests/c_client/ep_c_client is missing: run __graft_entry__.build()")
    say("C client: HT round trip through the C ABI")
    r = subprocess.run([CLIENT], capture_output=True, text=True, timeout=120)
    say(r.stdout.strip())
    assert r.returncode == 0, r.stdout + r.stderr
    assert "ep_c_client: OK" in r.stdout
