"""The library driven from plain C (tests/c/abi_check.c): no Python binding and
no torch in the caller.  The program checks two closed forms of softmax
attention (q = 0 gives the mean of the V rows; one dominant key gives its V
row, the key being a token the program appended through the slot mapping)."""
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
BIN = os.path.join(HERE, "c", "abi_check")


@pytest.mark.gpu
def test_plain_c_caller_append_and_decode():
    if not os.path.exists(BIN):
        pytest.fail("tests/c/abi_check is missing: run __graft_entry__.build() first")
    print("running", BIN, flush=True)
    r = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    sys.stdout.write(r.stdout)
    sys.stderr.write(r.stderr)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "abi_check: pass" in r.stdout
    assert "head_dim 96 refused" in r.stdout
