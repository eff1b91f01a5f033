"""The C ABI from plain C: tests/abi_smoke.c (built by __graft_entry__.build()
into tests/abi_smoke.bin) allocates device memory with the HIP runtime's C
API, drives libsq with no Python in between, and checks closed forms of the
step (write into a row, readout, slot check, argument errors)."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

BIN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "abi_smoke.bin")


def test_plain_c_caller():
    if not os.path.exists(BIN):
        pytest.skip("tests/abi_smoke.bin is not built (run __graft_entry__.build())")
    r = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr)
    assert r.returncode == 0, r.stderr
    assert "abi_smoke ok" in r.stdout
