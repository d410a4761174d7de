"""The C ABI from plain C++ (no Python, no torch): tests/c_client/hs_client runs resolve steps on hipMalloc'd
buffers and checks every step's outputs and tables on what the device returns."""
from __future__ import annotations

import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

BIN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_client", "hs_client")


def test_c_client_through_the_c_abi():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert os.path.exists(BIN), "the C client is not built (__graft_entry__.build() builds it)"
    res = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "consistent through the C ABI" in res.stdout
