"""The C ABI used from plain C: tests/capi/capi_check (built by
__graft_entry__.build()) drives every entry point of include/ddp.h on device
memory from hipMalloc, without Python or torch, and compares each result
with the oracle's C core bit for bit."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

BIN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "capi", "capi_check")


def test_c_abi_program_matches_oracle():
    assert os.path.exists(BIN), "tests/capi/capi_check is not built; run __graft_entry__.build()"
    print("running", BIN, flush=True)
    r = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "capi ok" in r.stdout
