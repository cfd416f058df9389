"""The C ABI from a plain host program: no Python binding and no torch.  The
program (tests/c_abi/mep_c_roundtrip.cpp, built by __graft_entry__.build())
allocates device memory with the HIP runtime, runs plan+dispatch (fused and
separate, one and two plan launches) and combine through the mep_* entry
points on the default stream, including the 128-token x 7168 decode shape,
and compares every output with the CPU oracle: bit-exact receive data,
combine within 1 bf16 ulp.  It runs as a child process; a second run reports
the host time of the ABI calls themselves (no Python) at the decode shape."""

import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

BIN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "mep_c_roundtrip")


def test_c_program_round_trip():
    assert os.path.exists(BIN), f"{BIN} is missing: build it with __graft_entry__.build()"
    r = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0, r.stderr
    assert "c_abi ok" in r.stdout


def test_c_program_host_cost():
    assert os.path.exists(BIN), f"{BIN} is missing: build it with __graft_entry__.build()"
    r = subprocess.run([BIN, "--host-cost"], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0, r.stderr
    assert "host us per call" in r.stdout
