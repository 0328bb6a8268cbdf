"""The C ABI without Python: tests/c/abi_parity (built by
__graft_entry__.build() or tests/c/build.py) links librma.so and the C
oracle, runs lockstep decode across three admits and a prompt block on a
small geometry, and checks every output within the decode tolerance and
the whole history bit for bit (see tests/c/abi_parity.c)."""
import os
import subprocess

import pytest

import gpu_util as gu

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c", "abi_parity")


def test_c_program_through_the_c_abi_matches_the_oracle():
    gu.log("case C ABI program (tests/c/abi_parity)")
    assert os.path.exists(EXE), f"{EXE} is missing: run __graft_entry__.build() first"
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    print(r.stdout + r.stderr)
    assert r.returncode == 0, f"exit status {r.returncode}: {r.stderr.strip()}"
    assert "c abi parity ok" in r.stdout
