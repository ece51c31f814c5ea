"""The C ABI from a plain C program (tests/c_abi_demo.c, no Python or PyTorch in the
process): gather and scatter through include/kvxfer.h, checked against the oracle's
C source linked into the same program, plus the allocator and a pinned ring."""
from __future__ import annotations

import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))


def test_c_program_uses_the_abi():
    exe = os.path.join(HERE, "c_abi_demo")
    assert os.path.exists(exe), "tests/c_abi_demo is not built: run __graft_entry__.build()"
    print("[c-abi] running tests/c_abi_demo", flush=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    print(r.stdout, flush=True)
    assert r.returncode == 0 and "c_abi_demo ok" in r.stdout, r.stdout + r.stderr
