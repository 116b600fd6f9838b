"""The C ABI used from plain C (tests/c_abi/smoke.c, built with gcc against
include/moonep.h and libmoonep.so): host-only calls on the CPU, and a whole
plan -> dispatch -> combine -> status on the GPU whose results are checked exactly
(every rank holds S*K rows, each row once, dispatched rows equal x, and a combine of K
equal rows with weights 1/K returns x)."""

import os
import subprocess

import pytest

import combine_top_id_amd as M
from combine_top_id_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SMOKE = os.path.join(ROOT, "tests", "c_abi", "smoke")


@pytest.fixture(scope="module")
def smoke():
    if not os.path.exists(M.LIB_PATH):
        pytest.fail("libmoonep.so is not built (run __graft_entry__.build())")
    if not os.path.exists(SMOKE) or os.path.getmtime(SMOKE) < os.path.getmtime(M.LIB_PATH):
        B.build_c_smoke()
    return SMOKE


def test_c_consumer_host_calls(smoke):
    r = subprocess.run([smoke, "host"], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "host checks ok" in r.stdout


@pytest.mark.gpu
def test_c_consumer_gpu_run(smoke):
    print("C ABI smoke program on the GPU", flush=True)
    r = subprocess.run([smoke, "gpu"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "gpu run ok" in r.stdout
