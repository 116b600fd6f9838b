"""CPU checks of bench.py's arithmetic and its one-GPU contract (no GPU needed).

The algorithmic byte counts are compared with figures worked out by hand from the
per-token formulas, dispatch (K+1)*2H + 4K and combine (K+1)*2H + 8K bytes, at the five
workloads' sizes; the percentile helper against numpy; and a request for more than one GPU
must exit with status 2 before touching a device."""

import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from gen import WORKLOADS  # noqa: E402


# (T, K, H) -> dispatch bytes, combine bytes, worked out by hand
HAND = {
    "tiny": (256, 2, 128, 256 * 3 * 256 + 256 * 8, 256 * 3 * 256 + 256 * 16),
    "r8-e64-k6": (8192, 6, 2048, 8192 * 7 * 4096 + 8192 * 24, 8192 * 7 * 4096 + 8192 * 48),
    "dsv3": (32768, 8, 7168, 4_228_907_008, 4_229_955_584),
    "kimi": (131072, 8, 7168, 16_915_628_032, 16_919_822_336),
    "decode": (8192, 8, 7168, 1_057_226_752, 1_057_488_896),
}


@pytest.mark.parametrize("wl", WORKLOADS, ids=lambda w: w.name)
def test_algorithmic_bytes(wl):
    T, K, H, d, c = HAND[wl.name]
    assert (wl.T, wl.K, wl.H) == (T, K, H)
    assert bench.dispatch_bytes(wl.T, wl.K, wl.H) == d
    assert bench.combine_bytes(wl.T, wl.K, wl.H) == c


def test_reduce_bytes_counts_slot_replicas_only():
    # expert 3: two slot replicas; expert 5: one; expert 7: a fallback piece only
    pieces = [(3, 1, 0), (3, 2, 0), (5, 4, 1), (7, 6, -1)]
    G = 1000
    assert bench.reduce_bytes(pieces, G) == (2 + 2) * 4 * G + (1 + 2) * 4 * G


@pytest.mark.parametrize("q", [0, 10, 50, 90, 100])
def test_percentile_matches_numpy(q):
    rng = np.random.default_rng(3)
    v = list(rng.normal(size=37))
    assert abs(bench.pctl(v, q) - float(np.percentile(v, q))) < 1e-12


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == ""
