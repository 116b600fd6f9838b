"""Independent problems planned, dispatched and combined at the same time from two host
threads on two streams give the same bits as the same calls run one after another: the
library keeps no global mutable state, and each call touches only the buffers it is
given.  Streams are created at the default priority."""

import threading

import pytest
import torch

import combine_top_id_amd as M
from gen import make_routing, make_hidden
from tests.gpu_util import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    M.lib()


PROBLEMS = [(8, 64, 6, 300, 8, 512, 3.0, 61), (4, 16, 2, 500, 4, 256, 1.0, 62),
            (16, 128, 8, 100, 2, 1024, 8.0, 63)]


def _inputs(p):
    R, E, K, S, slots, H, mv, seed = p
    ids, w, _, _ = make_routing(R, E, K, S, mv, seed, device="cuda")
    x = make_hidden(R * S, H, seed + 1, device="cuda")
    return ids, w, x


def _step(p, ids, w, x):
    R, E, K, S, slots, H, mv, seed = p
    plan = M.moonep_plan(ids, w, R, E, K, S, slots)
    recv = M.moonep_dispatch(plan, x)
    out = M.moonep_combine(plan, recv)
    return plan.dst_row.clone(), out


def test_concurrent_streams_match_sequential():
    inputs = [_inputs(p) for p in PROBLEMS]
    ref = [_step(p, *inp) for p, inp in zip(PROBLEMS, inputs)]
    torch.cuda.synchronize()
    results = [None] * len(PROBLEMS)
    errors = []
    start = threading.Barrier(len(PROBLEMS))

    def worker(j):
        try:
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.default_stream())
            with torch.cuda.stream(s):
                start.wait()
                outs = []
                for _ in range(4):
                    outs.append(_step(PROBLEMS[j], *inputs[j]))
                s.synchronize()
            results[j] = outs
        except Exception as exc:     # reported on the main thread
            errors.append(exc)

    say(f"concurrent streams: {len(PROBLEMS)} threads x 4 steps")
    threads = [threading.Thread(target=worker, args=(j,)) for j in range(len(PROBLEMS))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not errors, errors
    torch.cuda.synchronize()
    for j, outs in enumerate(results):
        assert outs is not None, f"thread {j} did not finish"
        for dst, out in outs:
            assert torch.equal(dst, ref[j][0]), f"problem {j}: dst_row"
            assert torch.equal(out.view(torch.int16), ref[j][1].view(torch.int16)), f"problem {j}: out"
