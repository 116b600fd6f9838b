"""Seeded random problems across the parameter space (R from 1 to 64, any E multiple of R,
K up to min(E, 32), S from 1, slot budgets from 0 to E/R + 4, routing from balanced to
maxvio 30), each planned, dispatched and combined on the GPU and compared with the oracle:
plan arrays, dst_row and dispatched rows bit-exact, combine bit-exact (same fp32 order).
Small sizes keep the oracle fast; the spread covers the planner's paths (no shedding,
placement entirely by the parallel cut, cut then one expert at a time, fallback pieces)."""

import numpy as np
import pytest
import torch

import combine_top_id_amd as M
from gen import make_routing, make_hidden, bf16_bits, bits_to_bf16
from oracle import moonep_oracle as O
from tests.gpu_util import say, read_plan, assert_plan_matches, to_dev_ids

pytestmark = pytest.mark.gpu

N_CASES = 240


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    M.lib()


def _case(rng):
    R = int(rng.choice([1, 2, 3, 4, 5, 8, 12, 16, 32, 64]))
    E = R * int(rng.choice([1, 2, 3, 4, 8, 16]))
    E = min(E, 1024 - 1024 % R)
    K = int(rng.integers(1, min(E, 32) + 1))
    S = int(rng.integers(1, 120))
    slots = int(rng.integers(0, E // R + 5))
    H = 8 * int(rng.integers(1, 9))
    mv = float(rng.choice([0.05, 0.5, 1.0, 3.0, 8.0, 30.0]))
    return R, E, K, S, slots, H, mv


def test_random_problems():
    rng = np.random.default_rng(20261203)
    kinds = {"no pieces": 0, "slot pieces only": 0, "fallback pieces": 0}
    for n in range(N_CASES):
        R, E, K, S, slots, H, mv = _case(rng)
        seed = 31000 + n
        say(f"fuzz {n}: R={R} E={E} K={K} S={S} slots={slots} H={H} maxvio={mv}")
        ids, wt, _, _ = make_routing(R, E, K, S, mv, seed)
        ids_np, w_np = ids.numpy(), wt.numpy()
        plan = M.moonep_plan(*to_dev_ids(ids_np, w_np), R, E, K, S, slots)
        p = O.plan(ids_np, R, E, K, S, slots)
        dst = O.slot_map(p, ids_np)
        assert_plan_matches(read_plan(plan), p, dst)
        x = make_hidden(R * S, H, seed + 1, device="cuda")
        recv = M.moonep_dispatch(plan, x)
        ref = O.dispatch(dst, bf16_bits(x), plan.sz.recv_rows)
        rows = dst.reshape(-1)
        got = bf16_bits(recv)
        assert (got[rows] == ref[rows]).all(), f"case {n}: dispatched rows"
        out = M.moonep_combine(plan, bits_to_bf16(ref, "cuda"))
        assert (bf16_bits(out) == O.combine(dst, w_np, ref)).all(), f"case {n}: combine"
        if p.n_pieces == 0:
            kinds["no pieces"] += 1
        elif p.n_fallback == 0:
            kinds["slot pieces only"] += 1
        else:
            kinds["fallback pieces"] += 1
    torch.cuda.synchronize()
    say(f"fuzz kinds: {kinds}")
    assert all(v > 0 for v in kinds.values()), kinds
