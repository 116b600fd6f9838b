"""GPU parity of the staged (non-zero-copy) A/B mode: its staging buffer matches the
oracle's arrival-order rows and its results are bit-identical to zero-copy."""

import numpy as np
import pytest
import torch

import combine_top_id_amd as M
from gen import DSV3, make_routing, make_hidden, bf16_bits
from oracle import moonep_oracle as O
from tests.gpu_util import say, to_dev_ids

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    M.lib()


@pytest.mark.parametrize("R,E,K,S,slots,H,mv", [(4, 16, 2, 64, 4, 128, 2.0),
                                                (8, 64, 5, 300, 2, 1000, 4.0),
                                                (16, 64, 3, 200, 4, 8, 3.0)])
def test_staged_small(R, E, K, S, slots, H, mv):
    seed = 1300 + R + E + K
    say(f"staged R={R} E={E} K={K} S={S} slots={slots} H={H}")
    ids, wt, _, _ = make_routing(R, E, K, S, mv, seed)
    plan = M.moonep_plan(*to_dev_ids(ids.numpy(), wt.numpy()), R, E, K, S, slots)
    p = O.plan(ids.numpy(), R, E, K, S, slots)
    dst = O.slot_map(p, ids.numpy())
    x = make_hidden(R * S, H, seed + 1, device="cuda")
    stage = torch.empty(R * S * K, H, dtype=torch.bfloat16, device="cuda")
    recv = M.moonep_dispatch_staged(plan, x, stage=stage)
    ref_stage, ref_recv = O.dispatch_staged(dst, bf16_bits(x), plan.sz.recv_rows)
    assert (bf16_bits(stage) == ref_stage).all()
    rows = dst.reshape(-1)
    assert (bf16_bits(recv)[rows] == ref_recv[rows]).all()
    y = make_hidden(plan.sz.recv_rows, H, seed + 2, device="cuda")
    out = M.moonep_combine_staged(plan, y, stage=stage)
    _, ref_out = O.combine_staged(dst, wt.numpy(), bf16_bits(y))
    assert (bf16_bits(out) == ref_out).all()
    assert torch.equal(out, M.moonep_combine(plan, y))
    torch.cuda.synchronize()


def test_staged_full_size_equals_zero_copy():
    wl = DSV3
    say("staged full size dsv3 maxvio 20")
    ids, wt, _, _ = make_routing(wl.R, wl.E, wl.K, wl.S, 20.0, wl.seed(3), device="cuda")
    plan = M.moonep_plan(ids, wt, wl.R, wl.E, wl.K, wl.S, wl.slots)
    x = make_hidden(wl.T, wl.H, 77, device="cuda")
    r1 = M.moonep_dispatch(plan, x)
    r2 = torch.empty_like(r1)
    r2 = M.moonep_dispatch_staged(plan, x, recv=r2)
    d = plan.dst_row.reshape(-1).long()
    for c0 in range(0, d.numel(), 32768):
        sel = d[c0:c0 + 32768]
        assert torch.equal(r1[sel], r2[sel])
    del r2
    o1 = M.moonep_combine(plan, r1)
    o2 = M.moonep_combine_staged(plan, r1)
    assert torch.equal(o1, o2)
    torch.cuda.synchronize()
