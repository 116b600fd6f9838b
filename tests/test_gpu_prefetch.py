"""GPU parity of replica weight prefetch and of the expert stub's weight routing (home
group: home weights; slot group: the prefetched copy; fallback piece: home weights read
across partitions) against the CPU oracle.  Both are bit copies or single roundings:
bit-exact."""

import numpy as np
import pytest
import torch

import combine_top_id_amd as M
from gen import DSV3, DECODE, make_routing, make_hidden, bf16_bits
from oracle import moonep_oracle as O
from tests.gpu_util import say, to_dev_ids

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    M.lib()


@pytest.mark.parametrize("R,E,K,S,slots,H,W_el,mv", [
    (4, 16, 2, 64, 4, 128, 136, 2.0),
    (8, 64, 5, 300, 2, 64, 4096, 4.0),       # slots bind: fallback pieces
    (64, 384, 8, 40, 4, 128, 128, 20.0),
    (8, 64, 6, 200, 0, 16, 24, 3.0),         # no slots at all
])
def test_prefetch_and_stub_small(R, E, K, S, slots, H, W_el, mv):
    seed = 900 + R + E + K
    say(f"prefetch/stub R={R} E={E} K={K} S={S} slots={slots} H={H} W_el={W_el}")
    ids, wt, _, _ = make_routing(R, E, K, S, mv, seed)
    ids_np = ids.numpy()
    ids_d, w_d = to_dev_ids(ids_np, wt.numpy())
    plan = M.moonep_plan(ids_d, w_d, R, E, K, S, slots)
    p = O.plan(ids_np, R, E, K, S, slots)
    dst = O.slot_map(p, ids_np)
    home_w = make_hidden(E, W_el, seed + 1, device="cuda")
    slot_w = torch.full((R, slots, W_el), float("nan"), dtype=torch.bfloat16, device="cuda")
    M.moonep_prefetch_weight(plan, home_w, slot_w)
    ref_slot = O.prefetch_weight(p, bf16_bits(home_w))
    got = bf16_bits(slot_w)
    used = np.zeros((R, slots), dtype=bool)
    for (e, r, sl, cnt, start, fb) in p.pieces:
        if sl >= 0:
            used[r, sl] = True
    assert (got[used] == ref_slot[used]).all(), "prefetched slots"
    assert np.isnan(O.bf16_to_f32(got[~used])).all(), "unused slots must not be written"

    x = make_hidden(R * S, H, seed + 2, device="cuda")
    recv = M.moonep_dispatch(plan, x)
    y = torch.full_like(recv, float("nan"))
    M.moonep_expert_stub(plan, ids_d, recv, home_w, slot_w, y)
    ref_y = O.expert_stub(p, bf16_bits(recv), bf16_bits(home_w), ref_slot, H)
    rows = dst.reshape(-1)
    assert (bf16_bits(y)[rows] == ref_y[rows]).all(), "expert stub"
    torch.cuda.synchronize()


@pytest.mark.parametrize("wl,mi", [(DSV3, 3), (DECODE, 0)], ids=lambda v: getattr(v, "name", str(v)))
def test_prefetch_and_stub_full_size(wl, mi):
    """Full size: every used slot equals its home slab, and every assignment's stub output
    equals the no-replication result x[t] * home_w[e][:H] (checked with torch on the GPU)."""
    seed = wl.seed(mi)
    say(f"prefetch/stub full size {wl.name} maxvio={wl.maxvio[mi]}")
    ids, wt, _, _ = make_routing(wl.R, wl.E, wl.K, wl.S, wl.maxvio[mi], seed, device="cuda")
    plan = M.moonep_plan(ids, wt, wl.R, wl.E, wl.K, wl.S, wl.slots)
    st = M.moonep_plan_status(plan)
    W_el = wl.H * 2
    home_w = make_hidden(wl.E, W_el, seed + 1, device="cuda")
    slot_w = M.moonep_prefetch_weight(plan, home_w)
    pieces = plan.array("pieces", plan.sz.P_max * 8).view(-1, 8)[:st["n_pieces"]].cpu().numpy()
    n_slot = 0
    for (e, r, sl) in pieces[:, :3]:
        if sl >= 0:
            assert torch.equal(slot_w[r, sl], home_w[e])
            n_slot += 1
    assert n_slot == st["n_replicas"]
    x = make_hidden(wl.T, wl.H, seed + 2, device="cuda")
    recv = M.moonep_dispatch(plan, x)
    y = M.moonep_expert_stub(plan, ids, recv, home_w, slot_w)
    d = plan.dst_row.long()
    for c0 in range(0, wl.T, 2048):
        c1 = min(c0 + 2048, wl.T)
        got = y[d[c0:c1].reshape(-1)].view(c1 - c0, wl.K, wl.H)
        ref = (x[c0:c1, None, :].float() * home_w[ids[c0:c1].long(), :wl.H].float()).to(torch.bfloat16)
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
    if wl.slots < wl.E // wl.R:
        assert st["n_fallback"] > 0      # the decode batch does exercise fallback reads
    torch.cuda.synchronize()
