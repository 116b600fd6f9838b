"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bar: plan arrays, dst_row, copied weights and dispatched rows bit-exact; combine within
rtol 1e-2 (bf16 output) and reduce within rtol 1e-5 (fp32), both also expected to be
bit-exact because the kernels round each product and sum in the oracle's order.
Small workloads are compared element by element; the full-size workloads compare every
plan array, every dst_row, every dispatched row (and that padding rows stay untouched),
every combined token and every reduced expert.
"""

import json
import os

import numpy as np
import pytest
import torch

import combine_top_id_amd as M
from gen import (TINY, SMALL, DSV3, KIMI, DECODE, make_routing, make_balanced_routing,
                 make_hidden, make_scales, make_grads, bf16_bits, bits_to_bf16)
from oracle import moonep_oracle as O
from tests.gpu_util import say, read_plan, assert_plan_matches, to_dev_ids
from tests.tol import assert_close, RTOL_BF16, RTOL_FP32
from tests import adversarial

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    M.lib()   # raises if the HIP library is missing: no fallback


def full_case(R, E, K, S, slots, H, ids_np, w_np, seed, G_el=0, scale_expert=True):
    """Every stage at a size the oracle handles whole; element-by-element comparison."""
    say(f"case R={R} E={E} K={K} S={S} slots={slots} H={H} seed={seed} G_el={G_el}")
    T = R * S
    ids, w = to_dev_ids(ids_np, w_np)
    plan = M.moonep_plan(ids, w, R, E, K, S, slots)
    st = M.moonep_plan_status(plan)
    p = O.plan(ids_np, R, E, K, S, slots)
    dst = O.slot_map(p, ids_np)
    got = read_plan(plan)
    assert_plan_matches(got, p, dst)
    assert st["n_pieces"] == p.n_pieces and st["status"] == 0
    assert (got["w"].view(np.uint32) == np.asarray(w_np, np.float32).view(np.uint32)).all()

    # dispatch
    x = make_hidden(T, H, seed + 1, device="cuda")
    x_np = bf16_bits(x)
    recv = torch.full((plan.sz.recv_rows, H), float("nan"), dtype=torch.bfloat16, device="cuda")
    M.moonep_dispatch(plan, x, recv)
    recv_np = bf16_bits(recv)
    ref = O.dispatch(dst, x_np, plan.sz.recv_rows)
    rows = dst.reshape(-1)
    assert (recv_np[rows] == ref[rows]).all(), "dispatched rows"
    untouched = np.ones(plan.sz.recv_rows, dtype=bool)
    untouched[rows] = False
    assert (recv_np[untouched] == bf16_bits(torch.tensor([float("nan")], dtype=torch.bfloat16))[0]).all(), \
        "padding rows must not be written"

    # combine through a toy expert: y = bf16(s_e * x) on the rows of expert e (test stub)
    y_np = ref.copy()
    if scale_expert:
        s = make_scales(E, seed + 2).numpy()
        exp_of_row = np.full(plan.sz.recv_rows, -1)
        exp_of_row[rows] = np.asarray(ids_np).reshape(-1)
        m = exp_of_row >= 0
        y_np[m] = O.f32_to_bf16_rne(s[exp_of_row[m]][:, None] * O.bf16_to_f32(ref[m]))
    y = bits_to_bf16(y_np, "cuda")
    out = M.moonep_combine(plan, y)
    out_np = bf16_bits(out)
    ref_out = O.combine(dst, w_np, y_np)
    assert_close(O.bf16_to_f32(out_np), O.bf16_to_f32(ref_out), RTOL_BF16)
    assert (out_np == ref_out).all(), "combine expected bit-exact (same fp32 op order)"

    # reduce
    if G_el and slots:
        home, rep = make_grads(E, R, slots, G_el, seed + 3, device="cuda")
        home_np, rep_np = home.cpu().numpy(), rep.cpu().numpy()
        M.moonep_reduce_grad(plan, home, rep)
        ref_home = O.reduce_grad(p, home_np, rep_np)
        got_home = home.cpu().numpy()
        assert_close(got_home, ref_home, RTOL_FP32)
        assert (got_home.view(np.uint32) == ref_home.view(np.uint32)).all(), "reduce bit-exact"
    torch.cuda.synchronize()
    return p


# ----------------------------------------------------------------------------------------
# small workloads, element by element
# ----------------------------------------------------------------------------------------

def test_tiny_workload():
    w = TINY
    ids, wt, _, _ = make_routing(w.R, w.E, w.K, w.S, w.maxvio[0], w.seed(0))
    p = full_case(w.R, w.E, w.K, w.S, w.slots, w.H, ids.numpy(), wt.numpy(), w.seed(0), G_el=64)
    assert p.n_pieces > 0


def test_small_workload():
    w = SMALL
    ids, wt, _, _ = make_routing(w.R, w.E, w.K, w.S, w.maxvio[0], w.seed(0))
    full_case(w.R, w.E, w.K, w.S, w.slots, w.H, ids.numpy(), wt.numpy(), w.seed(0), G_el=256)


CASES = [
    # R, E, K, S, slots, H, maxvio     (ragged H, odd K, binding slots, several blocks)
    (2, 4, 1, 3, 1, 8, 0.5),
    (3, 6, 2, 5, 1, 136, 1.0),
    (4, 16, 3, 100, 2, 1000, 3.0),
    (8, 64, 5, 300, 2, 2056, 4.0),     # slots bind -> fallback pieces
    (8, 64, 8, 1000, 0, 64, 2.0),      # no slots at all: everything shed is fallback
    (16, 64, 4, 700, 4, 520, 6.0),
    (64, 384, 8, 40, 4, 128, 20.0),    # decode-like, R = 64 lanes
    (1, 8, 2, 257, 3, 24, 1.0),        # one rank: no pieces
    (5, 10, 10, 33, 2, 8, 0.0001),     # K = E: every token takes every expert
    (8, 32, 7, 2049, 4, 16, 2.5),      # several map blocks with a ragged last block
    (32, 1024, 32, 64, 8, 8, 3.0),     # the largest E and K
    (8, 8, 2, 50, 2, 16, 2.0),         # one expert per rank
    (4, 16, 3, 1, 4, 8, 1.0),          # one token per rank
    (4, 8, 2, 300, 256, 8, 3.0),       # the largest slot budget
    (64, 64, 4, 16, 1, 8, 5.0),        # 64 ranks, one expert and one slot each
    (4, 16, 2, 64, 4, 16384, 2.0),     # 32 KB rows
    (16, 64, 4, 100, 128, 8, 3.0),     # R*slots = 2048 slot entries
    (4, 16, 3, 40, 4, 8200, 3.0),      # 1025 vectors per row: no thread shape fits exactly
]


@pytest.mark.parametrize("R,E,K,S,slots,H,mv", CASES)
def test_random_cases(R, E, K, S, slots, H, mv):
    seed = 777 + R * 1000 + E + K + S
    ids, wt, _, _ = make_routing(R, E, K, S, mv, seed)
    full_case(R, E, K, S, slots, H, ids.numpy(), wt.numpy(), seed, G_el=8 if slots else 0)


@pytest.mark.parametrize("R,E,K,S,slots,H,mv", [
    (4, 1024, 8, 8192, 4, 16, 1.0),    # 16 chunks per histogram wave: map parts of 8
    (8, 1024, 8, 8100, 8, 8, 3.0),     # 32 chunks per wave, 4 parts, ragged last block
])
def test_split_map_waves(R, E, K, S, slots, H, mv):
    """Large assignment counts with many experts: each histogram wave's range is mapped by
    several waves, each starting from the counts the histogram recorded for it."""
    sz = M.moonep_query(R, E, K, S, slots)
    assert sz.blk // 512 > 8, "case must split histogram waves"
    seed = 5150 + S
    ids, wt, _, _ = make_routing(R, E, K, S, mv, seed, device="cuda")
    full_case(R, E, K, S, slots, H, ids.cpu().numpy(), wt.cpu().numpy(), seed)


@pytest.mark.parametrize("case", adversarial.routings(), ids=lambda c: c[0])
def test_adversarial_routings_on_gpu(case):
    name, R, E, K, S, slots, ids = case
    T = R * S
    w = np.full((T, K), 1.0 / K, dtype=np.float32)
    full_case(R, E, K, S, slots, 64, ids, w, 4100 + R + E + K, G_el=8 if slots else 0)


@pytest.mark.parametrize("R,E,K,S,slots,mv", [
    (64, 1024, 16, 1024, 8, 3.0),     # 64 blocks per column thread: two register rounds
    (50, 1000, 16, 1010, 4, 8.0),     # 50 blocks: a ragged second round and last block
])
def test_long_block_columns(R, E, K, S, slots, mv):
    """Many assignments with many experts: each planner thread scans more block counts than
    it holds in registers, so the column scan and the bases it writes (wave 0's by wave 1)
    take the multi-round path."""
    sz = M.moonep_query(R, E, K, S, slots)
    tpc = 1
    while tpc * 2 * E <= 1024 and tpc * 2 <= sz.nblk:
        tpc *= 2
    assert (sz.nblk + tpc - 1) // tpc > 32, "case must exceed one register round"
    seed = 6100 + R
    ids, wt, _, _ = make_routing(R, E, K, S, mv, seed, device="cuda")
    full_case(R, E, K, S, slots, 8, ids.cpu().numpy(), wt.cpu().numpy(), seed)


def _cut_prefix(p):
    """For coverage only: how many shedding experts (in plan order) come before the first
    one that, were there no slot budget, would give some rank more than `slots` pieces.
    The planner places that prefix in parallel and the rest one expert at a time."""
    sz = p.sz
    order = [int(e) for e in p.order if p.shed[e] > 0]
    ends = np.cumsum([int(p.shed[e]) for e in order])
    starts = ends - np.array([int(p.shed[e]) for e in order])
    dend = np.cumsum(p.deficit)
    dbeg = dend - p.deficit
    first_bad = len(order)
    for r in range(sz.R):
        if p.deficit[r] == 0:
            continue
        hit = [q for q in range(len(order)) if starts[q] < dend[r] and ends[q] > dbeg[r]]
        if len(hit) > sz.slots:
            first_bad = min(first_bad, hit[sz.slots])
    return first_bad, len(order)


def test_tight_slot_budgets():
    """Plans under small slot budgets and strong skew, where placement switches from the
    parallel cut to one expert at a time part way through the shedding experts."""
    rng = np.random.default_rng(4321)
    kinds = set()
    for i in range(32):
        R = int(rng.choice([2, 3, 4, 7, 8, 16, 32, 64]))
        E = R * int(rng.choice([1, 2, 3, 4, 6]))
        K = int(rng.integers(1, min(E, 8) + 1))
        S = int(rng.integers(4, 200))
        slots = int(rng.choice([1, 2, 3, 4]))
        mv = float(rng.choice([0.5, 1.0, 3.0, 8.0, 20.0]))
        seed = 9000 + i
        say(f"tight slots case {i}: R={R} E={E} K={K} S={S} slots={slots} maxvio={mv}")
        ids, wt, _, _ = make_routing(R, E, K, S, mv, seed)
        ids_np = ids.numpy()
        plan = M.moonep_plan(*to_dev_ids(ids_np, wt.numpy()), R, E, K, S, slots)
        p = O.plan(ids_np, R, E, K, S, slots)
        assert_plan_matches(read_plan(plan), p, O.slot_map(p, ids_np))
        q, n = _cut_prefix(p)
        kinds.add("none" if n == 0 else ("all" if q == n else ("part" if q > 0 else "zero")))
    torch.cuda.synchronize()
    assert "part" in kinds and "all" in kinds, kinds


def test_balanced_routing_has_no_pieces():
    R, E, K, S = 8, 64, 8, 128
    ids, wt = make_balanced_routing(R, E, K, S)
    p = full_case(R, E, K, S, 8, 64, ids.numpy(), wt.numpy(), 5)
    assert p.n_pieces == 0


@pytest.mark.parametrize("name", ["plan_r2_e4_k2_s4.json", "plan_r3_e6_fallback.json"])
def test_golden_plans_on_gpu(name):
    g = json.load(open(os.path.join(GOLDEN, name)))
    ids = np.array(g["ids"], dtype=np.int32)
    T, K = ids.shape
    w = np.full((T, K), 1.0 / K, dtype=np.float32)
    say(f"golden {name}")
    plan = M.moonep_plan(*to_dev_ids(ids, w), g["R"], g["E"], g["K"], g["S"], g["slots"])
    got = read_plan(plan)
    assert got["dst_row"].tolist() == g["dst_row"]
    assert got["pieces"][:, :6].tolist() == g["pieces"]
    assert got["off"].tolist() == g["off"]


def test_slot_exhaustion_on_gpu():
    g = json.load(open(os.path.join(GOLDEN, "plan_r7_e56_slot_exhaustion.json")))
    R, E, K, S, slots = g["R"], g["E"], g["K"], g["S"], g["slots"]
    flat = np.repeat(np.arange(E), g["load"]).astype(np.int32)
    ids = flat.reshape(R * S, K)
    w = np.full((R * S, K), 0.5, dtype=np.float32)
    p = full_case(R, E, K, S, slots, 64, ids, w, 11, G_el=16)
    assert p.n_fallback == 4


# ----------------------------------------------------------------------------------------
# edge cases and the error paths
# ----------------------------------------------------------------------------------------

def test_bad_ids_give_empty_plan():
    R, E, K, S, slots, H = 4, 16, 2, 64, 4, 64
    ids, wt, _, _ = make_routing(R, E, K, S, 1.0, 3)
    ids = ids.clone()
    ids[10, 1] = E          # out of range
    ids[50, 0] = -3
    say("bad ids")
    plan = M.moonep_plan(*to_dev_ids(ids.numpy(), wt.numpy()), R, E, K, S, slots)
    st = M.moonep_plan_status(plan)
    assert st["status"] == 1 and st["bad_index"] == 10 * K + 1
    got = read_plan(plan)
    assert (got["dst_row"] == -1).all()
    x = make_hidden(R * S, H, 1, device="cuda")
    recv = torch.zeros(plan.sz.recv_rows, H, dtype=torch.bfloat16, device="cuda")
    M.moonep_dispatch(plan, x, recv)
    assert (recv == 0).all()
    out = M.moonep_combine(plan, recv)
    assert (out == 0).all()
    # the staged A/B path keeps the same contract: nothing mapped, zero output rows, even
    # when the staging buffer holds NaN from earlier use
    stage = torch.full((R * S * K, H), float("nan"), dtype=torch.bfloat16, device="cuda")
    recv_s = torch.zeros_like(recv)
    M.moonep_dispatch_staged(plan, x, recv_s, stage)
    assert (recv_s == 0).all()
    stage.fill_(float("nan"))
    out_s = M.moonep_combine_staged(plan, recv, stage=stage)
    assert (bf16_bits(out_s) == 0).all(), "staged combine of an invalid plan must write zero rows"
    home, rep = make_grads(E, R, slots, 16, 2, device="cuda")
    h0 = home.clone()
    M.moonep_reduce_grad(plan, home, rep)
    assert torch.equal(home, h0)


def test_argument_errors():
    dev = "cuda"
    ids = torch.zeros(8, 2, dtype=torch.int32, device=dev)
    w = torch.zeros(8, 2, dtype=torch.float32, device=dev)
    with pytest.raises(M.MoonepError):
        M.moonep_query(3, 16, 2, 4, 4)          # E % R != 0
    with pytest.raises(M.MoonepError):
        M.moonep_query(65, 65, 2, 4, 4)         # R beyond one wave
    with pytest.raises(M.MoonepError):
        M.moonep_query(4, 16, 17, 4, 4)         # K > E
    plan = M.moonep_plan(ids, w, 4, 16, 2, 2, 4)
    x = torch.zeros(8, 12, dtype=torch.bfloat16, device=dev)
    with pytest.raises(M.MoonepError):
        M.moonep_dispatch(plan, x)              # H % 8 != 0
    big = torch.zeros(8 * 16 + 8, dtype=torch.bfloat16, device=dev)
    M.moonep_dispatch(plan, big[8:136].view(8, 16))       # 16-byte aligned: fine
    with pytest.raises(M.MoonepError):
        M.moonep_dispatch(plan, big[1:129].view(8, 16))   # 2-byte offset: EALIGN
    # the staged wrappers check every tensor's size on the host: nothing is launched
    H = 16
    ok_x = torch.zeros(8, H, dtype=torch.bfloat16, device=dev)
    ok_recv = torch.zeros(plan.sz.recv_rows, H, dtype=torch.bfloat16, device=dev)
    with pytest.raises(M.MoonepError):
        M.moonep_dispatch_staged(plan, ok_x[:7], ok_recv)                 # x too small
    with pytest.raises(M.MoonepError):
        M.moonep_dispatch_staged(plan, ok_x, ok_recv[:-1])                # recv too small
    with pytest.raises(M.MoonepError):
        M.moonep_combine_staged(plan, ok_recv[:-1])                       # y too small
    with pytest.raises(M.MoonepError):
        M.moonep_combine_staged(plan, ok_recv, ok_x[:7])                  # out too small
    with pytest.raises(M.MoonepError):
        M.moonep_dispatch_staged(plan, ok_x, ok_recv, torch.zeros(1, H, dtype=torch.bfloat16,
                                                                   device=dev))   # stage
    # weights on another device than the ids: refused before any launch
    with pytest.raises(M.MoonepError):
        M.moonep_plan(ids, w.cpu(), 4, 16, 2, 2, 4)
    torch.cuda.synchronize()


def test_plan_is_deterministic_and_reusable():
    w = DSV3
    ids, wt, _, _ = make_routing(w.R, w.E, w.K, w.S, 20.0, w.seed(3), device="cuda")
    say("determinism dsv3 maxvio 20")
    p1 = M.moonep_plan(ids, wt, w.R, w.E, w.K, w.S, w.slots)
    b1 = p1.blob.clone()
    p2 = M.moonep_plan(ids, wt, w.R, w.E, w.K, w.S, w.slots, plan=p1)
    assert torch.equal(b1, p2.blob)
    x = make_hidden(w.T, w.H, 9, device="cuda")
    recv = M.moonep_dispatch(p2, x)
    o1 = M.moonep_combine(p2, recv)
    o2 = M.moonep_combine(p2, recv)
    assert torch.equal(o1, o2)
    # dispatch -> no-op expert -> combine returns x (weights sum to 1)
    assert torch.equal(o1.float(), x.float())


def test_one_workspace_serves_every_size():
    """One zero-filled workspace, reused call after call for problems of different sizes
    (the workgroup counts of the planning launch differ): every plan equals the oracle's,
    and the arrival word at the workspace's head is zero again after each call."""
    cases = [(DSV3, 0), (TINY, 0), (SMALL, 0), (DECODE, 1), (TINY, 0), (DSV3, 3)]
    sizes = [M.moonep_query(wl.R, wl.E, wl.K, wl.S, wl.slots) for wl, _ in cases]
    ws = torch.zeros(max(sz.workspace_bytes for sz in sizes) // 4 + 64, dtype=torch.int32,
                     device="cuda")
    for (wl, mi), sz in zip(cases, sizes):
        say(f"shared workspace: {wl.name} maxvio {wl.maxvio[mi]}")
        ids, w, _, _ = make_routing(wl.R, wl.E, wl.K, wl.S, wl.maxvio[mi], wl.seed(mi),
                                    device="cuda")
        blob = torch.empty(sz.plan_bytes // 4, dtype=torch.int32, device="cuda")
        plan = M.moonep_plan(ids, w, wl.R, wl.E, wl.K, wl.S, wl.slots,
                             plan=M.Plan(sz, blob, ws[: sz.workspace_bytes // 4]))
        assert plan.workspace.data_ptr() == ws.data_ptr()
        ids_np = ids.cpu().numpy()
        p = O.plan(ids_np, wl.R, wl.E, wl.K, wl.S, wl.slots)
        assert_plan_matches(read_plan(plan), p, O.slot_map(p, ids_np))
        assert int(ws[0].item()) == 0


def test_plan_repeats_identically_over_random_sizes():
    """Many problem sizes, so the planning launch runs with anything from one to a few
    hundred workgroups: planning four times into the same blob and workspace gives the same
    blob each time, the arrival word is zero after each call, and the small problems match
    the oracle."""
    import random
    rng = random.Random(20260001)
    done = 0
    while done < 150:
        R = rng.choice([1, 2, 4, 8, 16, 32, 64])
        E = R * rng.choice([1, 2, 4, 6, 8, 16, 24, 32])
        if E > 1024:
            continue
        K = rng.randint(1, min(E, 10))
        S = rng.choice([1, 7, 64, 300, 1024, 4096])
        if R * S * K > 2_000_000:
            continue
        slots = rng.choice([0, 1, 2, 4, 8, E // R])
        mv = rng.choice([0.2, 1.0, 5.0, 20.0])
        ids, w, _, _ = make_routing(R, E, K, S, mv, rng.randint(0, 10 ** 6), device="cuda")
        plan, first = None, None
        for rep in range(4):
            plan = M.moonep_plan(ids, w, R, E, K, S, slots, plan=plan)
            torch.cuda.synchronize()
            assert int(plan.workspace[0].item()) == 0
            if first is None:
                first = plan.blob.clone()
                if R * S * K <= 20000:
                    ids_np = ids.cpu().numpy()
                    p = O.plan(ids_np, R, E, K, S, slots)
                    assert_plan_matches(read_plan(plan), p, O.slot_map(p, ids_np))
            else:
                assert torch.equal(plan.blob, first), (R, E, K, S, slots, mv, rep)
        done += 1


# ----------------------------------------------------------------------------------------
# full-size workloads: whole plan, dst_row, every dispatched row, padding, every combined
# token and every reduced expert
# ----------------------------------------------------------------------------------------

BIG = [(DSV3, i) for i in range(4)] + [(KIMI, 0)] + [(DECODE, i) for i in range(2)]


@pytest.mark.parametrize("wl,mi", BIG, ids=lambda v: getattr(v, "name", str(v)))
def test_full_size(wl, mi):
    mv = wl.maxvio[mi]
    seed = wl.seed(mi)
    say(f"full size {wl.name} maxvio={mv}")
    ids, wt, _, got_mv = make_routing(wl.R, wl.E, wl.K, wl.S, mv, seed, device="cuda")
    ids_np, w_np = ids.cpu().numpy(), wt.cpu().numpy()
    plan = M.moonep_plan(ids, wt, wl.R, wl.E, wl.K, wl.S, wl.slots)
    p = O.plan(ids_np, wl.R, wl.E, wl.K, wl.S, wl.slots)
    dst = O.slot_map(p, ids_np)
    got = read_plan(plan)
    assert_plan_matches(got, p, dst)

    x = make_hidden(wl.T, wl.H, seed + 1, device="cuda")
    nan_bits = int(bf16_bits(torch.tensor([float("nan")], dtype=torch.bfloat16))[0])
    recv = torch.full((plan.sz.recv_rows, wl.H), float("nan"), dtype=torch.bfloat16, device="cuda")
    M.moonep_dispatch(plan, x, recv)
    rng = np.random.default_rng(seed)
    tok = np.unique(np.concatenate([rng.choice(wl.T, 384, replace=False), [0, wl.T - 1]]))
    x_s = bf16_bits(x[torch.from_numpy(tok).cuda()])
    rows = dst[tok]                                        # [n, K] oracle rows
    r_t = torch.from_numpy(rows.reshape(-1).astype(np.int64)).cuda()
    got_rows = bf16_bits(recv[r_t]).reshape(len(tok), wl.K, wl.H)
    assert (got_rows == x_s[:, None, :]).all(), "dispatched rows"
    # every assignment's row (whole dst_row is already bit-exact): property on the GPU
    all_rows = torch.from_numpy(dst.reshape(-1).astype(np.int64)).cuda()
    for c0 in range(0, wl.T, 4096):
        c1 = min(c0 + 4096, wl.T)
        g = recv[all_rows[c0 * wl.K:c1 * wl.K]].view(c1 - c0, wl.K, wl.H)
        assert torch.equal(g, x[c0:c1, None, :].expand(-1, wl.K, -1))
    # padding rows (no assignment maps there) are never written
    pad = torch.ones(plan.sz.recv_rows, dtype=torch.bool, device="cuda")
    pad[all_rows] = False
    pad_rows = recv[pad].view(torch.int16)
    assert pad_rows.shape[0] == plan.sz.recv_rows - wl.A
    assert bool((pad_rows == np.int16(np.uint16(nan_bits).view(np.int16))).all()), \
        "padding rows must not be written"
    del recv, pad, pad_rows

    # combine on an independent expert output y (seeded): every token against the oracle,
    # in chunks of tokens (rows gathered on the GPU, the oracle run on the host)
    y = make_hidden(plan.sz.recv_rows, wl.H, seed + 2, device="cuda")
    out = M.moonep_combine(plan, y)
    ch = 2048
    local_dst = np.arange(ch * wl.K).reshape(ch, wl.K)
    for c0 in range(0, wl.T, ch):
        c1 = min(c0 + ch, wl.T)
        y_rows = bf16_bits(y[all_rows[c0 * wl.K:c1 * wl.K]])
        ref = O.combine(local_dst[:c1 - c0], w_np[c0:c1], y_rows)
        got_out = bf16_bits(out[c0:c1])
        assert_close(O.bf16_to_f32(got_out), O.bf16_to_f32(ref), RTOL_BF16)
        assert (got_out == ref).all(), f"combine tokens {c0}..{c1}"
    del y, out

    if wl.G_el:
        # every expert of the reduce list against home + its slot replicas in piece order;
        # every other expert untouched
        home, rep = make_grads(wl.E, wl.R, wl.slots, wl.G_el, seed + 3, device="cuda")
        red = got["red"]
        assert len(red) == len({int(q[0]) for q in p.pieces if q[2] >= 0})
        is_red = torch.zeros(wl.E, dtype=torch.bool, device="cuda")
        is_red[torch.from_numpy(red.astype(np.int64)).cuda()] = True
        o_before = home[~is_red].clone()
        h_before = home[is_red].cpu().numpy()           # experts in id order
        red_ids = np.flatnonzero(is_red.cpu().numpy())
        need = sorted({(int(q[1]), int(q[2])) for q in p.pieces if q[2] >= 0})
        rep_s = {k: rep[k[0], k[1]].cpu().numpy() for k in need}
        M.moonep_reduce_grad(plan, home, rep)
        h_after = home[is_red].cpu().numpy()
        for n, e in enumerate(red_ids):
            ref_e = h_before[n].copy()
            for (pe, r, slot, cnt, start, fb) in p.pieces:
                if pe == e and slot >= 0:
                    ref_e = (ref_e + rep_s[(int(r), int(slot))]).astype(np.float32)
            assert_close(h_after[n], ref_e, RTOL_FP32)
            assert (h_after[n].view(np.uint32) == ref_e.view(np.uint32)).all(), f"reduce expert {e}"
        assert torch.equal(home[~is_red], o_before)     # experts without replicas untouched
        del home, rep, o_before
    torch.cuda.synchronize()
