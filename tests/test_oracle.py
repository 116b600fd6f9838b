"""Pins for the CPU oracle: each check ties it to something other than itself.

* hand-derived worked examples of the plan rule (tests/golden/*.json, each citing the
  passages it follows);
* an independent one-assignment-at-a-time derivation of the greedy plan;
* when no slot budget binds, the plan equals a merge (interval intersection) of the
  shed stream and the deficit stream, a different formulation of the same rule;
* exhaustive enumeration of every routing at R=2, E=4, K=1, S=3;
* invariants the pages fix: exactly S*K per rank ('Moonshot AI Open-Sources MoonEP',
  paragraph 3), static S*K+padding buffers and a bijective slot map
  ('MoonshotAI/MoonEP 딥다이브', section 4, pattern 2), slot budget (paragraph 5 of the
  first page);
* closed forms that need no plan at all: dispatch -> no-op -> combine returns x (the deep
  dive's section 8, exercise C); combine through the plan equals the no-replication
  combine; reduce through the plan equals the no-replication gradient sum (section 4,
  pattern 3);
* a brute-force streaming slot map on tiny inputs;
* the bf16 rounding helper against torch's own conversion.
"""

import collections
import itertools
import json
import os

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

from gen import TINY, SMALL, make_routing, make_balanced_routing, make_hidden, make_scales, bf16_bits
from oracle import moonep_oracle as O
from tests.tol import assert_close, RTOL_FP32
from tests import adversarial

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------------------
# independent re-derivations used as pins
# ----------------------------------------------------------------------------------------

def unit_step_plan(load, R, E, K, S, slots):
    """The greedy rule moved one assignment at a time, with no piece arithmetic."""
    E_loc, C = E // R, S * K
    home = [e // E_loc for e in range(E)]
    hl = [sum(load[e] for e in range(E) if home[e] == r) for r in range(R)]
    X = [max(0, h - C) for h in hl]
    D = [max(0, C - h) for h in hl]
    order = sorted(range(E), key=lambda e: (-load[e], e))
    shed = [0] * E
    for e in order:
        while X[home[e]] > 0 and shed[e] < load[e]:
            shed[e] += 1
            X[home[e]] -= 1
    used = [0] * R
    units = []
    for e in order:
        cur = None
        for _ in range(shed[e]):
            if cur is None or D[cur[0]] == 0:
                free = [r for r in range(R) if D[r] > 0 and used[r] < slots]
                if free:
                    cur = (free[0], used[free[0]])
                    used[free[0]] += 1
                else:
                    cur = (min(r for r in range(R) if D[r] > 0), -1)
            D[cur[0]] -= 1
            units.append((e, cur[0], cur[1]))
    pieces, fb = [], [0] * R
    given = collections.Counter()
    for key, grp in itertools.groupby(units):
        e, r, slot = key
        cnt = len(list(grp))
        start = (load[e] - shed[e]) + given[e]
        fbpos = fb[r] if slot < 0 else 0
        if slot < 0:
            fb[r] += cnt
        given[e] += cnt
        pieces.append((e, r, slot, cnt, start, fbpos))
    return shed, pieces


def merge_plan_pieces(load, R, E, K, S):
    """Pieces as intersections of two partitions of one line: experts' shed amounts laid
    end to end in (load desc, id asc) order, and receivers' deficits laid end to end in id
    order.  Valid only when no receiver needs more slots than it has."""
    E_loc, C = E // R, S * K
    hl = [sum(load[r * E_loc:(r + 1) * E_loc]) for r in range(R)]
    order = sorted(range(E), key=lambda e: (-load[e], e))
    # shed per rank: heaviest first (ties by id), within that rank only
    shed = [0] * E
    for r in range(R):
        x = max(0, hl[r] - C)
        for e in sorted(range(r * E_loc, (r + 1) * E_loc), key=lambda e: (-load[e], e)):
            take = min(load[e], x)
            shed[e] = take
            x -= take
    segs_e, pos = [], 0
    for e in order:
        if shed[e] > 0:
            segs_e.append((e, pos, pos + shed[e]))
            pos += shed[e]
    segs_r, pos = [], 0
    for r in range(R):
        d = max(0, C - hl[r])
        if d > 0:
            segs_r.append((r, pos, pos + d))
            pos += d
    pieces, per_rank = [], collections.Counter()
    for e, a0, a1 in segs_e:
        for r, b0, b1 in segs_r:
            lo, hi = max(a0, b0), min(a1, b1)
            if hi > lo:
                pieces.append((e, r, per_rank[r], hi - lo, load[e] - shed[e] + (lo - a0), 0))
                per_rank[r] += 1
    return shed, pieces, max(per_rank.values(), default=0)


def streaming_slot_map(p, ids):
    """Slot map by walking assignments in increasing i with one counter per expert."""
    sz = p.sz
    flat = np.asarray(ids).reshape(-1)
    seen = collections.Counter()
    out = []
    for i, e in enumerate(flat):
        e = int(e)
        j = seen[e]
        seen[e] += 1
        if j < p.keep[e]:
            h = e // sz.E_loc
            out.append(h * sz.NvS + int(p.off[h, e - h * sz.E_loc]) + j)
            continue
        for q in range(p.n_pieces):
            pe, r, slot, cnt, start, fbpos = (int(v) for v in p.pieces[q])
            if pe == e and start <= j < start + cnt:
                base = p.off[r, sz.E_loc + slot] if slot >= 0 else p.off[r, sz.G] + fbpos
                out.append(r * sz.NvS + int(base) + (j - start))
                break
        else:
            raise AssertionError("assignment not covered by any piece")
    return np.array(out).reshape(sz.T, sz.K)


def check_invariants(p, ids=None):
    sz = p.sz
    assert p.load.sum() == sz.A
    # every rank serves exactly S*K assignments
    for r in range(sz.R):
        assert p.group_size[r].sum() == sz.C, (r, p.group_size[r])
        assert p.off[r, sz.G] + p.group_size[r, sz.G] <= sz.NvS
    # keep + pieces of e == load of e
    got = p.keep.copy()
    for (e, r, slot, cnt, start, fbpos) in p.pieces:
        got[e] += cnt
        assert cnt > 0
        assert p.deficit[r] > 0            # only ranks that started short receive
        assert p.excess[e // sz.E_loc] > 0  # only overloaded homes shed
    assert (got == p.load).all()
    # slot budget
    for r in range(sz.R):
        assert ((p.pieces[:, 1] == r) & (p.pieces[:, 2] >= 0)).sum() <= sz.slots if p.n_pieces else True
    assert p.n_pieces <= sz.E + sz.R
    # per overloaded rank: a shed prefix in (load desc, id) order with one partial at most
    for r in range(sz.R):
        es = sorted(range(r * sz.E_loc, (r + 1) * sz.E_loc), key=lambda e: (-p.load[e], e))
        sh = [int(p.shed[e]) for e in es]
        assert sum(sh) == p.excess[r]
        partial_seen = False
        for e, s in zip(es, sh):
            if partial_seen:
                assert s == 0
            elif s < p.load[e]:
                partial_seen = True
    if ids is not None:
        dst = O.slot_map(p, ids).reshape(-1)
        assert len(np.unique(dst)) == sz.A          # every assignment has its own row
        # every row lies inside a group of its rank, never in padding
        for row in dst:
            r, loc = divmod(int(row), sz.NvS)
            inside = False
            for g in range(sz.G + 1):
                if p.off[r, g] <= loc < p.off[r, g] + p.group_size[r, g]:
                    inside = True
            assert inside


# ----------------------------------------------------------------------------------------
# golden worked examples
# ----------------------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["plan_r2_e4_k2_s4.json", "plan_r3_e6_fallback.json"])
def test_golden_full_examples(name):
    g = json.load(open(os.path.join(GOLDEN, name)))
    ids = np.array(g["ids"], dtype=np.int32)
    p = O.plan(ids, g["R"], g["E"], g["K"], g["S"], g["slots"])
    assert p.sz.NvS == g["NvS"]
    assert p.load.tolist() == g["load"]
    assert p.shed.tolist() == g["shed"]
    assert p.keep.tolist() == g["keep"]
    assert p.pieces.tolist() == g["pieces"]
    assert p.slot_expert.tolist() == g["slot_expert"]
    assert p.off.tolist() == g["off"]
    assert p.n_replicas == g["n_replicas"] and p.n_fallback == g["n_fallback"]
    assert O.slot_map(p, ids).tolist() == g["dst_row"]
    check_invariants(p, ids)


def test_golden_slot_exhaustion():
    g = json.load(open(os.path.join(GOLDEN, "plan_r7_e56_slot_exhaustion.json")))
    sz = O.sizes(g["R"], g["E"], g["K"], g["S"], g["slots"])
    p = O.plan_from_loads(np.array(g["load"]), sz)
    assert sz.NvS == g["NvS"]
    assert p.pieces.tolist() == g["pieces"]
    assert p.slot_expert[0].tolist() == g["slot_expert_rank0"]
    assert p.off[0].tolist() == g["off_rank0"]
    for r in range(1, 7):
        assert p.off[r].tolist() == g["off_rank1"]
    assert p.n_replicas == g["n_replicas"] and p.n_fallback == g["n_fallback"]
    check_invariants(p)


# ----------------------------------------------------------------------------------------
# independent derivations
# ----------------------------------------------------------------------------------------

def _random_loads(rng, R, E, K, S, skew):
    T = R * S
    p = rng.dirichlet(np.full(E, skew))
    ids = np.stack([rng.choice(E, size=K, replace=False, p=p) for _ in range(T)])
    return ids.astype(np.int32)


@pytest.mark.parametrize("seed", range(40))
def test_unit_step_and_merge_agree(seed):
    rng = np.random.default_rng(1000 + seed)
    R = int(rng.choice([1, 2, 3, 4, 8]))
    E = R * int(rng.integers(1, 7))
    K = int(rng.integers(1, min(E, 4) + 1))
    S = int(rng.integers(1, 12))
    slots = int(rng.integers(0, 5))
    ids = _random_loads(rng, R, E, K, S, skew=float(rng.choice([0.1, 0.5, 3.0])))
    p = O.plan(ids, R, E, K, S, slots)
    check_invariants(p, ids)
    load = p.load.tolist()
    shed_u, pieces_u = unit_step_plan(load, R, E, K, S, slots)
    assert p.shed.tolist() == shed_u
    assert [tuple(x) for x in p.pieces.tolist()] == pieces_u
    shed_m, pieces_m, max_per_rank = merge_plan_pieces(load, R, E, K, S)
    assert p.shed.tolist() == shed_m
    if max_per_rank <= slots:
        assert p.n_fallback == 0
        assert [tuple(x) for x in p.pieces.tolist()] == pieces_m
    assert (O.slot_map(p, ids) == streaming_slot_map(p, ids)).all()


@pytest.mark.parametrize("case", adversarial.routings(), ids=lambda c: c[0])
def test_adversarial_routings(case):
    """Extreme routings (one expert takes every token, a rank with no load, everything on
    one rank, identical routing, no slots): invariants hold and the one-assignment-at-a-
    time derivation agrees."""
    name, R, E, K, S, slots, ids = case
    p = O.plan(ids, R, E, K, S, slots)
    check_invariants(p, ids)
    shed_u, pieces_u = unit_step_plan(p.load.tolist(), R, E, K, S, slots)
    assert p.shed.tolist() == shed_u
    assert [tuple(x) for x in p.pieces.tolist()] == pieces_u
    assert (O.slot_map(p, ids) == streaming_slot_map(p, ids)).all()
    assert p.n_pieces > 0


def test_exhaustive_r2_e4_k1_s3():
    R, E, K, S = 2, 4, 1, 3
    for slots in (0, 1, 2):
        for combo in itertools.product(range(E), repeat=R * S * K):
            ids = np.array(combo, dtype=np.int32).reshape(R * S, K)
            p = O.plan(ids, R, E, K, S, slots)
            check_invariants(p, ids)
            shed_u, pieces_u = unit_step_plan(p.load.tolist(), R, E, K, S, slots)
            assert [tuple(x) for x in p.pieces.tolist()] == pieces_u
            assert (O.slot_map(p, ids) == streaming_slot_map(p, ids)).all()


def test_balanced_and_single_rank_have_no_pieces():
    for (R, E, K, S) in [(4, 16, 2, 64), (8, 64, 8, 16), (1, 8, 2, 5)]:
        ids, _ = make_balanced_routing(R, E, K, S)
        p = O.plan(ids.numpy(), R, E, K, S, 2)
        assert p.n_pieces == 0
        check_invariants(p, ids.numpy())
        # with no pieces, each rank's slot map lists its experts' assignments in order
        dst = O.slot_map(p, ids.numpy()).reshape(-1)
        flat = ids.numpy().reshape(-1)
        for r in range(R):
            mine = np.nonzero(flat // (E // R) == r)[0]
            by_row = mine[np.argsort(dst[mine])]
            # rows grouped by expert, increasing i inside each expert
            assert (np.diff(flat[by_row]) >= 0).all()
    rng = np.random.default_rng(5)
    ids = _random_loads(rng, 1, 8, 3, 40, 0.2)
    assert O.plan(ids, 1, 8, 3, 40, 4).n_pieces == 0


def test_plan_depends_only_on_loads():
    rng = np.random.default_rng(7)
    ids = _random_loads(rng, 4, 16, 2, 32, 0.3)
    p1 = O.plan(ids, 4, 16, 2, 32, 4)
    perm = rng.permutation(ids.reshape(-1)).reshape(ids.shape)
    p2 = O.plan(perm, 4, 16, 2, 32, 4)
    assert (p1.pieces == p2.pieces).all() and (p1.off == p2.off).all()


@st.composite
def _load_problems(draw):
    R = draw(st.integers(1, 6))
    E = R * draw(st.integers(1, 4))
    K = draw(st.integers(1, min(3, E)))
    S = draw(st.integers(1, 6))
    slots = draw(st.integers(0, 4))
    A = R * S * K
    cuts = sorted(draw(st.lists(st.integers(0, A), min_size=E - 1, max_size=E - 1)))
    load = np.diff(np.array([0] + cuts + [A], dtype=np.int64))
    return R, E, K, S, slots, load


@settings(max_examples=400, deadline=None)
@given(_load_problems())
def test_plan_properties_on_searched_loads(prob):
    """Property search over load vectors (any split of R*S*K assignments over E experts):
    the plan keeps every invariant and equals the one-assignment-at-a-time derivation."""
    R, E, K, S, slots, load = prob
    p = O.plan_from_loads(load, O.sizes(R, E, K, S, slots))
    check_invariants(p)
    shed_u, pieces_u = unit_step_plan(load.tolist(), R, E, K, S, slots)
    assert p.shed.tolist() == shed_u
    assert [tuple(x) for x in p.pieces.tolist()] == pieces_u


def test_loads_brute_force_and_bad_ids():
    rng = np.random.default_rng(3)
    ids = rng.integers(0, 16, size=(64, 2)).astype(np.int32)
    c = collections.Counter(ids.reshape(-1).tolist())
    assert O.expert_loads(ids, 16).tolist() == [c[e] for e in range(16)]
    with pytest.raises(ValueError):
        O.expert_loads(np.array([[0, 16]]), 16)
    with pytest.raises(ValueError):
        O.expert_loads(np.array([[-1, 0]]), 16)
    with pytest.raises(ValueError):
        O.sizes(3, 16, 2, 4, 4)   # E % R != 0


# ----------------------------------------------------------------------------------------
# closed forms for dispatch, combine and reduce
# ----------------------------------------------------------------------------------------

def _tiny_inputs(maxvio=2.0, seed=20260100):
    w = TINY
    ids, wt, _, mv = make_routing(w.R, w.E, w.K, w.S, maxvio, seed)
    x = make_hidden(w.T, w.H, seed + 1)
    return w, ids.numpy(), wt.numpy(), bf16_bits(x)


def test_generator_hits_maxvio_and_is_deterministic():
    w = TINY
    ids1, w1, a1, mv1 = make_routing(w.R, w.E, w.K, w.S, 2.0, 11)
    ids2, w2, a2, mv2 = make_routing(w.R, w.E, w.K, w.S, 2.0, 11)
    assert torch.equal(ids1, ids2) and torch.equal(w1, w2)
    assert abs(mv1 - 2.0) <= 0.05 * 2.0
    assert torch.allclose(w1.sum(1), torch.ones(w.T), atol=1e-6)
    # each token's K experts are distinct
    assert all(len(set(r)) == w.K for r in ids1.tolist())
    s = SMALL
    ids3, _, _, mv3 = make_routing(s.R, s.E, s.K, s.S, 0.2, 12)
    assert abs(mv3 - 0.2) <= 0.02


def test_dispatch_noop_combine_is_identity():
    w, ids, wt, x = _tiny_inputs()
    p = O.plan(ids, w.R, w.E, w.K, w.S, w.slots)
    assert p.n_pieces > 0                     # the example does exercise replicas
    dst = O.slot_map(p, ids)
    recv = O.dispatch(dst, x, w.R * p.sz.NvS)
    for i, row in enumerate(dst.reshape(-1)):
        assert (recv[row] == x[i // w.K]).all()
    out = O.combine(dst, wt, recv)
    assert (O.bf16_to_f32(out) == O.bf16_to_f32(x)).all()


def test_combine_equals_no_replication_closed_form():
    w, ids, wt, x = _tiny_inputs(seed=20260101)
    s = make_scales(w.E, 99).numpy()
    p = O.plan(ids, w.R, w.E, w.K, w.S, w.slots)
    assert p.n_pieces > 0
    dst = O.slot_map(p, ids)
    recv = O.dispatch(dst, x, w.R * p.sz.NvS)
    # the toy expert: a per-expert fp32 scale; a replica applies its home expert's scale
    expert_of_row = np.full(recv.shape[0], -1)
    expert_of_row[dst.reshape(-1)] = ids.reshape(-1)
    y = recv.copy()
    used = expert_of_row >= 0
    y[used] = O.f32_to_bf16_rne(s[expert_of_row[used]][:, None] * O.bf16_to_f32(recv[used]))
    out = O.combine(dst, wt, y)
    # no plan: each token applies its K experts directly
    xf = O.bf16_to_f32(x)
    ref = np.zeros_like(xf)
    for t in range(w.T):
        acc = np.zeros(w.H, dtype=np.float32)
        for k in range(w.K):
            yk = O.bf16_to_f32(O.f32_to_bf16_rne(np.float32(s[ids[t, k]]) * xf[t]))
            acc = (acc + (np.float32(wt[t, k]) * yk).astype(np.float32)).astype(np.float32)
        ref[t] = acc
    assert (out == O.f32_to_bf16_rne(ref)).all()


@pytest.mark.parametrize("R,E,K,S,slots,skew,seed", [
    (4, 16, 2, 48, 4, 0.15, 17),
    (4, 32, 2, 40, 8, 0.08, 18),
    (8, 64, 4, 16, 8, 0.05, 19),
])
def test_reduce_equals_no_replication_gradient(R, E, K, S, slots, skew, seed):
    _reduce_case(R, E, K, S, slots, skew, seed)


def _reduce_case(R, E, K, S, slots, skew, seed):
    """Each assignment contributes a gradient vector to its expert; with replicas the
    contributions are split between the home slab and the replica slabs, and the reduce
    must give back the per-expert total (up to fp32 summation order)."""
    rng = np.random.default_rng(seed)
    G_el = 37
    ids = _random_loads(rng, R, E, K, S, skew)
    p = O.plan(ids, R, E, K, S, slots)
    assert p.n_replicas > 0 and p.n_fallback == 0
    dst = O.slot_map(p, ids).reshape(-1)
    contrib = rng.standard_normal((R * S * K, G_el)).astype(np.float32) * 1e-3
    flat = ids.reshape(-1)
    home = np.zeros((E, G_el), dtype=np.float32)
    rep = np.zeros((R, slots, G_el), dtype=np.float32)
    # which group (home expert or slot) of which rank each row lies in
    for i, row in enumerate(dst):
        r, loc = divmod(int(row), p.sz.NvS)
        gs = [g for g in range(p.sz.G) if p.off[r, g] <= loc < p.off[r, g] + p.group_size[r, g]]
        assert len(gs) == 1
        g = gs[0]
        if g < p.sz.E_loc:
            assert r * p.sz.E_loc + g == flat[i]
            home[flat[i]] += contrib[i]
        else:
            assert p.slot_expert[r, g - p.sz.E_loc] == flat[i]
            rep[r, g - p.sz.E_loc] += contrib[i]
    out = O.reduce_grad(p, home, rep)
    ref = np.zeros((E, G_el), dtype=np.float64)
    np.add.at(ref, flat, contrib.astype(np.float64))
    assert_close(out, ref, RTOL_FP32)
    return p


def test_reduce_exercises_several_slots_per_rank():
    p = _reduce_case(4, 32, 2, 40, 8, 0.08, 18)
    per_rank = collections.Counter(int(r) for r in p.pieces[p.pieces[:, 2] >= 0][:, 1])
    assert max(per_rank.values()) >= 2


def test_combine_rounding_golden():
    g = json.load(open(os.path.join(GOLDEN, "combine_rounding.json")))
    for case in g["cases"]:
        K = len(case["w"])
        y = np.array(case["y_bits"], dtype=np.uint16)[:, None]
        dst = np.arange(K)[None, :]
        w = np.array(case["w"], dtype=np.float32)[None, :]
        out = O.combine(dst, w, y)
        assert int(out[0, 0]) == case["out_bits"], case["name"]


# ----------------------------------------------------------------------------------------
# bf16 helpers against torch
# ----------------------------------------------------------------------------------------

def test_bf16_rne_matches_torch():
    hi = np.arange(1 << 16, dtype=np.uint32) << np.uint32(16)
    lows = np.array([0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x4000, 0xC000], dtype=np.uint32)
    bits = (hi[:, None] | lows[None, :]).reshape(-1)
    rng = np.random.default_rng(0)
    bits = np.concatenate([bits, rng.integers(0, 1 << 32, size=1 << 20, dtype=np.uint64).astype(np.uint32)])
    f = bits.view(np.float32)
    ours = O.f32_to_bf16_rne(f)
    theirs = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(f)
    assert (ours[~nan] == theirs[~nan]).all()
    # NaN stays NaN (payload conventions differ between implementations)
    assert np.isnan(O.bf16_to_f32(ours[nan])).all() and np.isnan(O.bf16_to_f32(theirs[nan])).all()
    # widening is exact
    u = np.arange(1 << 16, dtype=np.uint16)
    t = torch.from_numpy(u.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    w = O.bf16_to_f32(u)
    same = (w.view(np.uint32) == t.view(np.uint32)) | (np.isnan(w) & np.isnan(t))
    assert same.all()


# ----------------------------------------------------------------------------------------
# the five workloads at full size (routing generated on the CPU)
# ----------------------------------------------------------------------------------------

def _vector_invariants(p, dst):
    sz = p.sz
    flat = dst.reshape(-1)
    assert len(np.unique(flat)) == sz.A
    valid = np.zeros(sz.R * sz.NvS, dtype=bool)
    for r in range(sz.R):
        assert p.group_size[r].sum() == sz.C
        for g in range(sz.G + 1):
            lo = r * sz.NvS + p.off[r, g]
            valid[lo:lo + p.group_size[r, g]] = True
    assert valid[flat].all() and valid.sum() == sz.A


@pytest.mark.parametrize("wl,mi", [(w, i) for w in __import__("gen").WORKLOADS
                                   for i in range(len(w.maxvio))],
                         ids=lambda v: getattr(v, "name", str(v)))
def test_workload_plans(wl, mi):
    ids, wt, alpha, mv = make_routing(wl.R, wl.E, wl.K, wl.S, wl.maxvio[mi], wl.seed(mi))
    assert abs(mv - wl.maxvio[mi]) <= 0.05 * wl.maxvio[mi]
    p = O.plan(ids.numpy(), wl.R, wl.E, wl.K, wl.S, wl.slots)
    dst = O.slot_map(p, ids.numpy())
    _vector_invariants(p, dst)
    shed_u, pieces_u = unit_step_plan(p.load.tolist(), wl.R, wl.E, wl.K, wl.S, wl.slots)
    assert [tuple(x) for x in p.pieces.tolist()] == pieces_u
    if wl.slots == wl.E // wl.R:
        # training budget E/R: these routings need no fallback
        assert p.n_fallback == 0


# ----------------------------------------------------------------------------------------
# backward pair
# ----------------------------------------------------------------------------------------

def _bwd_case(seed=20260102):
    w, ids, wt, x = _tiny_inputs(seed=seed)
    p = O.plan(ids, w.R, w.E, w.K, w.S, w.slots)
    dst = O.slot_map(p, ids)
    rows = w.R * p.sz.NvS
    rng = np.random.default_rng(seed)
    g_recv = O.f32_to_bf16_rne(rng.standard_normal((rows, w.H)).astype(np.float32))
    dout = O.f32_to_bf16_rne(rng.standard_normal((w.T, w.H)).astype(np.float32))
    y = O.f32_to_bf16_rne(rng.standard_normal((rows, w.H)).astype(np.float32))
    return w, ids, wt, x, p, dst, rows, g_recv, dout, y


def test_dispatch_bwd_is_the_adjoint_of_dispatch():
    """<dispatch(x), g> == <x, dispatch_bwd(g)> over the mapped rows (float64; the
    bf16 rounding of gx is undone by comparing against the fp32 sums' tolerance)."""
    w, ids, wt, x, p, dst, rows, g_recv, dout, y = _bwd_case()
    recv = O.dispatch(dst, x, rows)
    mapped = np.zeros(rows, dtype=bool)
    mapped[dst.reshape(-1)] = True
    lhs = (O.bf16_to_f32(recv[mapped]).astype(np.float64) *
           O.bf16_to_f32(g_recv[mapped]).astype(np.float64)).sum()
    gx = O.dispatch_bwd(dst, g_recv)
    rhs = (O.bf16_to_f32(x).astype(np.float64) * O.bf16_to_f32(gx).astype(np.float64)).sum()
    # gx is rounded to bf16: bound the rounding by 2^-8 relative per element
    bound = (np.abs(O.bf16_to_f32(x)).astype(np.float64) *
             np.abs(O.bf16_to_f32(gx)).astype(np.float64)).sum() * 2.0 ** -8
    assert abs(lhs - rhs) <= bound
    # and exactly: gx[t] is the rounded fp32 sum of the K gradient rows of token t
    for t in range(0, w.T, 7):
        acc = np.zeros(w.H, dtype=np.float32)
        for k in range(w.K):
            acc = (acc + O.bf16_to_f32(g_recv[dst[t, k]])).astype(np.float32)
        assert (gx[t] == O.f32_to_bf16_rne(acc)).all()


def test_combine_bwd_matches_float64_autograd():
    """Autograd of the plan-free combine out[t] = sum_k w[t,k] * y_{t,k} in float64."""
    w, ids, wt, x, p, dst, rows, g_recv, dout, y = _bwd_case(20260103)
    g_y, dw = O.combine_bwd(dst, wt, dout, y, rows)
    yk = torch.tensor(O.bf16_to_f32(y[dst]).astype(np.float64), requires_grad=True)   # [T,K,H]
    wk = torch.tensor(wt.astype(np.float64), requires_grad=True)                         # [T,K]
    out = (wk[:, :, None] * yk).sum(1)
    out.backward(torch.tensor(O.bf16_to_f32(dout).astype(np.float64)))
    assert_close(dw, wk.grad.numpy(), RTOL_FP32)
    # g_y rows are the rounded per-assignment gradients w * dout
    ref = yk.grad.numpy()                                                                # [T,K,H]
    assert_close(O.bf16_to_f32(g_y[dst]), ref, 2.0 ** -8)
    exact = O.f32_to_bf16_rne((wt[:, :, None] * O.bf16_to_f32(dout)[:, None, :]).astype(np.float32))
    assert (g_y[dst] == exact).all()


def test_backward_round_trip_closed_form():
    """combine_bwd then dispatch_bwd gives sum_k bf16(w[t,k] dout[t]) for each token: the
    gradient of x through dispatch -> identity expert -> combine."""
    w, ids, wt, x, p, dst, rows, g_recv, dout, y = _bwd_case(20260104)
    g_y, dw = O.combine_bwd(dst, wt, dout, y, rows)
    gx = O.dispatch_bwd(dst, g_y)
    d32 = O.bf16_to_f32(dout)
    acc = np.zeros_like(d32)
    for k in range(w.K):
        acc = (acc + O.bf16_to_f32(O.f32_to_bf16_rne((wt[:, k:k + 1] * d32).astype(np.float32)))).astype(np.float32)
    assert (gx == O.f32_to_bf16_rne(acc)).all()
    # weights sum to one, so this is dout up to bf16 rounding of the K pieces
    assert_close(O.bf16_to_f32(gx), d32, 2 * 2.0 ** -8)


# ----------------------------------------------------------------------------------------
# prefetch and the grouped expert stub
# ----------------------------------------------------------------------------------------

@pytest.mark.parametrize("R,E,K,S,slots,skew,seed", [
    (4, 16, 2, 64, 4, 0.2, 31),
    (8, 64, 5, 100, 2, 0.05, 32),      # slots bind: fallback pieces read home weights
])
def test_prefetch_and_stub_equal_no_replication(R, E, K, S, slots, skew, seed):
    rng = np.random.default_rng(seed)
    ids = _random_loads(rng, R, E, K, S, skew)
    p = O.plan(ids, R, E, K, S, slots)
    assert p.n_replicas > 0
    if seed == 32:
        assert p.n_fallback > 0
    H, W_el = 24, 40
    dst = O.slot_map(p, ids)
    x = O.f32_to_bf16_rne(rng.standard_normal((R * S, H)).astype(np.float32))
    home_w = O.f32_to_bf16_rne(rng.standard_normal((E, W_el)).astype(np.float32))
    slot_w = O.prefetch_weight(p, home_w)
    # every used slot holds exactly its replica's home slab
    for (e, r, slot, cnt, start, fbpos) in p.pieces:
        if slot >= 0:
            assert (slot_w[r, slot] == home_w[e]).all()
    recv = O.dispatch(dst, x, R * p.sz.NvS)
    y = O.expert_stub(p, recv, home_w, slot_w, H)
    # no plan: assignment (t, k) applies its own expert to x[t]
    for t in range(R * S):
        for k in range(K):
            e = ids[t, k]
            ref = O.f32_to_bf16_rne((O.bf16_to_f32(x[t]) * O.bf16_to_f32(home_w[e, :H])).astype(np.float32))
            assert (y[dst[t, k]] == ref).all()


def test_staged_equals_zero_copy():
    w, ids, wt, x = _tiny_inputs(seed=20260105)
    p = O.plan(ids, w.R, w.E, w.K, w.S, w.slots)
    dst = O.slot_map(p, ids)
    rows = w.R * p.sz.NvS
    stage, recv_s = O.dispatch_staged(dst, x, rows)
    recv = O.dispatch(dst, x, rows)
    assert (recv_s == recv).all()
    # arrival order: assignment i's staging row holds token i // K
    assert (stage == x[np.arange(w.T * w.K) // w.K]).all()
    stage_c, out_s = O.combine_staged(dst, wt, recv)
    assert (out_s == O.combine(dst, wt, recv)).all()
    assert (stage_c == recv[dst.reshape(-1)]).all()
