"""Helpers for the GPU parity tests: run the HIP path through the C ABI and read its plan
blob back; compare with the oracle."""

import numpy as np
import torch

import combine_top_id_amd as M
from oracle import moonep_oracle as O

HDR = dict(magic=0, status=1, n_pieces=2, n_replicas=3, n_fallback=4, max_ppr=5, n_red=6,
           bad_index=7, n_shed=8, max_load=9)


def say(*a):
    print(*a, flush=True)


def read_plan(plan):
    """The plan blob's arrays on the host."""
    sz = plan.sz
    blob = plan.blob.cpu().numpy()

    def arr(name, n):
        o = getattr(sz, "o_" + name)
        return blob[o:o + n]

    hdr = arr("hdr", 64)
    n_p = int(hdr[HDR["n_pieces"]])
    slots = max(sz.slots, 1)
    return dict(
        hdr={k: int(hdr[v]) for k, v in HDR.items()},
        load=arr("load", sz.E), shed=arr("shed", sz.E), keep=arr("keep", sz.E),
        home_row=arr("home_row", sz.E), pfirst=arr("pfirst", sz.E), pnum=arr("pnum", sz.E),
        pieces=arr("pieces", sz.P_max * 8).reshape(sz.P_max, 8)[:n_p],
        slot_expert=arr("slot_expert", sz.R * slots).reshape(sz.R, slots)[:, :sz.slots],
        off=arr("off", sz.R * (sz.G + 1)).reshape(sz.R, sz.G + 1),
        red=arr("red", sz.E)[:int(hdr[HDR["n_red"]])],
        dst_row=arr("dst_row", sz.A).reshape(sz.T, sz.K),
        w=arr("w", sz.A).view(np.float32).reshape(sz.T, sz.K),
    )


def assert_plan_matches(got, p: O.Plan, dst_ref=None):
    """Bit-exact comparison of every plan array with the oracle's."""
    sz = p.sz
    assert got["hdr"]["status"] == 0
    assert (got["load"] == p.load).all(), "load"
    assert (got["shed"] == p.shed).all(), "shed"
    assert (got["keep"] == p.keep).all(), "keep"
    assert got["hdr"]["n_pieces"] == p.n_pieces
    assert got["hdr"]["n_replicas"] == p.n_replicas
    assert got["hdr"]["n_fallback"] == p.n_fallback
    assert (got["pieces"][:, :6] == p.pieces).all(), "pieces"
    for q in range(p.n_pieces):
        assert got["pieces"][q, 6] == p.piece_row0(q)
    assert (got["slot_expert"] == p.slot_expert).all(), "slot_expert"
    assert (got["off"] == p.off).all(), "off"
    for e in range(sz.E):
        h = e // sz.E_loc
        assert got["home_row"][e] == h * sz.NvS + p.off[h, e - h * sz.E_loc]
    per_rank = np.zeros(sz.R, dtype=np.int64)
    for q in range(p.n_pieces):
        per_rank[p.pieces[q, 1]] += 1
    assert got["hdr"]["max_ppr"] == (per_rank.max() if p.n_pieces else 0)
    assert got["hdr"]["max_load"] == p.load.max()
    # reduce work list: experts with slot pieces, in plan order
    exp_red = []
    for e in p.order:
        rows = p.pieces[p.pieces[:, 0] == e] if p.n_pieces else []
        if len(rows) and rows[0][2] >= 0:
            exp_red.append(int(e))
    assert got["red"].tolist() == exp_red
    if dst_ref is not None:
        assert (got["dst_row"] == dst_ref).all(), "dst_row"


def to_dev_ids(ids_np, w_np, dev="cuda"):
    ids = torch.from_numpy(np.ascontiguousarray(ids_np, dtype=np.int32)).to(dev)
    w = torch.from_numpy(np.ascontiguousarray(w_np, dtype=np.float32)).to(dev)
    return ids, w
