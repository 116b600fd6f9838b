"""The planning entry point that allocates nothing (moonep_plan_noalloc, for callers that
cannot allocate device memory) against moonep_plan: two calls in a row, the second on a
smaller problem, each bit-identical to moonep_plan's plan blob, on the same stream.  The
C call is reached through the ctypes binding; the plan blob is allocated by the test."""

import pytest
import torch

import combine_top_id_amd as M
from gen import DSV3, TINY, make_routing, make_hidden
from tests.gpu_util import say, read_plan

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    M.lib()


def _fresh(plan_like):
    """A zero-filled plan blob of the same size: the gaps between the blob's arrays are
    never written, so comparing two blobs word for word needs equal starting contents."""
    return M.Plan(plan_like.sz, torch.zeros_like(plan_like.blob), None)


def test_noalloc_plan_matches_plan_twice_then_smaller():
    cases = [(DSV3, 3), (TINY, 0)]       # large first, then a smaller problem
    for wl, mi in cases:
        say(f"noalloc {wl.name} maxvio={wl.maxvio[mi]}")
        ids, w, _, _ = make_routing(wl.R, wl.E, wl.K, wl.S, wl.maxvio[mi], wl.seed(mi), device="cuda")
        ref = M.moonep_plan(ids, w, wl.R, wl.E, wl.K, wl.S, wl.slots)
        ref.blob.zero_()
        ref = M.moonep_plan(ids, w, wl.R, wl.E, wl.K, wl.S, wl.slots, plan=ref)
        got = M.moonep_plan_noalloc(ids, w, wl.R, wl.E, wl.K, wl.S, wl.slots, plan=_fresh(ref))
        torch.cuda.synchronize()
        assert M.moonep_plan_status(got) == M.moonep_plan_status(ref)
        assert torch.equal(got.blob, ref.blob), f"{wl.name}: plan blob differs"
        a, b = read_plan(got), read_plan(ref)
        assert (a["dst_row"] == b["dst_row"]).all()
        # the plan drives dispatch and combine like any other
        x = make_hidden(wl.T, wl.H, wl.seed(mi) + 1, device="cuda")
        r1 = M.moonep_dispatch(ref, x)
        o1 = M.moonep_combine(ref, r1)
        r2 = M.moonep_dispatch(got, x)
        o2 = M.moonep_combine(got, r2)
        assert torch.equal(o1, o2)
        del r1, r2


def test_noalloc_rejects_a_workspace_beyond_its_array():
    # kimi-like sizes with 32 slots fit; a problem whose workspace exceeds 8 MiB is refused
    # on the host before anything is enqueued
    sz = M.moonep_query(64, 1024, 32, 1 << 13, 8)
    assert sz.workspace_bytes > (8 << 20)
    ids = torch.zeros(sz.A, dtype=torch.int32, device="cuda")
    w = torch.zeros(sz.A, dtype=torch.float32, device="cuda")
    with pytest.raises(M.MoonepError, match="limits"):
        M.moonep_plan_noalloc(ids, w, 64, 1024, 32, 1 << 13, 8)
    torch.cuda.synchronize()
