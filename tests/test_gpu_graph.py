"""Static shapes and no host sync ("MoonshotAI/MoonEP 딥다이브", section 2, point 3, and
section 4, design pattern 2): the whole plan -> dispatch -> combine step can be captured
once in a HIP graph and replayed for new router outputs of the same sizes.  Each replay
is checked against an eager run of the same inputs, with eager work and synchronisation
between replays."""

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


@pytest.mark.parametrize("R,E,K,S,slots,H", [(8, 64, 6, 256, 8, 512), (16, 128, 8, 128, 2, 256)])
def test_captured_step_replays_match_eager(R, E, K, S, slots, H):
    say(f"graph capture R={R} E={E} K={K} S={S} slots={slots} H={H}")
    T = R * S
    ids_buf = torch.empty(T, K, dtype=torch.int32, device="cuda")
    w_buf = torch.empty(T, K, dtype=torch.float32, device="cuda")
    x_buf = torch.empty(T, H, dtype=torch.bfloat16, device="cuda")

    def load_inputs(i):
        ids, w, _, _ = make_routing(R, E, K, S, [0.5, 3.0, 8.0, 1.0][i % 4], 555 + i, device="cuda")
        ids_buf.copy_(ids)
        w_buf.copy_(w)
        x_buf.copy_(make_hidden(T, H, 700 + i, device="cuda"))

    load_inputs(0)
    plan = M.moonep_plan(ids_buf, w_buf, R, E, K, S, slots)
    recv = torch.zeros(plan.sz.recv_rows, H, dtype=torch.bfloat16, device="cuda")
    out = torch.empty(T, H, dtype=torch.bfloat16, device="cuda")
    M.moonep_dispatch(plan, x_buf, recv)
    M.moonep_combine(plan, recv, out)
    torch.cuda.synchronize()

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            M.moonep_plan(ids_buf, w_buf, R, E, K, S, slots, plan=plan)
            M.moonep_dispatch(plan, x_buf, recv)
            M.moonep_combine(plan, recv, out)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()

    eager_plan = None
    for i in range(1, 5):
        load_inputs(i)                      # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got_dst = plan.dst_row.clone()
        got_out = out.clone()
        eager_plan = M.moonep_plan(ids_buf, w_buf, R, E, K, S, slots, plan=eager_plan)
        e_recv = M.moonep_dispatch(eager_plan, x_buf)
        e_out = M.moonep_combine(eager_plan, e_recv)
        torch.cuda.synchronize()
        assert torch.equal(got_dst, eager_plan.dst_row), f"replay {i}: dst_row"
        assert torch.equal(got_out, e_out), f"replay {i}: combine output"
        st = M.moonep_plan_status(eager_plan)
        assert st["status"] == 0
    torch.cuda.synchronize()
