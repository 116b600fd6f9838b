"""GPU parity of the backward pair (dispatch-bwd, combine-bwd) against the CPU oracle.

Bar: gx and g_y bit-exact (same fp32 operation order as the oracle); dw, an fp32 dot
product whose summation order the GPU chooses, within rtol 1e-5 of the oracle's float64
dot (tolerance form: |a-b| <= rtol * (|b| + rms(b))).
"""

import numpy as np
import pytest
import torch

import combine_top_id_amd as M
from gen import DSV3, DECODE, make_routing, make_hidden, bf16_bits, bits_to_bf16
from oracle import moonep_oracle as O
from tests.gpu_util import say, to_dev_ids
from tests.tol import assert_close, RTOL_FP32

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    M.lib()


def bwd_case(R, E, K, S, slots, H, mv, seed):
    say(f"backward R={R} E={E} K={K} S={S} slots={slots} H={H} maxvio={mv}")
    ids, wt, _, _ = make_routing(R, E, K, S, mv, seed)
    ids_np, w_np = ids.numpy(), wt.numpy()
    plan = M.moonep_plan(*to_dev_ids(ids_np, w_np), R, E, K, S, slots)
    p = O.plan(ids_np, R, E, K, S, slots)
    dst = O.slot_map(p, ids_np)
    rows = plan.sz.recv_rows
    g_recv = make_hidden(rows, H, seed + 5, device="cuda")
    y = make_hidden(rows, H, seed + 6, device="cuda")
    dout = make_hidden(R * S, H, seed + 7, device="cuda")

    gx = M.moonep_dispatch_bwd(plan, g_recv)
    ref_gx = O.dispatch_bwd(dst, bf16_bits(g_recv))
    assert (bf16_bits(gx) == ref_gx).all(), "dispatch_bwd"

    g_y = torch.full_like(y, float("nan"))
    g_y, dw = M.moonep_combine_bwd(plan, dout, y, g_y=g_y)
    ref_gy, ref_dw = O.combine_bwd(dst, w_np, bf16_bits(dout), bf16_bits(y), rows)
    got_gy = bf16_bits(g_y)
    m = dst.reshape(-1)
    assert (got_gy[m] == ref_gy[m]).all(), "combine_bwd g_y"
    untouched = np.ones(rows, dtype=bool)
    untouched[m] = False
    assert np.isnan(O.bf16_to_f32(got_gy[untouched])).all(), "padding rows must not be written"
    assert_close(dw.cpu().numpy(), ref_dw, RTOL_FP32)

    # in place: g_y written over y itself gives the same rows and dw
    y2 = y.clone()
    g2, dw2 = M.moonep_combine_bwd(plan, dout, y2, g_y=y2)
    assert (bf16_bits(g2)[m] == ref_gy[m]).all()
    assert torch.equal(dw2, dw)
    torch.cuda.synchronize()


@pytest.mark.parametrize("R,E,K,S,slots,H,mv", [
    (4, 16, 2, 64, 4, 128, 2.0),
    (8, 64, 6, 300, 8, 2048, 0.2),
    (8, 64, 5, 300, 2, 1000, 4.0),       # fallback pieces, odd K, ragged H
    (16, 64, 3, 200, 4, 8, 3.0),         # generic-K path, one vector per row
    (64, 384, 8, 40, 4, 520, 20.0),
])
def test_backward_small(R, E, K, S, slots, H, mv):
    bwd_case(R, E, K, S, slots, H, mv, 4242 + R + E + K)


@pytest.mark.parametrize("wl,mi", [(DSV3, 3), (DECODE, 0)], ids=lambda v: getattr(v, "name", str(v)))
def test_backward_full_size(wl, mi):
    """Full size: gx and g_y checked on every mapped row with torch on the GPU (a property
    of the bit-exact definitions), dw on sampled tokens against the oracle."""
    seed = wl.seed(mi)
    say(f"backward full size {wl.name} maxvio={wl.maxvio[mi]}")
    ids, wt, _, _ = make_routing(wl.R, wl.E, wl.K, wl.S, wl.maxvio[mi], seed, device="cuda")
    plan = M.moonep_plan(ids, wt, wl.R, wl.E, wl.K, wl.S, wl.slots)
    ids_np, w_np = ids.cpu().numpy(), wt.cpu().numpy()
    p = O.plan(ids_np, wl.R, wl.E, wl.K, wl.S, wl.slots)
    dst = O.slot_map(p, ids_np)
    assert (plan.dst_row.cpu().numpy() == dst).all()
    rows = plan.sz.recv_rows
    y = make_hidden(rows, wl.H, seed + 6, device="cuda")
    dout = make_hidden(wl.T, wl.H, seed + 7, device="cuda")
    g_y, dw = M.moonep_combine_bwd(plan, dout, y)
    gx = M.moonep_dispatch_bwd(plan, g_y)
    d_t = torch.from_numpy(dst.astype(np.int64)).cuda()
    wt_d = wt.cuda()
    for c0 in range(0, wl.T, 2048):
        c1 = min(c0 + 2048, wl.T)
        dd = dout[c0:c1].float()
        exp = (wt_d[c0:c1, :, None] * dd[:, None, :]).to(torch.bfloat16)      # [n,K,H]
        got = g_y[d_t[c0:c1].reshape(-1)].view(c1 - c0, wl.K, wl.H)
        assert torch.equal(got.view(torch.int16), exp.view(torch.int16)), "g_y"
        acc = torch.zeros_like(dd)
        for k in range(wl.K):
            acc = acc + got[:, k].float()
        assert torch.equal(gx[c0:c1].view(torch.int16), acc.to(torch.bfloat16).view(torch.int16)), "gx"
    rng = np.random.default_rng(seed)
    tok = np.sort(rng.choice(wl.T, 256, replace=False))
    t_t = torch.from_numpy(tok).cuda()
    d_s = bf16_bits(dout[t_t])
    y_s = bf16_bits(y[d_t[t_t].reshape(-1)]).reshape(len(tok) * wl.K, wl.H)
    local = np.arange(len(tok) * wl.K).reshape(len(tok), wl.K)
    _, ref_dw = O.combine_bwd(local, w_np[tok], d_s, y_s, len(tok) * wl.K)
    assert_close(dw[t_t].cpu().numpy(), ref_dw, RTOL_FP32)
    torch.cuda.synchronize()
