"""GPU checks of the benchmark's memory streams (libmoonep_streams.so): the ceilings the
hot path is measured against come from kernels that move exactly the bytes they claim.

Each stream runs on small buffers whose results are checked in full: the copy is a bit
copy, the write stores its documented pattern, the read leaves its sink alone, the row
fan-out writes each source row to every listed row and nothing else, and the row gather
writes the XOR of the listed rows (rows outside the buffer skipped) or nothing at all.
The gather's residency-capped launch (a source above 256 MB) is covered too, and the
row update (the combine backward's mix) writes each listed row of b as that row of a XOR
its source row."""

import numpy as np
import pytest
import torch

from combine_top_id_amd import streams as ST

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    ST.lib()


def _rand_rows(n, row_vec, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    return torch.randint(-2 ** 31, 2 ** 31 - 1, (n, row_vec * 4), generator=g, dtype=torch.int64,
                         device="cuda").to(torch.int32)


@pytest.mark.parametrize("shape", [ST.SHAPE_WAVE_2K, ST.SHAPE_BLOCK_4K])
@pytest.mark.parametrize("policy", [0, 1])
def test_linear_streams(shape, policy):
    nvec = 128 * 37 + 5                      # several workgroups and a ragged tail
    src = _rand_rows(nvec, 1, 11)
    dst = torch.zeros_like(src)
    ST.copy(src, dst, shape=shape, policy=policy)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)
    ST.write(dst, shape=shape, policy=policy)
    torch.cuda.synchronize()
    want = torch.stack([torch.arange(nvec, dtype=torch.int64, device="cuda").to(torch.int32),
                        torch.full((nvec,), 0x5A5A5A5A, dtype=torch.int32, device="cuda"),
                        torch.full((nvec,), 0x3C3C3C3C, dtype=torch.int32, device="cuda"),
                        torch.zeros(nvec, dtype=torch.int32, device="cuda")], dim=1)
    assert torch.equal(dst, want)
    sink = torch.full((4,), 7, dtype=torch.int32, device="cuda")
    ST.read(src, sink, shape=shape, policy=policy)
    torch.cuda.synchronize()
    assert (sink == 7).all()


def _row_list(n, K, nrows, seed):
    rng = np.random.default_rng(seed)
    rows = rng.permutation(nrows)[: n * K].astype(np.int32)
    rows[::7] = -1                           # skipped
    rows[3::11] = nrows + 5                  # outside the buffer: skipped
    return rows


@pytest.mark.parametrize("row_vec,K", [(64, 8), (200, 3), (896, 8)])
def test_row_fanout(row_vec, K):
    n, nrows = 37, 400
    rows = _row_list(n, K, nrows, 5)
    src = _rand_rows(n, row_vec, 21)
    dst = torch.zeros(nrows, row_vec * 4, dtype=torch.int32, device="cuda")
    ST.fanout(torch.from_numpy(rows).cuda(), K, src, dst, read_src=True)
    torch.cuda.synchronize()
    want = np.zeros((nrows, row_vec * 4), dtype=np.int32)
    s_np = src.cpu().numpy()
    for i in range(n):
        for k in range(K):
            r = rows[i * K + k]
            if 0 <= r < nrows:
                want[r] = s_np[i]
    assert (dst.cpu().numpy() == want).all()
    # writes only: the pattern (i, vector, 0x77777777, 1) in every listed row
    dst.zero_()
    ST.fanout(torch.from_numpy(rows).cuda(), K, src, dst, read_src=False)
    torch.cuda.synchronize()
    got = dst.cpu().numpy().reshape(nrows, row_vec, 4)
    for i in range(n):
        for k in range(K):
            r = rows[i * K + k]
            if 0 <= r < nrows:
                assert (got[r, :, 0] == i).all() and (got[r, :, 1] == np.arange(row_vec)).all()
                assert (got[r, :, 2] == 0x77777777).all() and (got[r, :, 3] == 1).all()


@pytest.mark.parametrize("row_vec,K,nrows", [(64, 8, 400), (200, 3, 400), (896, 8, 20000)])
def test_row_gather(row_vec, K, nrows):
    # the last case's source is 287 MB, above the last-level cache: the capped launch
    n = 41
    rows = _row_list(n, K, nrows, 9)
    src = _rand_rows(nrows, row_vec, 31)
    dst = torch.zeros(n, row_vec * 4, dtype=torch.int32, device="cuda")
    ST.gather(torch.from_numpy(rows).cuda(), K, src, dst, write_dst=True)
    torch.cuda.synchronize()
    s_np = src.cpu().numpy()
    want = np.zeros((n, row_vec * 4), dtype=np.int32)
    for i in range(n):
        for k in range(K):
            r = rows[i * K + k]
            if 0 <= r < nrows:
                want[i] ^= s_np[r]
    assert (dst.cpu().numpy() == want).all()
    dst.fill_(3)
    ST.gather(torch.from_numpy(rows).cuda(), K, src, dst, write_dst=False)
    torch.cuda.synchronize()
    assert (dst == 3).all()


@pytest.mark.parametrize("row_vec,K,nrows", [(64, 8, 400), (200, 3, 400), (896, 8, 400), (1100, 10, 500),
                                             (2100, 4, 200)])
def test_row_update(row_vec, K, nrows):
    n = 37
    rows = _row_list(n, K, nrows, 13)
    src = _rand_rows(n, row_vec, 41)
    a = _rand_rows(nrows, row_vec, 43)
    b = torch.zeros_like(a)
    ST.update(torch.from_numpy(rows).cuda(), K, src, a, b)
    torch.cuda.synchronize()
    s_np, a_np = src.cpu().numpy(), a.cpu().numpy()
    want = np.zeros_like(a_np)
    for i in range(n):
        for k in range(K):
            r = rows[i * K + k]
            if 0 <= r < nrows:
                want[r] = a_np[r] ^ s_np[i]
    assert (b.cpu().numpy() == want).all()
