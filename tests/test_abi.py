"""The C ABI libraries load and export every function include/*.h declares
(include/moonep.h: libmoonep.so, the hot path; include/moonep_streams.h:
libmoonep_streams.so, the benchmark's memory streams), and their host-only calls behave
as documented.  No GPU work is launched here: moonep_query and the argument checks of the
other calls run on the host."""

import ctypes
import os
import re

import pytest

import combine_top_id_amd as M
from combine_top_id_amd.moonep import PlanDesc, Sizes
from oracle import moonep_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moonep.h")
STREAMS_HEADER = os.path.join(ROOT, "include", "moonep_streams.h")

EINVAL, ELIMIT, EPLAN, EHIP, EALIGN = -1, -2, -3, -4, -5


def declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moonep_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(M.LIB_PATH):
        pytest.fail("libmoonep.so is not built (run __graft_entry__.build())")
    return M.lib()


def test_every_declared_function_is_exported(lib):
    names = declared_functions()
    assert set(names) == set(M.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), n


def test_headers_cover_every_library():
    hdrs = sorted(f for f in os.listdir(os.path.join(ROOT, "include")) if f.endswith(".h"))
    assert hdrs == ["moonep.h", "moonep_streams.h"], hdrs


def test_streams_library_exports_its_header():
    from combine_top_id_amd import streams
    if not os.path.exists(streams.LIB_PATH):
        pytest.fail("libmoonep_streams.so is not built (run __graft_entry__.build())")
    L = streams.lib()
    names = declared_functions(STREAMS_HEADER)
    assert set(names) == set(streams.EXPORTS), names
    for n in names:
        assert hasattr(L, n), n
    # argument checks run on the host: nothing is launched
    fake = ctypes.c_void_p(256)
    assert L.moonep_stream_read(None, 4096, 1, 1, fake, None) == EINVAL
    assert L.moonep_stream_write(fake, 4095, 1, 1, None) == EINVAL        # not 16-byte sized
    assert L.moonep_stream_copy(fake, fake, 4096, 7, 1, None) == EINVAL    # unknown shape
    assert L.moonep_rows_fanout(fake, 4, 0, fake, fake, 8, 64, 1, None) == EINVAL   # K < 1
    assert L.moonep_rows_gather(fake, 4, 2, fake, 8, fake, 24, 1, None) == EINVAL   # row bytes


@pytest.mark.parametrize("R,E,K,S,slots", [(4, 16, 2, 64, 4), (8, 64, 6, 1024, 8),
                                           (8, 256, 8, 4096, 32), (16, 384, 8, 8192, 24),
                                           (64, 384, 8, 128, 4), (7, 56, 2, 24, 8),
                                           (1, 8, 2, 5, 0)])
def test_query_sizes_match_oracle(R, E, K, S, slots):
    s = M.moonep_query(R, E, K, S, slots)
    sz = O.sizes(R, E, K, S, slots)
    assert (s.R, s.E, s.K, s.S, s.slots) == (R, E, K, S, slots)
    assert s.NvS == sz.NvS and s.C == sz.C and s.G == sz.G and s.E_loc == sz.E_loc
    assert s.T == sz.T and s.A == sz.A and s.recv_rows == R * sz.NvS
    assert s.P_max == E + R
    # every array of the plan blob is 256-byte aligned and inside the blob
    offs = [getattr(s, f) for f, _ in Sizes._fields_ if f.startswith("o_")]
    assert all(o % 64 == 0 for o in offs)
    assert max(offs) * 4 < s.plan_bytes
    assert s.nblk * s.blk >= s.A and (s.nblk - 1) * s.blk < s.A
    assert s.workspace_bytes > 0


def test_query_errors(lib):
    s = Sizes()
    assert lib.moonep_query(3, 16, 2, 4, 4, ctypes.byref(s)) == EINVAL     # E % R
    assert lib.moonep_query(4, 16, 17, 4, 4, ctypes.byref(s)) == EINVAL    # K > E
    assert lib.moonep_query(0, 16, 2, 4, 4, ctypes.byref(s)) == EINVAL
    assert lib.moonep_query(4, 16, 2, 0, 4, ctypes.byref(s)) == EINVAL
    assert lib.moonep_query(4, 16, 2, 4, -1, ctypes.byref(s)) == EINVAL
    assert lib.moonep_query(65, 65, 2, 4, 4, ctypes.byref(s)) == ELIMIT    # R > 64
    assert lib.moonep_query(4, 2048, 2, 4, 4, ctypes.byref(s)) == ELIMIT   # E > 1024
    assert lib.moonep_query(4, 64, 33, 4, 4, ctypes.byref(s)) == ELIMIT    # K > 32
    assert lib.moonep_query(4, 16, 2, 4, 257, ctypes.byref(s)) == ELIMIT   # slots > 256
    assert lib.moonep_query(64, 1024, 32, 1 << 26, 4, ctypes.byref(s)) == ELIMIT  # int32 rows
    assert lib.moonep_query(4, 16, 2, 4, 4, None) == EINVAL


def test_calls_reject_bad_arguments_on_the_host(lib):
    d = PlanDesc()
    fake = ctypes.c_void_p(256)            # never dereferenced: checks fail first
    assert lib.moonep_plan(None, fake, 4, 16, 2, 4, 4, fake, fake, ctypes.byref(d), None) == EINVAL
    assert lib.moonep_plan(fake, fake, 3, 16, 2, 4, 4, fake, fake, ctypes.byref(d), None) == EINVAL
    assert lib.moonep_plan(fake, fake, 4, 16, 2, 4, 4, ctypes.c_void_p(260), fake,
                           ctypes.byref(d), None) == EALIGN
    # the no-allocation variant: the same host checks, and a workspace beyond its static
    # array is refused before any HIP call
    assert lib.moonep_plan_noalloc(None, fake, 4, 16, 2, 4, 4, fake, ctypes.byref(d), None) == EINVAL
    assert lib.moonep_plan_noalloc(fake, fake, 3, 16, 2, 4, 4, fake, ctypes.byref(d), None) == EINVAL
    big = M.moonep_query(64, 1024, 32, 1 << 13, 8)
    assert big.workspace_bytes > (8 << 20)
    assert lib.moonep_plan_noalloc(fake, fake, 64, 1024, 32, 1 << 13, 8, fake, ctypes.byref(d),
                                   None) == ELIMIT
    # an uninitialised descriptor is refused by every call that takes one
    assert lib.moonep_dispatch(ctypes.byref(d), fake, 16, fake, None) == EPLAN
    assert lib.moonep_combine(ctypes.byref(d), fake, 16, fake, None) == EPLAN
    assert lib.moonep_reduce_grad(ctypes.byref(d), fake, fake, 16, None) == EPLAN
    st = M.moonep.PlanStats()
    assert lib.moonep_plan_status(ctypes.byref(d), ctypes.byref(st), None) == EPLAN
    # a descriptor whose sizes were tampered with is refused too
    d.magic = 0x4D4F4E45
    d.dev = 256
    d.sz = M.moonep_query(4, 16, 2, 4, 4)
    d.sz.NvS += 16
    assert lib.moonep_dispatch(ctypes.byref(d), fake, 16, fake, None) == EPLAN


def test_strerror(lib):
    for code in (0, EINVAL, ELIMIT, EPLAN, EHIP, EALIGN, -99):
        assert lib.moonep_strerror(code)
