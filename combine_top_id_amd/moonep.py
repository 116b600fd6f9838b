"""Thin ctypes binding of libmoonep.so (the C ABI in include/moonep.h).

Argument marshalling only: torch tensors supply device pointers and the current HIP
stream; every step of the path runs in the library's HIP kernels.  There is no CPU
fallback: if the library is not built, or no GPU is present, calls raise.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoonep.so")

MOONEP_OK = 0
ROW_ALIGN = 16


class MoonepError(RuntimeError):
    pass


class Sizes(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("R", "E", "K", "S", "slots", "E_loc", "C", "G",
                                              "NvS", "P_max")] + \
               [(n, ctypes.c_int64) for n in ("T", "A", "recv_rows", "plan_bytes",
                                              "workspace_bytes")] + \
               [(n, ctypes.c_int32) for n in ("nblk", "blk")] + \
               [(n, ctypes.c_int64) for n in ("o_hdr", "o_load", "o_shed", "o_keep",
                                              "o_home_row", "o_pfirst", "o_pnum", "o_pieces",
                                              "o_slot_expert", "o_off", "o_red", "o_xtab",
                                              "o_ptab", "o_dst_row", "o_w")]


class PlanDesc(ctypes.Structure):
    _fields_ = [("magic", ctypes.c_uint32), ("sz", Sizes), ("dev", ctypes.c_void_p)]


class PlanStats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("status", "bad_index", "n_pieces", "n_replicas",
                                              "n_fallback", "max_pieces_per_rank", "n_red",
                                              "n_shed", "max_load")]


_lib = None


def lib():
    """Load libmoonep.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise MoonepError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    L.moonep_query.argtypes = [i32, i32, i32, i32, i32, ctypes.POINTER(Sizes)]
    L.moonep_plan.argtypes = [vp, vp, i32, i32, i32, i32, i32, vp, vp, ctypes.POINTER(PlanDesc), vp]
    L.moonep_plan_noalloc.argtypes = [vp, vp, i32, i32, i32, i32, i32, vp, ctypes.POINTER(PlanDesc),
                                      vp]
    L.moonep_dispatch.argtypes = [ctypes.POINTER(PlanDesc), vp, i32, vp, vp]
    L.moonep_combine.argtypes = [ctypes.POINTER(PlanDesc), vp, i32, vp, vp]
    L.moonep_reduce_grad.argtypes = [ctypes.POINTER(PlanDesc), vp, vp, i64, vp]
    L.moonep_dispatch_bwd.argtypes = [ctypes.POINTER(PlanDesc), vp, i32, vp, vp]
    L.moonep_combine_bwd.argtypes = [ctypes.POINTER(PlanDesc), vp, vp, i32, vp, vp, vp]
    L.moonep_dispatch_staged.argtypes = [ctypes.POINTER(PlanDesc), vp, i32, vp, vp, vp]
    L.moonep_combine_staged.argtypes = [ctypes.POINTER(PlanDesc), vp, i32, vp, vp, vp]
    L.moonep_prefetch_weight.argtypes = [ctypes.POINTER(PlanDesc), vp, i64, vp, vp]
    L.moonep_expert_stub.argtypes = [ctypes.POINTER(PlanDesc), vp, vp, vp, vp, i64, i32, vp, vp]
    L.moonep_plan_status.argtypes = [ctypes.POINTER(PlanDesc), ctypes.POINTER(PlanStats), vp]
    L.moonep_strerror.argtypes = [i32]
    L.moonep_strerror.restype = ctypes.c_char_p
    for f in ("moonep_query", "moonep_plan", "moonep_plan_noalloc", "moonep_dispatch",
              "moonep_combine",
              "moonep_reduce_grad", "moonep_plan_status", "moonep_dispatch_bwd",
              "moonep_combine_bwd", "moonep_prefetch_weight", "moonep_expert_stub",
              "moonep_dispatch_staged", "moonep_combine_staged"):
        getattr(L, f).restype = i32
    _lib = L
    return L


EXPORTS = ("moonep_query", "moonep_plan", "moonep_plan_noalloc", "moonep_dispatch",
           "moonep_combine",
           "moonep_reduce_grad", "moonep_plan_status", "moonep_strerror",
           "moonep_dispatch_bwd", "moonep_combine_bwd", "moonep_prefetch_weight",
           "moonep_expert_stub", "moonep_dispatch_staged", "moonep_combine_staged")


def _check(rc):
    if rc != MOONEP_OK:
        raise MoonepError(f"moonep error {rc}: {lib().moonep_strerror(rc).decode()}")


def _stream(stream, device):
    """The HIP stream handle to enqueue on: `stream`, else the current stream of the
    tensors' device (not of whichever device happens to be current)."""
    if stream is None:
        stream = torch.cuda.current_stream(device)
    elif stream.device != device:
        raise MoonepError(f"stream is on {stream.device}, the tensors on {device}")
    return ctypes.c_void_p(stream.cuda_stream)


def _dev(t, dtype, name, device=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise MoonepError(f"{name} must be a GPU tensor")
    if device is not None and t.device != device:
        raise MoonepError(f"{name} is on {t.device}, the plan on {device}")
    if t.dtype != dtype:
        raise MoonepError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise MoonepError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def moonep_query(R, E, K, S, slots) -> Sizes:
    s = Sizes()
    _check(lib().moonep_query(R, E, K, S, slots, ctypes.byref(s)))
    return s


class Plan:
    """A plan: host descriptor + the device blob it describes (+ its workspace)."""

    def __init__(self, sizes, blob, workspace):
        self.sz = sizes
        self.blob = blob
        self.workspace = workspace
        self.desc = PlanDesc()

    @property
    def NvS(self):
        return self.sz.NvS

    def array(self, name, count):
        """A view of one int32 array of the device blob (offset field `o_<name>`)."""
        o = getattr(self.sz, "o_" + name)
        return self.blob[o:o + count]

    @property
    def dst_row(self):
        return self.array("dst_row", self.sz.A).view(self.sz.T, self.sz.K)

    @property
    def weights(self):
        return self.array("w", self.sz.A).view(torch.float32).view(self.sz.T, self.sz.K)


def _blob(nbytes, device, zero=False):
    # int32 elements; torch's caching allocator returns 256-byte aligned blocks
    n = (nbytes + 3) // 4
    t = (torch.zeros if zero else torch.empty)(n, dtype=torch.int32, device=device)
    assert t.data_ptr() % 256 == 0
    return t


def moonep_plan(topk_ids, topk_w, R, E, K, S, slots, plan=None, stream=None) -> Plan:
    """Enqueue the planning kernels; returns the Plan (reusable by dispatch, combine and
    reduce).  Pass `plan` to reuse its blob and workspace (same sizes)."""
    sz = moonep_query(R, E, K, S, slots)
    ids_p = _dev(topk_ids, torch.int32, "topk_ids")
    w_p = _dev(topk_w, torch.float32, "topk_w", topk_ids.device)
    if topk_ids.numel() != sz.A or topk_w.numel() != sz.A:
        raise MoonepError("topk_ids / topk_w must hold R*S*K elements")
    if plan is None or plan.workspace is None or plan.sz.plan_bytes != sz.plan_bytes or \
            plan.sz.workspace_bytes != sz.workspace_bytes:
        # the workspace starts zero-filled; every plan call leaves it so
        plan = Plan(sz, _blob(sz.plan_bytes, topk_ids.device),
                    _blob(sz.workspace_bytes, topk_ids.device, zero=True))
    plan.sz = sz
    _check(lib().moonep_plan(ids_p, w_p, R, E, K, S, slots,
                             ctypes.c_void_p(plan.blob.data_ptr()),
                             ctypes.c_void_p(plan.workspace.data_ptr()),
                             ctypes.byref(plan.desc), _stream(stream, topk_ids.device)))
    return plan


def moonep_plan_noalloc(topk_ids, topk_w, R, E, K, S, slots, plan=None, stream=None) -> Plan:
    """moonep_plan through the entry point that allocates nothing: the planning workspace is
    the library's static per-GPU array (at most MOONEP_NOALLOC_WORKSPACE_MAX bytes).  The
    plan blob is the caller's (`plan`'s, else one allocated here, outside the C call)."""
    sz = moonep_query(R, E, K, S, slots)
    D = topk_ids.device
    ids_p = _dev(topk_ids, torch.int32, "topk_ids")
    w_p = _dev(topk_w, torch.float32, "topk_w", D)
    if topk_ids.numel() != sz.A or topk_w.numel() != sz.A:
        raise MoonepError("topk_ids / topk_w must hold R*S*K elements")
    if plan is None or plan.sz.plan_bytes != sz.plan_bytes or plan.blob.device != D:
        plan = Plan(sz, _blob(sz.plan_bytes, D), None)
    plan.sz = sz
    with torch.cuda.device(D):       # the library uses the current device's array
        _check(lib().moonep_plan_noalloc(ids_p, w_p, R, E, K, S, slots,
                                         ctypes.c_void_p(plan.blob.data_ptr()),
                                         ctypes.byref(plan.desc), _stream(stream, D)))
    return plan


def moonep_dispatch(plan: Plan, x, recv=None, stream=None):
    """recv[dst_row[t, k]] = x[t]; x is bf16 [T, H]; returns recv bf16 [R*NvS, H]."""
    D = plan.blob.device
    H = x.shape[-1]
    if x.numel() != plan.sz.T * H:
        raise MoonepError("x must be [T, H]")
    if recv is None:
        recv = torch.empty(plan.sz.recv_rows, H, dtype=torch.bfloat16, device=x.device)
    if recv.numel() != plan.sz.recv_rows * H:
        raise MoonepError("recv must be [R*NvS, H]")
    _check(lib().moonep_dispatch(ctypes.byref(plan.desc), _dev(x, torch.bfloat16, "x", D), H,
                                 _dev(recv, torch.bfloat16, "recv", D), _stream(stream, D)))
    return recv


def moonep_combine(plan: Plan, y, out=None, stream=None):
    """out[t] = bf16(sum_k w[t,k] * y[dst_row[t,k]]); y bf16 [R*NvS, H] -> out bf16 [T, H]."""
    D = plan.blob.device
    H = y.shape[-1]
    if y.numel() != plan.sz.recv_rows * H:
        raise MoonepError("y must be [R*NvS, H]")
    if out is None:
        out = torch.empty(plan.sz.T, H, dtype=torch.bfloat16, device=y.device)
    if out.numel() != plan.sz.T * H:
        raise MoonepError("out must be [T, H]")
    _check(lib().moonep_combine(ctypes.byref(plan.desc), _dev(y, torch.bfloat16, "y", D), H,
                                _dev(out, torch.bfloat16, "out", D), _stream(stream, D)))
    return out


def _stage(plan, H, stage, device):
    if stage is None:
        stage = torch.empty(plan.sz.A, H, dtype=torch.bfloat16, device=device)
    if stage.numel() != plan.sz.A * H:
        raise MoonepError("stage must be [T*K, H]")
    return stage


def moonep_dispatch_staged(plan: Plan, x, recv=None, stage=None, stream=None):
    """Non-zero-copy dispatch: x -> stage (arrival order) -> recv (epilogue copy)."""
    D = plan.blob.device
    H = x.shape[-1]
    if x.numel() != plan.sz.T * H:
        raise MoonepError("x must be [T, H]")
    stage = _stage(plan, H, stage, x.device)
    if recv is None:
        recv = torch.empty(plan.sz.recv_rows, H, dtype=torch.bfloat16, device=x.device)
    if recv.numel() != plan.sz.recv_rows * H:
        raise MoonepError("recv must be [R*NvS, H]")
    _check(lib().moonep_dispatch_staged(ctypes.byref(plan.desc), _dev(x, torch.bfloat16, "x", D), H,
                                        _dev(stage, torch.bfloat16, "stage", D),
                                        _dev(recv, torch.bfloat16, "recv", D), _stream(stream, D)))
    return recv


def moonep_combine_staged(plan: Plan, y, out=None, stage=None, stream=None):
    """Non-zero-copy combine: y -> stage (prologue copy) -> weighted sum -> out."""
    D = plan.blob.device
    H = y.shape[-1]
    if y.numel() != plan.sz.recv_rows * H:
        raise MoonepError("y must be [R*NvS, H]")
    stage = _stage(plan, H, stage, y.device)
    if out is None:
        out = torch.empty(plan.sz.T, H, dtype=torch.bfloat16, device=y.device)
    if out.numel() != plan.sz.T * H:
        raise MoonepError("out must be [T, H]")
    _check(lib().moonep_combine_staged(ctypes.byref(plan.desc), _dev(y, torch.bfloat16, "y", D), H,
                                       _dev(stage, torch.bfloat16, "stage", D),
                                       _dev(out, torch.bfloat16, "out", D), _stream(stream, D)))
    return out


def moonep_dispatch_bwd(plan: Plan, g_recv, gx=None, stream=None):
    """gx[t] = bf16(sum_k g_recv[dst_row[t,k]]); g_recv bf16 [R*NvS, H] -> gx bf16 [T, H]."""
    D = plan.blob.device
    H = g_recv.shape[-1]
    if g_recv.numel() != plan.sz.recv_rows * H:
        raise MoonepError("g_recv must be [R*NvS, H]")
    if gx is None:
        gx = torch.empty(plan.sz.T, H, dtype=torch.bfloat16, device=g_recv.device)
    if gx.numel() != plan.sz.T * H:
        raise MoonepError("gx must be [T, H]")
    _check(lib().moonep_dispatch_bwd(ctypes.byref(plan.desc),
                                     _dev(g_recv, torch.bfloat16, "g_recv", D),
                                     H, _dev(gx, torch.bfloat16, "gx", D), _stream(stream, D)))
    return gx


def moonep_combine_bwd(plan: Plan, dout, y, g_y=None, dw=None, stream=None):
    """g_y[dst_row[t,k]] = bf16(w[t,k] * dout[t]); dw[t,k] = <dout[t], y[dst_row[t,k]]>.
    dout bf16 [T, H], y bf16 [R*NvS, H]; returns (g_y bf16 [R*NvS, H], dw fp32 [T, K])."""
    D = plan.blob.device
    H = dout.shape[-1]
    if dout.numel() != plan.sz.T * H or y.numel() != plan.sz.recv_rows * H:
        raise MoonepError("dout must be [T, H] and y [R*NvS, H]")
    if g_y is None:
        g_y = torch.empty(plan.sz.recv_rows, H, dtype=torch.bfloat16, device=dout.device)
    if dw is None:
        dw = torch.empty(plan.sz.T, plan.sz.K, dtype=torch.float32, device=dout.device)
    if g_y.numel() != plan.sz.recv_rows * H or dw.numel() != plan.sz.T * plan.sz.K:
        raise MoonepError("g_y must be [R*NvS, H] and dw [T, K]")
    _check(lib().moonep_combine_bwd(ctypes.byref(plan.desc), _dev(dout, torch.bfloat16, "dout", D),
                                    _dev(y, torch.bfloat16, "y", D), H,
                                    _dev(g_y, torch.bfloat16, "g_y", D),
                                    _dev(dw, torch.float32, "dw", D), _stream(stream, D)))
    return g_y, dw


def moonep_prefetch_weight(plan: Plan, home_w, slot_w=None, stream=None):
    """slot_w[r, slot] = home_w[e] for every slot piece; home_w bf16 [E, W_el] ->
    slot_w bf16 [R, slots, W_el]."""
    D = plan.blob.device
    W_el = home_w.shape[-1]
    if home_w.numel() != plan.sz.E * W_el:
        raise MoonepError("home_w must be [E, W_el]")
    if slot_w is None:
        slot_w = torch.empty(plan.sz.R, plan.sz.slots, W_el, dtype=torch.bfloat16,
                             device=home_w.device)
    if slot_w.numel() != plan.sz.R * plan.sz.slots * W_el:
        raise MoonepError("slot_w must be [R, slots, W_el]")
    sp = _dev(slot_w, torch.bfloat16, "slot_w", D) if slot_w.numel() else ctypes.c_void_p(0)
    _check(lib().moonep_prefetch_weight(ctypes.byref(plan.desc),
                                        _dev(home_w, torch.bfloat16, "home_w", D), W_el, sp,
                                        _stream(stream, D)))
    return slot_w


def moonep_expert_stub(plan: Plan, topk_ids, recv, home_w, slot_w, y=None, stream=None):
    """y[row] = bf16(recv[row] * W[:H]) with W the weight slab the row's group reads."""
    D = plan.blob.device
    H = recv.shape[-1]
    W_el = home_w.shape[-1]
    if topk_ids.numel() != plan.sz.A:
        raise MoonepError("topk_ids must hold R*S*K elements")
    if recv.numel() != plan.sz.recv_rows * H:
        raise MoonepError("recv must be [R*NvS, H]")
    if home_w.numel() != plan.sz.E * W_el or slot_w.numel() != plan.sz.R * plan.sz.slots * W_el:
        raise MoonepError("home_w must be [E, W_el] and slot_w [R, slots, W_el]")
    if y is None:
        y = torch.empty_like(recv)
    if y.numel() != recv.numel():
        raise MoonepError("y must be [R*NvS, H]")
    sp = _dev(slot_w, torch.bfloat16, "slot_w", D) if slot_w.numel() else ctypes.c_void_p(0)
    _check(lib().moonep_expert_stub(ctypes.byref(plan.desc),
                                    _dev(topk_ids, torch.int32, "topk_ids", D),
                                    _dev(recv, torch.bfloat16, "recv", D),
                                    _dev(home_w, torch.bfloat16, "home_w", D), sp, W_el, H,
                                    _dev(y, torch.bfloat16, "y", D), _stream(stream, D)))
    return y


def moonep_reduce_grad(plan: Plan, home_grad, rep_grad, stream=None):
    """home_grad[e] += replica slabs of e (in place); home fp32 [E, G_el], rep fp32
    [R, slots, G_el]."""
    D = plan.blob.device
    G_el = home_grad.shape[-1]
    if home_grad.numel() != plan.sz.E * G_el:
        raise MoonepError("home_grad must be [E, G_el]")
    if rep_grad.numel() != plan.sz.R * plan.sz.slots * G_el:
        raise MoonepError("rep_grad must be [R, slots, G_el]")
    rep_p = _dev(rep_grad, torch.float32, "rep_grad", D) if rep_grad.numel() else ctypes.c_void_p(0)
    _check(lib().moonep_reduce_grad(ctypes.byref(plan.desc),
                                    _dev(home_grad, torch.float32, "home_grad", D), rep_p, G_el,
                                    _stream(stream, D)))
    return home_grad


def moonep_plan_status(plan: Plan, stream=None) -> dict:
    """Wait for the stream, then return the plan's statistics."""
    st = PlanStats()
    _check(lib().moonep_plan_status(ctypes.byref(plan.desc), ctypes.byref(st),
                                    _stream(stream, plan.blob.device)))
    return {n: getattr(st, n) for n, _ in PlanStats._fields_}
