"""CPU oracle for the balanced expert-parallel hot path: plan -> slot map -> zero-copy
dispatch -> weighted combine -> replica-gradient reduce.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the benchmark's CPU
baseline may import this module.  The HIP library never imports, links or calls it, and
it shares no code with the HIP library: it is written from the pages, plainly and slowly,
so that a reader can check each step against them by eye.

Sources (web pages; cited by title and section):
  [news]  "Moonshot AI Open-Sources MoonEP: A Perfectly Balanced Expert Parallelism
          Library for MoE Training" (tldrocket.com), paragraphs 3-5.
  [dive]  "MoonshotAI/MoonEP 딥다이브" (fiv.co.kr, a MoonEP deep dive in Korean),
          numbered sections 1-8.

What the pages fix:
  * every rank receives exactly S*K token-expert assignments, however skewed the router,
    by duplicating a few overloaded experts, planned from live router output [news, para 3];
  * per-rank buffers are a static S*K rows plus alignment padding [dive, section 4,
    design pattern 2];
  * dispatch writes each token row straight into its final expert position, with no
    permute and no staging copy [dive, section 2, point 2];
  * the plan is computed once and reused by combine and the backward passes [dive,
    section 4, design pattern 1];
  * a replica's gradient is summed into its home expert, so training equals training
    with no replication [dive, section 4, design pattern 3];
  * training keeps E/R prefetch slots per rank; inference keeps 3-4 and serves the
    overflow with slower remote reads [news, para 5];
  * dispatch -> no-op -> combine is the identity [dive, section 8, exercise C].

What the pages leave open and this oracle fixes (each reading is listed, with its
reason, in the design notes):
  * experts are homed in contiguous blocks: expert e lives on rank e // (E/R);
  * token t comes from rank t // S; assignment i = t*K + k;
  * shedding walks experts by (load descending, id ascending); an expert on an
    overloaded home sheds min(load, remaining excess of its home);
  * each shed unit goes to the lowest-id rank that still has deficit and a free slot;
    if none has a free slot, to the lowest-id rank that still has deficit, as a
    fallback piece (weights read remotely, slot -1);
  * within an expert, assignments are taken in increasing i (rank, token, k order): the
    home keeps the first `keep`, then the replica pieces in creation order;
  * a rank's buffer holds, in order, its home experts, its slots, then one fallback
    region; each home and slot group starts on a multiple of ROW_ALIGN rows;
  * combine accumulates in fp32, k ascending, a separate multiply then add, and rounds
    to bf16 (round to nearest even) once;
  * reduce adds the slot replicas to the home gradient in piece creation order, fp32.

Parity pins for every function here live in the CPU test-suite; none is unpinned.
"""

from dataclasses import dataclass

import numpy as np

ROW_ALIGN = 16


def align_up(n, a=ROW_ALIGN):
    return (n + a - 1) // a * a


# ----------------------------------------------------------------------------------------
# sizes
# ----------------------------------------------------------------------------------------

@dataclass(frozen=True)
class Sizes:
    R: int
    E: int
    K: int
    S: int
    slots: int

    @property
    def E_loc(self):          # experts homed on each rank
        return self.E // self.R

    @property
    def C(self):              # exact per-rank quota S*K [news, para 3]
        return self.S * self.K

    @property
    def G(self):              # aligned groups per rank: home experts, then slots
        return self.E_loc + self.slots

    @property
    def NvS(self):
        # S*K rows plus alignment padding [dive, section 4, pattern 2]: each of the G
        # aligned groups can waste at most ROW_ALIGN-1 rows; the fallback region after
        # them is not aligned inside.
        return align_up(self.C + self.G * (ROW_ALIGN - 1))

    @property
    def T(self):
        return self.R * self.S

    @property
    def A(self):
        return self.T * self.K


def sizes(R, E, K, S, slots):
    if R < 1 or E < 1 or K < 1 or S < 1 or slots < 0 or E % R != 0 or K > E:
        raise ValueError("invalid sizes")
    return Sizes(R, E, K, S, slots)


# ----------------------------------------------------------------------------------------
# bf16 (bit patterns held as uint16)
# ----------------------------------------------------------------------------------------

def bf16_to_f32(u):
    """bf16 bit patterns -> float32 (exact: the 16 bits are the top half of binary32)."""
    u = np.asarray(u, dtype=np.uint16)
    return (u.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16_rne(a):
    """float32 -> bf16 bit patterns, round to nearest, ties to even; NaN -> 0x7FC0."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    rounded = ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(a)
    return np.where(nan, np.uint16(0x7FC0), rounded).astype(np.uint16)


# ----------------------------------------------------------------------------------------
# plan
# ----------------------------------------------------------------------------------------

@dataclass
class Plan:
    sz: Sizes
    load: np.ndarray          # [E] assignments per expert
    home_load: np.ndarray     # [R] assignments whose expert is homed on the rank
    excess: np.ndarray        # [R] max(0, home_load - S*K) before shedding
    deficit: np.ndarray       # [R] max(0, S*K - home_load) before placing
    order: np.ndarray         # [E] experts by (load desc, id asc)
    shed: np.ndarray          # [E] assignments moved off the home
    keep: np.ndarray          # [E] assignments served at home
    pieces: np.ndarray        # [P, 6] (expert, rank, slot or -1, count, start, fbpos)
    slot_expert: np.ndarray   # [R, slots] expert held in each slot, -1 when unused
    group_size: np.ndarray    # [R, G+1] home groups, slot groups, fallback region
    off: np.ndarray           # [R, G+1] first row of each group

    @property
    def n_pieces(self):
        return len(self.pieces)

    @property
    def n_replicas(self):
        return int((self.pieces[:, 2] >= 0).sum()) if len(self.pieces) else 0

    @property
    def n_fallback(self):
        return int((self.pieces[:, 2] < 0).sum()) if len(self.pieces) else 0

    def piece_row0(self, p):
        """Global row (rank * NvS + row) of the first assignment of piece p."""
        e, r, slot, cnt, start, fbpos = (int(v) for v in self.pieces[p])
        sz = self.sz
        if slot >= 0:
            return r * sz.NvS + int(self.off[r, sz.E_loc + slot])
        return r * sz.NvS + int(self.off[r, sz.G]) + fbpos


def expert_loads(ids, E):
    """load[e] = number of assignments i with ids[i] == e (live router output,
    [news, para 3]).  Duplicate ids within a token count separately."""
    flat = np.asarray(ids).reshape(-1).astype(np.int64)
    if flat.size and (flat.min() < 0 or flat.max() >= E):
        raise ValueError("expert id outside [0, E)")
    load = np.zeros(E, dtype=np.int64)
    np.add.at(load, flat, 1)
    return load


def plan_from_loads(load, sz: Sizes) -> Plan:
    """The replica plan: which overloaded experts are duplicated, onto which ranks and
    slots, and how many assignments each copy serves, so that every rank ends with exactly
    S*K assignments [news, para 3; dive, section 4, pattern 1]."""
    R, E, E_loc, C, G, slots = sz.R, sz.E, sz.E_loc, sz.C, sz.G, sz.slots
    load = np.asarray(load, dtype=np.int64)
    assert load.shape == (E,) and load.sum() == sz.A

    home = np.arange(E) // E_loc
    home_load = np.array([load[home == r].sum() for r in range(R)], dtype=np.int64)
    excess = np.maximum(0, home_load - C)
    deficit = np.maximum(0, C - home_load)
    assert excess.sum() == deficit.sum()

    # experts ordered by load descending, ties by id ascending
    order = np.array(sorted(range(E), key=lambda e: (-int(load[e]), e)), dtype=np.int64)

    # shed: each overloaded home gives away its heaviest experts first, until its excess
    # is gone.
    x_left = excess.copy()
    shed = np.zeros(E, dtype=np.int64)
    for e in order:
        h = home[e]
        if x_left[h] > 0:
            shed[e] = min(load[e], x_left[h])
            x_left[h] -= shed[e]
    keep = load - shed

    # place: shed assignments fill the deficits, lowest-id receiver first; a receiver
    # takes a new replica only while it has a free prefetch slot, otherwise the pieces
    # become fallback pieces served by remote weight reads [news, para 5].
    d_left = deficit.copy()
    used = np.zeros(R, dtype=np.int64)
    fb_rows = np.zeros(R, dtype=np.int64)
    slot_expert = np.full((R, slots), -1, dtype=np.int64)
    pieces = []
    for e in order:
        rem = int(shed[e])
        start = int(keep[e])
        while rem > 0:
            with_slot = [r for r in range(R) if d_left[r] > 0 and used[r] < slots]
            if with_slot:
                r = with_slot[0]
                slot = int(used[r])
                used[r] += 1
                slot_expert[r, slot] = e
                fbpos = 0
            else:
                r = [r for r in range(R) if d_left[r] > 0][0]
                slot = -1
                fbpos = int(fb_rows[r])
            cnt = min(rem, int(d_left[r]))
            if slot < 0:
                fb_rows[r] += cnt
            pieces.append((int(e), int(r), slot, cnt, start, fbpos))
            d_left[r] -= cnt
            rem -= cnt
            start += cnt
    assert d_left.sum() == 0

    # layout of each rank's static buffer: home groups, slot groups, fallback region
    group_size = np.zeros((R, G + 1), dtype=np.int64)
    for r in range(R):
        for g in range(E_loc):
            group_size[r, g] = keep[r * E_loc + g]
        group_size[r, G] = fb_rows[r]
    for (e, r, slot, cnt, start, fbpos) in pieces:
        if slot >= 0:
            group_size[r, E_loc + slot] = cnt
    off = np.zeros((R, G + 1), dtype=np.int64)
    for r in range(R):
        for g in range(G):
            off[r, g + 1] = align_up(off[r, g] + group_size[r, g])

    pieces_arr = np.array(pieces, dtype=np.int64).reshape(-1, 6)
    return Plan(sz, load, home_load, excess, deficit, order, shed, keep, pieces_arr,
                slot_expert, group_size, off)


def plan(ids, R, E, K, S, slots) -> Plan:
    sz = sizes(R, E, K, S, slots)
    ids = np.asarray(ids)
    assert ids.shape == (sz.T, K)
    return plan_from_loads(expert_loads(ids, E), sz)


# ----------------------------------------------------------------------------------------
# token -> slot map
# ----------------------------------------------------------------------------------------

def slot_map(p: Plan, ids) -> np.ndarray:
    """dst_row[t, k]: the global row (rank * NvS + row) that assignment (t, k) is written
    to, its "final expert position" in the receiving rank's static buffer [dive,
    section 2, point 2; section 4, pattern 2]."""
    sz = p.sz
    flat = np.asarray(ids).reshape(-1).astype(np.int64)
    by_expert = np.argsort(flat, kind="stable")       # each expert's i, increasing
    first = np.concatenate([[0], np.cumsum(p.load)])
    dst = np.full(sz.A, -1, dtype=np.int64)
    piece_of = {}
    for q in range(p.n_pieces):
        piece_of.setdefault(int(p.pieces[q, 0]), []).append(q)
    for e in range(sz.E):
        members = by_expert[first[e]:first[e + 1]]
        h = e // sz.E_loc
        home_row0 = h * sz.NvS + p.off[h, e - h * sz.E_loc]
        kp = int(p.keep[e])
        dst[members[:kp]] = home_row0 + np.arange(kp)
        for q in piece_of.get(e, []):
            cnt, start = int(p.pieces[q, 3]), int(p.pieces[q, 4])
            dst[members[start:start + cnt]] = p.piece_row0(q) + np.arange(cnt)
    assert (dst >= 0).all()
    return dst.reshape(sz.T, sz.K)


# ----------------------------------------------------------------------------------------
# dispatch, combine, reduce
# ----------------------------------------------------------------------------------------

def dispatch(dst_row, x_bits, total_rows):
    """Zero-copy dispatch: recv[dst_row[t, k]] = x[t], a bit copy of the bf16 row
    [dive, section 2, point 2].  Rows no assignment maps to stay zero here (their
    contents are unspecified)."""
    dst_row = np.asarray(dst_row)
    T, K = dst_row.shape
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    recv = np.zeros((total_rows, x_bits.shape[1]), dtype=np.uint16)
    src = np.repeat(np.arange(T), K)
    recv[dst_row.reshape(-1)] = x_bits[src]
    return recv


def combine(dst_row, w, y_bits):
    """Weighted combine: out[t] = bf16( sum_k w[t,k] * y[dst_row[t,k]] ), summed in fp32,
    k ascending, each product and each sum rounded to fp32 [dive, section 1:
    dispatch -> expert -> combine]."""
    dst_row = np.asarray(dst_row)
    w = np.asarray(w, dtype=np.float32)
    T, K = dst_row.shape
    acc = np.zeros((T, y_bits.shape[1]), dtype=np.float32)
    for k in range(K):
        rows = bf16_to_f32(y_bits[dst_row[:, k]])
        prod = (w[:, k:k + 1] * rows).astype(np.float32)
        acc = (acc + prod).astype(np.float32)
    return f32_to_bf16_rne(acc)


def reduce_grad(p: Plan, home_grad, rep_grad):
    """home[e] += each slot replica's gradient of e, pieces in creation order, fp32
    [dive, section 4, pattern 3].  Fallback pieces own no slot and add nothing."""
    home = np.array(home_grad, dtype=np.float32, copy=True)
    rep = np.asarray(rep_grad, dtype=np.float32)
    for (e, r, slot, cnt, start, fbpos) in p.pieces:
        if slot >= 0:
            home[e] = (home[e] + rep[r, slot]).astype(np.float32)
    return home


# ----------------------------------------------------------------------------------------
# backward pair, reusing the plan ([dive, section 4, design pattern 1]: the plan computed
# in forward serves both backward passes)
# ----------------------------------------------------------------------------------------

def dispatch_bwd(dst_row, g_recv_bits):
    """Gradient of dispatch with respect to x: dispatch copied x[t] into K rows, so
    gx[t] = bf16( sum_k g_recv[dst_row[t, k]] ), summed in fp32, k ascending."""
    dst_row = np.asarray(dst_row)
    T, K = dst_row.shape
    acc = np.zeros((T, g_recv_bits.shape[1]), dtype=np.float32)
    for k in range(K):
        acc = (acc + bf16_to_f32(g_recv_bits[dst_row[:, k]])).astype(np.float32)
    return f32_to_bf16_rne(acc)


def combine_bwd(dst_row, w, dout_bits, y_bits, total_rows):
    """Gradient of combine out[t] = sum_k w[t,k] * y[dst_row[t,k]]:
      g_y[dst_row[t,k]] = bf16( w[t,k] * dout[t] )   (fp32 product, then bf16 RNE)
      dw[t, k]          = sum_h dout[t,h] * y[dst_row[t,k], h]   (float64 here)
    Rows of g_y no assignment maps to stay zero."""
    dst_row = np.asarray(dst_row)
    w = np.asarray(w, dtype=np.float32)
    T, K = dst_row.shape
    d32 = bf16_to_f32(dout_bits)
    g_y = np.zeros((total_rows, dout_bits.shape[1]), dtype=np.uint16)
    dw = np.zeros((T, K), dtype=np.float64)
    for k in range(K):
        g_y[dst_row[:, k]] = f32_to_bf16_rne((w[:, k:k + 1] * d32).astype(np.float32))
        yk = bf16_to_f32(y_bits[dst_row[:, k]]).astype(np.float64)
        dw[:, k] = (d32.astype(np.float64) * yk).sum(axis=1)
    return g_y, dw


# ----------------------------------------------------------------------------------------
# replica weight prefetch and the grouped expert stub (fallback pieces read home weights)
# ----------------------------------------------------------------------------------------

def prefetch_weight(p: Plan, home_w_bits):
    """Copy each slot replica's home weights into the receiving rank's slot before expert
    compute ([news, para 3]: duplicates are prefetched before computation starts;
    [dive, section 3]: Buffer.prefetch_weight).  home_w [E, W_el] bf16 bits ->
    slot_w [R, slots, W_el]; slots no piece uses stay zero here (unspecified)."""
    sz = p.sz
    home_w_bits = np.asarray(home_w_bits, dtype=np.uint16)
    slot_w = np.zeros((sz.R, sz.slots, home_w_bits.shape[1]), dtype=np.uint16)
    for (e, r, slot, cnt, start, fbpos) in p.pieces:
        if slot >= 0:
            slot_w[r, slot] = home_w_bits[e]
    return slot_w


def expert_stub(p: Plan, recv_bits, home_w_bits, slot_w_bits, H):
    """A toy grouped expert over the rank buffers: y[row, h] = bf16(recv[row, h] * W[h])
    for h < H, where W is the weight slab the row's group uses: its home expert's slab for
    a home group, the rank's prefetched copy for a slot group, and the home slab read
    across partitions for a fallback piece ([news, para 5]).  Rows no assignment maps to
    stay zero here."""
    sz = p.sz
    y = np.zeros_like(recv_bits)

    def apply(rows, w_bits):
        w32 = bf16_to_f32(w_bits[:H])
        y[rows] = f32_to_bf16_rne((bf16_to_f32(recv_bits[rows]) * w32).astype(np.float32))

    for e in range(sz.E):
        h = e // sz.E_loc
        r0 = h * sz.NvS + int(p.off[h, e - h * sz.E_loc])
        apply(np.arange(r0, r0 + int(p.keep[e])), home_w_bits[e])
    for q in range(p.n_pieces):
        e, r, slot, cnt = (int(v) for v in p.pieces[q, :4])
        rows = np.arange(p.piece_row0(q), p.piece_row0(q) + cnt)
        apply(rows, slot_w_bits[r, slot] if slot >= 0 else home_w_bits[e])
    return y


# ----------------------------------------------------------------------------------------
# staged (non-zero-copy) dispatch and combine: the copies zero-copy removes
# ----------------------------------------------------------------------------------------

def dispatch_staged(dst_row, x_bits, total_rows):
    """Rows first land in a staging buffer in arrival order, stage[t*K + k] = x[t]; an
    epilogue then permutes them into their final rows, recv[dst_row[t, k]] =
    stage[t*K + k] ([dive, section 2, point 2]: the receive-then-permute-and-copy scheme
    zero-copy replaces; section 8, exercise D).  Returns (stage, recv)."""
    dst_row = np.asarray(dst_row)
    T, K = dst_row.shape
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    stage = x_bits[np.repeat(np.arange(T), K)]
    recv = np.zeros((total_rows, x_bits.shape[1]), dtype=np.uint16)
    recv[dst_row.reshape(-1)] = stage
    return stage, recv


def combine_staged(dst_row, w, y_bits):
    """Prologue: stage[t*K + k] = y[dst_row[t, k]] (expert outputs gathered back into
    arrival order), then the weighted combine reads the staging buffer in order."""
    dst_row = np.asarray(dst_row)
    T, K = dst_row.shape
    stage = np.asarray(y_bits, dtype=np.uint16)[dst_row.reshape(-1)]
    return stage, combine(np.arange(T * K).reshape(T, K), w, stage)
