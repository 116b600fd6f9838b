// Planning on the GPU: live top-K router output -> replica plan + token->row map.
//
// "Moonshot AI Open-Sources MoonEP" (tldrocket.com), paragraph 3: every rank receives
// exactly S*K assignments because a few overloaded experts are duplicated, planned
// directly from live router output; paragraph 5: E/R prefetch slots in training, 3-4 in
// inference with remote-read fallback.  "MoonshotAI/MoonEP 딥다이브" (fiv.co.kr),
// section 4, pattern 1: the plan is computed once and reused; pattern 2: static S*K
// plus alignment padding buffers.
//
// Assignments are cut into blocks of `blk` = kMapThreads * M; block b is counted by one
// logical workgroup of kMapWaves waves, whose wave w owns the contiguous sub-block of 64*M
// assignments starting at b*blk + w*64*M.  Two launches on the caller's stream:
//   1. hist_plan_kernel  two logical blocks per workgroup of kPlanThreads.
//        histogram: one LDS histogram per wave -> the block's expert counts and, per
//          wave, the count of earlier waves of the block (and, for waves of more than 8
//          chunks, the wave's running counts at each 8-chunk boundary); the first
//          invalid id of the block.
//        planner, in the workgroup that finishes its histogram last: per-block bases
//          (exclusive scan of the counts over blocks), expert loads, per-rank excess and
//          deficit, shedding, greedy placement (wave 0, lane r = rank r: a parallel cut
//          of the shed stream up to the first expert that would overfill a slot budget,
//          then one expert at a time), buffer layout (one block-wide scan), piece rows,
//          statistics.  Everything stays in LDS until one final write of the plan.
//   2. map_kernel        one single-wave workgroup per map sub-block (a histogram wave's
//                        sub-block, or a part of at most 8 chunks of it, whose starting
//                        counts the histogram wave recorded): the stable rank j of each
//                        assignment among its expert's assignments (per-id LDS peer masks
//                        and an LDS counter per expert), then its row; copies the top-K
//                        weights.
#include <climits>

#include "moonep_internal.h"

namespace moonep {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int l = __lane_id();
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}

// DPP controls (GFX9): shift right within a row of 16 lanes; broadcast lane 15 / 31.
constexpr int kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr4 = 0x114, kRowShr8 = 0x118;
constexpr int kRowBcast15 = 0x142, kRowBcast31 = 0x143;

// Inclusive prefix sum over the 64 lanes of a wave, in data-parallel-primitive moves:
// four shifts inside each row of 16 lanes, then the row totals carried across rows.
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, kRowShr1, 0xf, 0xf, true);
  v += __builtin_amdgcn_update_dpp(0, v, kRowShr2, 0xf, 0xf, true);
  v += __builtin_amdgcn_update_dpp(0, v, kRowShr4, 0xf, 0xf, true);
  v += __builtin_amdgcn_update_dpp(0, v, kRowShr8, 0xf, 0xf, true);
  v += __builtin_amdgcn_update_dpp(0, v, kRowBcast15, 0xa, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, kRowBcast31, 0xc, 0xf, false);
  return v;
}

// Inclusive prefix maximum over the 64 lanes, same moves as wave_incl_scan; for values
// >= 0 (lanes without a source read 0).
__device__ __forceinline__ int wave_incl_max(int v) {
  v = max(v, __builtin_amdgcn_update_dpp(0, v, kRowShr1, 0xf, 0xf, true));
  v = max(v, __builtin_amdgcn_update_dpp(0, v, kRowShr2, 0xf, 0xf, true));
  v = max(v, __builtin_amdgcn_update_dpp(0, v, kRowShr4, 0xf, 0xf, true));
  v = max(v, __builtin_amdgcn_update_dpp(0, v, kRowShr8, 0xf, 0xf, true));
  v = max(v, __builtin_amdgcn_update_dpp(0, v, kRowBcast15, 0xa, 0xf, false));
  v = max(v, __builtin_amdgcn_update_dpp(0, v, kRowBcast31, 0xc, 0xf, false));
  return v;
}

__device__ __forceinline__ int lane63(int v) { return __builtin_amdgcn_readlane(v, 63); }

__device__ __forceinline__ int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

// Number of entries of the ascending array a[0, n) that are <= x.
__device__ __forceinline__ int count_le(const int32_t* a, int n, int x) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (a[mid] <= x) lo = mid + 1; else hi = mid;
  }
  return lo;
}

__device__ __forceinline__ int align_rows(int n) { return (n + kRowAlign - 1) / kRowAlign * kRowAlign; }

// ---------------------------------------------------------------------------------------
// 1. per-block histogram (device function; the launch is hist_plan_kernel below)
// ---------------------------------------------------------------------------------------
// One logical block of kMapWaves waves (tid in [0, kMapThreads)) counts blk assignments
// into its own LDS histograms `lds_blk` ([kMapWaves][E]); b >= nblk counts nothing but
// still takes part in the workgroup's barriers.
template <int M>
__device__ __forceinline__ void hist_block(const int32_t* __restrict__ ids, int32_t* __restrict__ ws,
                                           const moonep_sizes& s, int b, int tid, int32_t* lds_blk,
                                           int* bad) {
  const int E = s.E;
  const bool active = b < s.nblk;
  const int wave = tid >> 6, lane = tid & 63;
  const int64_t i_wave = (int64_t)b * s.blk + (int64_t)wave * (64 * M);
  int idv[M];
#pragma unroll
  for (int c = 0; c < M; ++c) {
    const int64_t i = i_wave + c * 64 + lane;
    idv[c] = active && i < s.A ? ids[i] : 0;
  }
  int32_t* mine = lds_blk + wave * E;
  for (int e = lane; e < E; e += 64) mine[e] = 0;
  if (tid == 0) *bad = INT_MAX;
  __syncthreads();
  int mybad = INT_MAX;
  // Q > 1: the map splits this wave's chunks into Q sub-blocks of MC chunks, and needs
  // the wave's running counts at each inner boundary (one wave's LDS operations take
  // effect in program order, so the reads see every earlier add of the wave)
  constexpr int MC = M < kMapChunks ? M : kMapChunks;
  constexpr int Q = M / MC;
  int32_t* snap = ws + ws_snap(s) + ((int64_t)b * kMapWaves + wave) * (Q - 1) * E;
#pragma unroll
  for (int c = 0; c < M; ++c) {
    if (Q > 1 && active && c > 0 && c % MC == 0) {
      int32_t* sn = snap + (int64_t)(c / MC - 1) * E;
      for (int e = lane; e < E; e += 64) sn[e] = mine[e];
    }
    const int64_t i = i_wave + c * 64 + lane;
    if (active && i < s.A) {
      const int id = idv[c];
      if ((unsigned)id < (unsigned)E)
        atomicAdd(&mine[id], 1);
      else
        mybad = min(mybad, (int)i);
    }
  }
  if (mybad != INT_MAX) atomicMin(bad, mybad);
  __syncthreads();
  if (!active) return;
  int32_t* cnt = ws + (int64_t)b * E;
  int32_t* sub = ws + ws_sub(s) + (int64_t)b * kMapWaves * E;
  for (int e = tid; e < E; e += kMapThreads) {
    int acc = 0;
#pragma unroll
    for (int v = 0; v < kMapWaves; ++v) {
      const int c = lds_blk[v * E + e];
      sub[v * E + e] = acc;
      acc += c;
    }
    cnt[e] = acc;
  }
  if (tid == 0) ws[ws_bad(s) + b] = *bad;
}

// ---------------------------------------------------------------------------------------
// 2. the planner (device function of one workgroup of kPlanThreads)
// ---------------------------------------------------------------------------------------

// Does expert a come before expert b in (load descending, id ascending) order?
__device__ __forceinline__ bool before(int la, int a, int lb, int b) {
  return la > lb || (la == lb && a < b);
}

constexpr int kColRegs = 32;   // block counts a column thread keeps in registers

__device__ __forceinline__ void planner_block(int32_t* __restrict__ plan, int32_t* __restrict__ ws,
                                              const moonep_sizes& s, int32_t* lds) {
  const int E = s.E, R = s.R, E_loc = s.E_loc, C = s.C, slots = s.slots, G = s.G;
  const int NvS = s.NvS, PM = s.P_max;
  int32_t* load_s = lds;            // [E]
  int32_t* shed_s = load_s + E;     // [E]
  int32_t* keep_s = shed_s + E;     // [E]
  int32_t* order_s = keep_s + E;    // [E] shedding experts, plan order
  int32_t* list_s = order_s + E;    // [E] shedding experts, id order
  int32_t* pfirst_s = list_s + E;   // [E]
  int32_t* pnum_s = pfirst_s + E;   // [E]
  int32_t* pe_s = pnum_s + E;             // pieces: expert, rank, slot, count, start,
  int32_t* pr_s = pe_s + PM;              //   [P_max] each
  int32_t* psl_s = pr_s + PM;
  int32_t* pc_s = psl_s + PM;
  int32_t* pst_s = pc_s + PM;
  int32_t* prel_s = pst_s + PM;           //   row inside its slot or fallback region
  int32_t* qbase_s = prel_s + PM;         // [nshed] fast placement's per-expert base
  int32_t* home_s = list_s;         // [E] home group rows, after the ordering is done
  int32_t* part_s = pe_s;           // [kPlanThreads] column segment sums, used before the
                                    // pieces exist
  __shared__ int32_t hl_s[64], used_s[64], fb_s[64], nfb_s[64], sr_s[64], ht_s[64], dend_s[64],
      xs_s[64], wtot_s[kPlanThreads / 64], colbase0_s[64];
  __shared__ int bad_s, nshed_s, npieces_s, err_s, maxload_s;

  int32_t* hdr = plan + s.o_hdr;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const uint64_t lt = lanemask_lt();

  // ---- per-block bases and expert loads -----------------------------------------------------
  // ws[b][e] holds block b's count of expert e.  Each column is split into `tpc` segments
  // of consecutive blocks, one thread per (segment, expert): segment sums, then the
  // exclusive scan over blocks, kept in registers and written back over the counts later
  // (by the waves that are idle during placement; wave 0 at the end).
  if (tid == 0) { bad_s = INT_MAX; err_s = 0; }
  const int nblk = s.nblk;
  int tpc = 1;
  while (tpc * 2 * E <= kPlanThreads && tpc * 2 <= nblk) tpc *= 2;
  const int seg = (nblk + tpc - 1) / tpc;
  const bool col_thread = tid < tpc * E;
  const int ce = tid % E, cg = tid / E;
  const int b0 = cg * seg, b1 = min(b0 + seg, nblk);
  const bool in_regs = seg <= kColRegs;
  int v[kColRegs];
  if (col_thread) {
    int sum = 0;
    if (in_regs) {
#pragma unroll
      for (int u = 0; u < kColRegs; ++u) v[u] = b0 + u < b1 ? ws[(int64_t)(b0 + u) * E + ce] : 0;
#pragma unroll
      for (int u = 0; u < kColRegs; ++u) sum += v[u];
    } else {
      for (int b = b0; b < b1; b += kColRegs) {
        int w[kColRegs];
#pragma unroll
        for (int u = 0; u < kColRegs; ++u) w[u] = b + u < b1 ? ws[(int64_t)(b + u) * E + ce] : 0;
#pragma unroll
        for (int u = 0; u < kColRegs; ++u) sum += w[u];
      }
    }
    part_s[cg * E + ce] = sum;
  }
  // first invalid id per block (nblk <= kPlanThreads while blocks hold up to 32 chunks
  // per wave; larger counts loop)
  int mybad = INT_MAX;
  for (int b = tid; b < nblk; b += kPlanThreads) mybad = min(mybad, ws[ws_bad(s) + b]);
  __syncthreads();
  if (mybad != INT_MAX) atomicMin(&bad_s, mybad);
  int colbase = 0;   // the column thread's first base (blocks before b0)
  if (col_thread) {
    for (int g = 0; g < cg; ++g) colbase += part_s[g * E + ce];
    if (cg == tpc - 1) load_s[ce] = colbase + part_s[cg * E + ce];
  }
  if (wave == 0) colbase0_s[lane] = colbase;   // wave 1 writes wave 0's bases later
  __syncthreads();
  if (tid < R) {
    // home load of rank tid (independent LDS reads, unrolled)
    int hl = 0;
#pragma unroll 8
    for (int g = 0; g < E_loc; ++g) hl += load_s[tid * E_loc + g];
    hl_s[tid] = hl;
  }
  __syncthreads();

  if (bad_s != INT_MAX) {
    // an expert id outside [0, E): publish an empty plan that maps nothing
    for (int e = tid; e < E; e += kPlanThreads) {
      plan[s.o_load + e] = 0; plan[s.o_shed + e] = 0; plan[s.o_keep + e] = 0;
      plan[s.o_pfirst + e] = 0; plan[s.o_pnum + e] = 0; plan[s.o_home_row + e] = -1;
    }
    if (tid < H_WORDS) {
      int val = 0;
      switch (tid) {
        case H_MAGIC: val = (int32_t)kMagic; break;
        case H_STATUS: val = 1; break;
        case H_BADIDX: val = bad_s; break;
        case H_R: val = R; break;
        case H_E: val = E; break;
        case H_K: val = s.K; break;
        case H_S: val = s.S; break;
        case H_SLOTS: val = slots; break;
        case H_NVS: val = NvS; break;
        default: break;
      }
      hdr[tid] = val;
    }
    return;
  }

  // ---- shed: an overloaded home gives away its heaviest experts first -----------------
  if (tid < E) {                   // E <= kPlanThreads
    const int e = tid;
    const int h = e / E_loc;
    const int X = max(0, hl_s[h] - C);
    const int le = load_s[e];
    int sh = 0;
    if (X > 0) {
      int ahead = 0;   // load of the home's experts that come before e
#pragma unroll 8
      for (int e2 = h * E_loc; e2 < (h + 1) * E_loc; ++e2) {
        const int l2 = load_s[e2];
        if (before(l2, e2, le, e)) ahead += l2;
      }
      sh = clampi(X - ahead, 0, le);
    }
    shed_s[e] = sh;
    keep_s[e] = le - sh;
    pfirst_s[e] = 0;
    pnum_s[e] = 0;
  }
  __syncthreads();

  // per-block bases for the map kernel, written over the counts
  auto write_bases = [&]() {
    int run = colbase;
    if (in_regs) {
#pragma unroll
      for (int u = 0; u < kColRegs; ++u) {
        if (b0 + u < b1) {
          ws[(int64_t)(b0 + u) * E + ce] = run;
          run += v[u];
        }
      }
    } else {
      for (int b = b0; b < b1; b += kColRegs) {
        int w[kColRegs];
#pragma unroll
        for (int u = 0; u < kColRegs; ++u) w[u] = b + u < b1 ? ws[(int64_t)(b + u) * E + ce] : 0;
#pragma unroll
        for (int u = 0; u < kColRegs; ++u) {
          if (b + u < b1) {
            ws[(int64_t)(b + u) * E + ce] = run;
            run += w[u];
          }
        }
      }
    }
  };

  // ---- wave 0: order the shedding experts, then place them --------------------------------
  if (wave == 0) {
    // shedding experts in id order (ballot compaction), then ranked by (load desc, id asc)
    int n = 0;
    for (int e0 = 0; e0 < E; e0 += 64) {
      const int e = e0 + lane;
      const bool f = e < E && shed_s[e] > 0;
      const uint64_t m = __ballot(f);
      if (f) list_s[n + __popcll(m & lt)] = e;
      n += __popcll(m);
    }
    const int nshed = n;
    for (int t0 = 0; t0 < nshed; t0 += 64) {
      const int t = t0 + lane;
      if (t < nshed) {
        const int e = list_s[t];
        const int le = load_s[e];
        int rank = 0;
        for (int j = 0; j < nshed; ++j) {
          const int e2 = list_s[j];
          rank += before(load_s[e2], e2, le, e) ? 1 : 0;
        }
        order_s[rank] = e;
      }
    }

    // Placement, lane r = rank r.  For one expert, the lowest-id ranks that are short and
    // have a free slot are filled in id order until its shed count is used up (each piece
    // fills its receiver except possibly the last); any rest goes, again in id order, to
    // ranks that are short but have no free slot (fallback pieces).  This is the
    // one-assignment-at-a-time greedy, done one expert at a time.
    //
    // Fast path.  Without a slot budget the greedy simply cuts the shed stream (the
    // shedding experts' assignments laid end to end in plan order, positions [0, tot)) at
    // the boundaries of the ranks' deficit ranges (short ranks laid end to end in id
    // order): piece (q, r) is the overlap of expert q's range with rank r's.  Run in step
    // with the budgeted greedy, the two agree on every expert before the first one that
    // would give some rank its (slots+1)-th piece.  That prefix is placed by the cut, in
    // parallel over ranks, and the one-expert-at-a-time loop carries on from there.
    const int D0 = lane < R ? max(0, C - hl_s[lane]) : 0;
    const int dend = wave_incl_scan(D0);            // rank lane's deficit range [dbeg, dend)
    const int dbeg = dend - D0;
    const int dtot = lane63(dend);
    const uint64_t mD = __ballot(D0 > 0);
    const int posr = __popcll(mD & lt);             // short ranks before lane
    dend_s[lane] = dend;
    int32_t* sq_s = list_s;     // [nshed] first stream position of expert q (list_s is free)
    int32_t* qb_s = qbase_s;    // [nshed] piece index of expert q's first piece minus the
                                //   short-rank position of its first receiver
    int tot = 0;
    for (int q0 = 0; q0 < nshed; q0 += 64) {
      const int q = q0 + lane;
      const int sh = q < nshed ? shed_s[order_s[q]] : 0;
      const int incl = wave_incl_scan(sh);
      if (q < nshed) sq_s[q] = tot + incl - sh;
      tot += lane63(incl);
    }
    int np = 0;
    bool ok = tot <= dtot;      // always true when every rank's quota is S*K
    for (int q0 = 0; q0 < nshed && ok; q0 += 64) {
      const int q = q0 + lane;
      int n = 0, lo = 0;
      if (q < nshed) {
        const int x0 = sq_s[q];
        const int x1 = (q + 1 < nshed ? sq_s[q + 1] : tot) - 1;   // last position
        lo = count_le(dend_s, R, x0);               // receiving ranks: lo .. hi
        const int hi = count_le(dend_s, R, x1);
        const uint64_t upto = hi >= 63 ? ~0ull : ((2ull << hi) - 1);
        n = __popcll(mD & upto & ~((1ull << lo) - 1));
      }
      const int incl = wave_incl_scan(n);
      if (q < nshed) {
        const int e = order_s[q];
        pfirst_s[e] = np + incl - n;
        pnum_s[e] = n;
        qb_s[q] = np + incl - n - __popcll(mD & ((1ull << lo) - 1));
      }
      np += lane63(incl);
    }
    const bool gets = lane < R && D0 > 0 && dbeg < tot;
    const int hi_pos = min(dend, tot);
    const int qf = gets ? count_le(sq_s, nshed, dbeg) - 1 : 0;
    const int ql = gets ? count_le(sq_s, nshed, hi_pos - 1) - 1 : -1;
    // first expert that would overfill some rank's slots (nshed when none would)
    int qstar = gets && ql - qf + 1 > slots ? qf + slots : nshed;
    for (int d = 32; d >= 1; d >>= 1) qstar = min(qstar, __shfl_xor(qstar, d, 64));
    if (!ok || np > PM) qstar = 0;

    int D = D0, used = 0, fbrows = 0, nfb = 0, slotrows = 0;
    bool err = false;
    {
      const int qe = min(ql, qstar - 1);
      for (int q = qf; q <= qe; ++q) {     // this rank's pieces of the prefix, <= slots
        const int e = order_s[q];
        const int s0 = sq_s[q];
        const int s1 = q + 1 < nshed ? sq_s[q + 1] : tot;
        const int x = max(dbeg, s0);
        const int take = min(dend, s1) - x;
        const int p = qb_s[q] + posr;
        pe_s[p] = e; pr_s[p] = lane; psl_s[p] = q - qf; pc_s[p] = take;
        pst_s[p] = keep_s[e] + (x - s0); prel_s[p] = slotrows;
        slotrows += align_rows(take);
        used += 1;
      }
      const int send = qstar < nshed ? sq_s[qstar] : tot;   // end of the prefix's stream
      if (lane < R && D0 > 0 && dbeg < send) D -= min(dend, send) - dbeg;
      np = qstar == 0 ? 0 : (qstar < nshed ? pfirst_s[order_s[qstar]] : np);
    }
    // 64 experts at a time sit in lane registers; each iteration broadcasts its expert's
    // id, shed and keep counts with readlane, so the inner loop only stores to LDS
    for (int q0 = qstar; q0 < nshed; q0 += 64) {
     const int qq = q0 + lane;
     const int q_e = qq < nshed ? order_s[qq] : 0;
     const int q_shed = qq < nshed ? shed_s[q_e] : 0;
     const int q_keep = qq < nshed ? keep_s[q_e] : 0;
     // wait for these loads here: otherwise the loop below waits on every iteration, unable
     // to tell them from its own outstanding LDS stores (lgkmcnt(0); vmcnt, expcnt untouched)
     __builtin_amdgcn_s_waitcnt(0xC07F);
     const int qn = min(64, nshed - q0);
     for (int qi = 0; qi < qn; ++qi) {
      const int e = __builtin_amdgcn_readlane(q_e, qi);
      int rem = __builtin_amdgcn_readlane(q_shed, qi);
      int start = __builtin_amdgcn_readlane(q_keep, qi);
      const int first = np;
      {
        const bool elig = lane < R && D > 0 && used < slots;
        const int d = elig ? D : 0;
        const int incl = wave_incl_scan(d);
        const int excl = incl - d;
        const int take = clampi(rem - excl, 0, d);
        const uint64_t m = __ballot(take > 0);
        if (take > 0) {
          const int p = np + __popcll(m & lt);
          if (p < PM) {
            pe_s[p] = e; pr_s[p] = lane; psl_s[p] = used; pc_s[p] = take;
            pst_s[p] = start + excl; prel_s[p] = slotrows;
          } else {
            err = true;
          }
          used += 1;
          slotrows += align_rows(take);
          D -= take;
        }
        const int moved = min(rem, lane63(incl));
        np += __popcll(m);
        rem -= moved;
        start += moved;
      }
      if (rem > 0) {
        const int d = lane < R ? D : 0;
        const int incl = wave_incl_scan(d);
        const int excl = incl - d;
        const int take = clampi(rem - excl, 0, d);
        const uint64_t m = __ballot(take > 0);
        if (take > 0) {
          const int p = np + __popcll(m & lt);
          if (p < PM) {
            pe_s[p] = e; pr_s[p] = lane; psl_s[p] = -1; pc_s[p] = take;
            pst_s[p] = start + excl; prel_s[p] = fbrows;
          } else {
            err = true;
          }
          fbrows += take;
          nfb += 1;
          D -= take;
        }
        const int moved = min(rem, lane63(incl));
        np += __popcll(m);
        rem -= moved;
        start += moved;
      }
      if (lane == 0) {
        pfirst_s[e] = first;
        pnum_s[e] = np - first;
      }
      err = err || rem != 0;
     }
    }
    used_s[lane] = used;
    fb_s[lane] = fbrows;
    nfb_s[lane] = nfb;
    sr_s[lane] = slotrows;
    if (__ballot(err || (lane < R && D != 0))) { if (lane == 0) err_s = 1; }
    if (lane == 0) { npieces_s = min(np, PM); nshed_s = nshed; }
  } else {
    // the other waves are idle until the layout: they write the block bases now, wave 1
    // also wave 0's (its counts re-read, its first bases from colbase0_s), and wave 2
    // finds the largest expert load for the statistics
    if (col_thread) write_bases();
    if (wave == 1 && lane < tpc * E) {
      const int ce0 = lane % E, cg0 = lane / E;
      const int bb1 = min(cg0 * seg + seg, nblk);
      int run = colbase0_s[lane];
      for (int b = cg0 * seg; b < bb1; b += kColRegs) {
        int w[kColRegs];
#pragma unroll
        for (int u = 0; u < kColRegs; ++u) w[u] = b + u < bb1 ? ws[(int64_t)(b + u) * E + ce0] : 0;
#pragma unroll
        for (int u = 0; u < kColRegs; ++u) {
          if (b + u < bb1) {
            ws[(int64_t)(b + u) * E + ce0] = run;
            run += w[u];
          }
        }
      }
    }
    if (wave == 2) {
      int m = 0;
      for (int e = lane; e < E; e += 64) m = max(m, load_s[e]);
      m = lane63(wave_incl_max(m));
      if (lane == 0) maxload_s = m;
    }
  }
  __syncthreads();

  // ---- layout of each rank's buffer -----------------------------------------------------
  // Home groups, then slot groups (slot order = the order the rank's slot pieces were
  // created), then the fallback region; each home and slot group starts on a multiple of
  // ROW_ALIGN rows.  Slot and fallback rows were fixed relative to their regions while
  // placing.  Home offsets: one exclusive scan over all experts (thread = expert), minus
  // the scan's value at the rank's first expert.
  const int np = npieces_s;
  int32_t* off = plan + s.o_off;
  int32_t* slot_expert = plan + s.o_slot_expert;
  {
    const int e = tid;
    const int a = e < E ? align_rows(keep_s[e]) : 0;
    const int incl = wave_incl_scan(a);
    if (lane == 63) wtot_s[wave] = incl;
    __syncthreads();
    int pre = 0;
    for (int v = 0; v < wave; ++v) pre += wtot_s[v];
    const int X = pre + incl - a;           // exclusive scan over experts
    const int r = e / E_loc, g = e - r * E_loc;
    if (e < E && g == 0) xs_s[r] = X;
    __syncthreads();
    if (e < E) {
      const int o_in = X - xs_s[r];
      off[(int64_t)r * (G + 1) + g] = o_in;
      home_s[e] = r * NvS + o_in;
      if (g == E_loc - 1) {
        const int ht = o_in + a;
        ht_s[r] = ht;
        off[(int64_t)r * (G + 1) + G] = ht + sr_s[r];
        if (ht + sr_s[r] + fb_s[r] > NvS) err_s = 1;
      }
    }
  }
  __syncthreads();

  // ---- write the plan ---------------------------------------------------------------------
  for (int p = tid; p < np; p += kPlanThreads) {
    const int r = pr_s[p], sl = psl_s[p], rel = prel_s[p];
    const int rowin = ht_s[r] + (sl >= 0 ? rel : sr_s[r] + rel);   // row inside rank r
    const int row0 = r * NvS + rowin;
    if (sl >= 0) {
      off[(int64_t)r * (G + 1) + E_loc + sl] = rowin;
      slot_expert[r * slots + sl] = pe_s[p];
    }
    int32_t* pc = plan + s.o_pieces + (int64_t)p * kPieceInts;
    pc[P_E] = pe_s[p]; pc[P_R] = r; pc[P_SLOT] = sl; pc[P_CNT] = pc_s[p];
    pc[P_START] = pst_s[p]; pc[P_FBPOS] = sl >= 0 ? 0 : rel; pc[P_ROW0] = row0; pc[7] = 0;
    // packed (start, count, first row) for the map kernel
    reinterpret_cast<i32x4*>(plan + s.o_ptab)[p] = i32x4{pst_s[p], pc_s[p], row0, 0};
  }
  for (int i = tid; i < R * slots; i += kPlanThreads) {   // unused slots
    const int r = i / slots, sl = i - r * slots;
    if (sl >= used_s[r]) {
      off[(int64_t)r * (G + 1) + E_loc + sl] = ht_s[r] + sr_s[r];
      slot_expert[i] = -1;
    }
  }
  for (int e = tid; e < E; e += kPlanThreads) {
    plan[s.o_load + e] = load_s[e];
    plan[s.o_shed + e] = shed_s[e];
    plan[s.o_keep + e] = keep_s[e];
    plan[s.o_home_row + e] = home_s[e];
    plan[s.o_pfirst + e] = pfirst_s[e];
    plan[s.o_pnum + e] = pnum_s[e];
    // packed (keep, home row, first piece, piece count) for the map kernel
    reinterpret_cast<i32x4*>(plan + s.o_xtab)[e] =
        i32x4{keep_s[e], home_s[e], pfirst_s[e], pnum_s[e]};
  }
  if (wave == 0) {
    // experts with slot replicas, in plan order (the reduce work list)
    const int nshed = nshed_s;
    int n = 0;
    for (int q0 = 0; q0 < nshed; q0 += 64) {
      const int q = q0 + lane;
      bool has = false;
      int e = 0;
      if (q < nshed) {
        e = order_s[q];
        has = pnum_s[e] > 0 && psl_s[pfirst_s[e]] >= 0;
      }
      const uint64_t m = __ballot(has);
      if (has) plan[s.o_red + n + __popcll(m & lt)] = e;
      n += __popcll(m);
    }
    // statistics over ranks (lane r)
    const int nrep = lane63(wave_incl_scan(used_s[lane]));
    const int nfb = lane63(wave_incl_scan(nfb_s[lane]));
    const int ppr = lane63(wave_incl_max(used_s[lane] + nfb_s[lane]));
    const bool err = err_s != 0;
    int val = 0;
    switch (lane) {
      case H_MAGIC: val = (int32_t)kMagic; break;
      case H_STATUS: val = err ? 2 : 0; break;
      case H_NPIECES: val = np; break;
      case H_NREPLICAS: val = nrep; break;
      case H_NFALLBACK: val = nfb; break;
      case H_MAXPPR: val = ppr; break;
      case H_NRED: val = err ? 0 : n; break;
      case H_BADIDX: val = -1; break;
      case H_NSHED: val = nshed; break;
      case H_MAXLOAD: val = maxload_s; break;
      case H_R: val = R; break;
      case H_E: val = E; break;
      case H_K: val = s.K; break;
      case H_S: val = s.S; break;
      case H_SLOTS: val = slots; break;
      case H_NVS: val = NvS; break;
      default: break;
    }
    hdr[lane] = val;   // H_WORDS == 64: one word per lane
  }
}

// ---------------------------------------------------------------------------------------
// 1+2. histogram and planner in one launch
// ---------------------------------------------------------------------------------------
// Each workgroup of kPlanThreads holds two logical histogram blocks (waves 0-7 and 8-15;
// the block and wave numbering the map kernel reads is unchanged).  A workgroup that has
// written its counts makes them visible device-wide, then counts itself in an arrival
// word; the workgroup that arrives last sees every count and runs the planner.  Nothing
// waits on another workgroup, so no residency assumption is made, and the kernel
// boundary between histogram and planner (3.3 us at DeepSeek-V3 shape, device
// timestamps) disappears.  The arrival word is word 0 of `ctl`; the last workgroup
// returns it to zero, so it is zero at every call as long as the workspace was zero
// before its first use.
// A device-scope fence on gfx950 writes back and invalidates the XCD's whole L2, so only
// one wave per workgroup fences, after every wave has waited for its own stores: with
// every wave fencing the kernel took 37.7 us instead of 16.7 us (rocprofv3, DeepSeek-V3
// shape; the two kernels it replaces took 3.7 + 12.2 us plus the boundary).
template <int M>
__global__ __launch_bounds__(kPlanThreads) void hist_plan_kernel(const int32_t* __restrict__ ids,
                                                                 int32_t* __restrict__ plan,
                                                                 int32_t* __restrict__ ctl,
                                                                 int32_t* __restrict__ ws,
                                                                 const moonep_sizes s) {
  extern __shared__ int32_t lds[];
  __shared__ int bad2[2];
  __shared__ int last;
  const int half = (int)threadIdx.x / kMapThreads;
  hist_block<M>(ids, ws, s, (int)blockIdx.x * 2 + half, (int)threadIdx.x - half * kMapThreads,
                lds + half * kMapWaves * s.E, &bad2[half]);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's stores have reached the L2
  __syncthreads();                    // ... and every other wave's
  if (threadIdx.x == 0) {
    __threadfence();                  // one wave releases them device-wide
    last = atomicAdd(&ctl[0], 1) == (int)gridDim.x - 1;
  }
  __syncthreads();
  if (!last) return;
  if (threadIdx.x == 0) {
    __threadfence();                  // and, in the last workgroup, acquires the others'
    atomicExch(&ctl[0], 0);
  }
  __syncthreads();
  planner_block(plan, ws, s, lds);
}

// ---------------------------------------------------------------------------------------
// 3. token -> row map
// ---------------------------------------------------------------------------------------

// One single-wave workgroup per map sub-block of 64*M assignments: part q of wave w of
// block b in the histogram's numbering (a histogram wave with more than kMapChunks chunks
// is split into Q parts).  Every global load it needs is issued first: ids, weights, the
// per-expert tables, the sub-block's base per expert (block base from the planner +
// earlier waves of the block + the wave's own earlier parts, both from the histogram),
// the piece table.
constexpr int kTab = 8;   // table entries per lane loaded per round trip

template <int M> struct MapGroup { static constexpr int value = M < 8 ? M : 8; };

template <int M>
__global__ __launch_bounds__(64) void map_kernel(const int32_t* __restrict__ ids,
                                                 const float* __restrict__ w,
                                                 int32_t* __restrict__ plan,
                                                 const int32_t* __restrict__ ws,
                                                 const moonep_sizes s) {
  extern __shared__ i32x4 lds4[];
  const int E = s.E;
  const int P = s.P_max;
  i32x4* xtab_s = lds4;                            // [E] keep, home row, first piece, count
  i32x4* ptab_s = xtab_s + E;                      // [P] start, count, first row
  int32_t* run = reinterpret_cast<int32_t*>(ptab_s + P);   // [E] running count per expert
  uint64_t* mask_s = reinterpret_cast<uint64_t*>(run + ((E + 1) & ~1));   // [E+1] lanes per id

  constexpr int kMapGroup = MapGroup<M>::value;   // chunks ranked per pass
  const int lane = threadIdx.x;
  const int Q = map_split(s);                     // map sub-blocks per histogram wave
  const int per_blk = kMapWaves * Q;
  const int b = blockIdx.x / per_blk, sb = blockIdx.x % per_blk;
  const int sw = sb / Q, q = sb - sw * Q;         // histogram wave, part of it
  const int64_t A = s.A;
  const int64_t i_wave = (int64_t)b * s.blk + (int64_t)sb * (64 * M);
  int32_t* dst = plan + s.o_dst_row;
  float* wout = reinterpret_cast<float*>(plan + s.o_w);
  if (i_wave >= A) return;

  // every load is issued before the first wait: status, ids, weights, expert tables and
  // this sub-block's bases, piece table (P_max entries, whatever the piece count)
  const int status = plan[s.o_hdr + H_STATUS];
  int idv[M];
  float wt[M];
#pragma unroll
  for (int c = 0; c < M; ++c) {
    const int64_t i = i_wave + c * 64 + lane;
    idv[c] = i < A ? ids[i] : E;    // E marks lanes past the end
    wt[c] = i < A ? w[i] : 0.f;
  }
  const i32x4* xtab = reinterpret_cast<const i32x4*>(plan + s.o_xtab);
  const i32x4* ptab = reinterpret_cast<const i32x4*>(plan + s.o_ptab);
  const int32_t* bbase = ws + (int64_t)b * E;
  const int32_t* wbase = ws + ws_sub(s) + ((int64_t)b * kMapWaves + sw) * E;
  // running count of the histogram wave before this part (none for its first part: the
  // pointer then stays valid and the value is multiplied by 0)
  const int32_t* qbase = q > 0 ? ws + ws_snap(s) + (((int64_t)b * kMapWaves + sw) * (Q - 1) + q - 1) * E
                               : wbase;
  const int qon = q > 0 ? 1 : 0;
  // loads use clamped (always valid) indices so that they stay unconditional and the
  // values stay in registers; only the LDS stores are guarded
  for (int e0 = 0; e0 < E || e0 < P; e0 += 64 * kTab) {
    i32x4 xt[kTab], pt[kTab];
    int bb[kTab], wb[kTab], qb[kTab];
#pragma unroll
    for (int k = 0; k < kTab; ++k) {
      const int e = e0 + k * 64 + lane;
      const int ec = min(e, E - 1), pc = min(e, P - 1);
      xt[k] = xtab[ec];
      bb[k] = bbase[ec];
      wb[k] = wbase[ec];
      qb[k] = qbase[ec];
      pt[k] = ptab[pc];
    }
#pragma unroll
    for (int k = 0; k < kTab; ++k) {
      const int e = e0 + k * 64 + lane;
      if (e < E) { xtab_s[e] = xt[k]; run[e] = bb[k] + wb[k] + qon * qb[k]; }
      if (e < P) ptab_s[e] = pt[k];
    }
  }
  for (int e = lane; e <= E; e += 64) mask_s[e] = 0;
  if (status != 0) {
    // invalid plan: map nothing
#pragma unroll
    for (int c = 0; c < M; ++c) {
      const int64_t i = i_wave + c * 64 + lane;
      if (i < A) { dst[i] = -1; wout[i] = 0.f; }
    }
    return;
  }
  // One wave: its LDS accesses are performed in program order, so no barrier is needed.
  //
  // Stable rank of each assignment among its expert's assignments, chunk by chunk (64
  // assignments, lane order = i order).  Peers (lanes of the chunk with the same id): each
  // lane ORs its bit into mask[id], reads mask[id] back, and clears it, three LDS
  // operations that take effect in that order for the whole wave, so the read sees exactly
  // the chunk's lanes and the next chunk starts from zeros.  `below` = peers in lower
  // lanes; the group's lowest lane adds the group size to the expert's LDS counter and
  // gets the count of all earlier chunks back (atomics of one wave are applied in issue
  // order, so they are issued back to back without waiting), then hands it to its peers
  // with a lane shuffle.
  const uint64_t lt = lanemask_lt();
  const uint64_t mybit = 1ull << lane;
  for (int c0 = 0; c0 < M; c0 += kMapGroup) {
    uint64_t peers[kMapGroup];
#pragma unroll
    for (int u = 0; u < kMapGroup; ++u) {
      // lanes past the end share the spare slot E
      uint64_t* m = mask_s + min((unsigned)idv[c0 + u], (unsigned)E);
      __hip_atomic_fetch_or(m, mybit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      peers[u] = __hip_atomic_load(m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      __hip_atomic_store(m, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    int below[kMapGroup], base[kMapGroup];
#pragma unroll
    for (int u = 0; u < kMapGroup; ++u) {
      const int id = idv[c0 + u];
      below[u] = __popcll(peers[u] & lt);
      base[u] = 0;
      if (below[u] == 0 && (unsigned)id < (unsigned)E)
        base[u] = atomicAdd(&run[id], __popcll(peers[u]));
    }
    int j[kMapGroup];
    i32x4 xt[kMapGroup];
#pragma unroll
    for (int u = 0; u < kMapGroup; ++u) {
      j[u] = __shfl(base[u], __builtin_ctzll(peers[u]), 64) + below[u];
      xt[u] = xtab_s[min((unsigned)idv[c0 + u], (unsigned)(E - 1))];   // keep, home row, pieces
    }
#pragma unroll
    for (int u = 0; u < kMapGroup; ++u) {
      const int c = c0 + u;
      const int id = idv[c];
      const int64_t i = i_wave + c * 64 + lane;
      if ((unsigned)id < (unsigned)E) {
        int row = -1;
        if (j[u] < xt[u].x) {
          row = xt[u].y + j[u];
        } else {
          // the expert's pieces cover [keep, load) in order: j falls in the last piece
          // whose start is <= j.  Eight starts are read per LDS round trip.
          // clamped to the piece table: a plan the planner did not write can hold anything
          const int pf = min(max(xt[u].z, 0), P), pn = min(max(xt[u].w, 0), P - pf);
          const int32_t* pstart = reinterpret_cast<const int32_t*>(ptab_s + pf);
          int n_le = 0;
          for (int p0 = 0; p0 < pn; p0 += 8) {
            int st[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) st[k] = pstart[4 * min(p0 + k, pn - 1)];
#pragma unroll
            for (int k = 0; k < 8; ++k) n_le += (p0 + k < pn && st[k] <= j[u]) ? 1 : 0;
          }
          if (n_le > 0) {
            const i32x4 pt = ptab_s[pf + n_le - 1];   // start, count, first row
            if (j[u] < pt.x + pt.y) row = pt.z + (j[u] - pt.x);
          }
        }
        dst[i] = row;
        wout[i] = wt[c];
      }
    }
  }
}

template <int M>
hipError_t launch_map(const moonep_sizes& s, const int32_t* ids, const float* w, int32_t* plan,
                      const int32_t* ws, hipStream_t st) {
  const size_t lds = (size_t)16 * (s.E + s.P_max) + 4 * ((s.E + 1) & ~1) + 8 * (s.E + 1);
  hipLaunchKernelGGL(map_kernel<M>, dim3(s.nblk * kMapWaves * map_split(s)), dim3(64), lds, st,
                     ids, w, plan, ws, s);
  return hipGetLastError();
}

template <int M>
hipError_t launch_hist_plan(const moonep_sizes& s, const int32_t* ids, int32_t* plan, int32_t* ctl,
                            int32_t* ws, hipStream_t st) {
  const size_t hist_lds = (size_t)2 * kMapWaves * s.E * sizeof(int32_t);
  const size_t plan_lds = (size_t)(7 * s.E + max(kPlanThreads, 7 * s.P_max)) * sizeof(int32_t);
  hipLaunchKernelGGL(hist_plan_kernel<M>, dim3((unsigned)((s.nblk + 1) / 2)), dim3(kPlanThreads),
                     hist_lds > plan_lds ? hist_lds : plan_lds, st, ids, plan, ctl, ws, s);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_plan(const moonep_sizes& s, const int32_t* ids, const float* w,
                       int32_t* plan, int32_t* ws, hipStream_t st) {
  // workspace: kWsCtl control words (the arrival word first), then the per-block arrays
  int32_t* ctl = ws;
  int32_t* body = ws + kWsCtl;
  hipError_t err;
  switch (s.blk / kMapThreads) {
    case 1: err = launch_hist_plan<1>(s, ids, plan, ctl, body, st); break;
    case 2: err = launch_hist_plan<2>(s, ids, plan, ctl, body, st); break;
    case 4: err = launch_hist_plan<4>(s, ids, plan, ctl, body, st); break;
    case 8: err = launch_hist_plan<8>(s, ids, plan, ctl, body, st); break;
    case 16: err = launch_hist_plan<16>(s, ids, plan, ctl, body, st); break;
    case 32: err = launch_hist_plan<32>(s, ids, plan, ctl, body, st); break;
    default: return hipErrorInvalidValue;
  }
  if (err != hipSuccess) return err;
  switch (map_chunks(s)) {
    case 1: return launch_map<1>(s, ids, w, plan, body, st);
    case 2: return launch_map<2>(s, ids, w, plan, body, st);
    case 4: return launch_map<4>(s, ids, w, plan, body, st);
    case 8: return launch_map<8>(s, ids, w, plan, body, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace moonep
