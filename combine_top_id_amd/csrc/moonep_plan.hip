// Planning on the GPU: live top-K router output -> replica plan + token->row map.
//
// "Moonshot AI Open-Sources MoonEP" (tldrocket.com), paragraph 3: every rank receives
// exactly S*K assignments because a few overloaded experts are duplicated, planned
// directly from live router output; paragraph 5: E/R prefetch slots in training, 3-4 in
// inference with remote-read fallback.  "MoonshotAI/MoonEP 딥다이브" (fiv.co.kr),
// section 4, pattern 1: the plan is computed once and reused; pattern 2: static S*K
// plus alignment padding buffers.
//
// Three launches on the caller's stream:
//   1. hist_kernel     one workgroup per block of `blk` assignments: LDS histogram of
//                      expert ids -> per-block counts, first invalid id per block.
//   2. planner_kernel  one workgroup: expert loads, per-rank excess and deficit,
//                      shedding, greedy placement (one wave, one lane per rank),
//                      buffer layout, piece rows, statistics.
//   3. map_kernel      one workgroup per block: the stable rank j of every assignment
//                      among its expert's assignments (wave64 ballot peer masks plus
//                      per-wave LDS counters and block prefixes), then its row;
//                      also copies the top-K weights into the plan.
#include <climits>

#include "moonep_internal.h"

namespace moonep {
namespace {

__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int l = lane_id();
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int l = lane_id();
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int t = __shfl_up(v, d, 64);
    if (l >= d) v += t;
  }
  return v;
}

__device__ __forceinline__ int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

// ---------------------------------------------------------------------------------------
// 1. per-block histogram
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(kMapThreads) void hist_kernel(const int32_t* __restrict__ ids,
                                                           int32_t* __restrict__ ws,
                                                           const moonep_sizes s) {
  extern __shared__ int32_t lds[];
  __shared__ int bad;
  const int E = s.E;
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += kMapThreads) lds[e] = 0;
  if (tid == 0) bad = INT_MAX;
  __syncthreads();
  const int64_t i0 = (int64_t)blockIdx.x * s.blk;
  const int64_t i1 = min(i0 + (int64_t)s.blk, s.A);
  int mybad = INT_MAX;
  for (int64_t i = i0 + tid; i < i1; i += kMapThreads) {
    const int id = ids[i];
    if ((unsigned)id < (unsigned)E)
      atomicAdd(&lds[id], 1);
    else
      mybad = min(mybad, (int)i);
  }
  if (mybad != INT_MAX) atomicMin(&bad, mybad);
  __syncthreads();
  int32_t* cnt = ws + (int64_t)blockIdx.x * E;
  for (int e = tid; e < E; e += kMapThreads) cnt[e] = lds[e];
  if (tid == 0) ws[ws_bad(s) + blockIdx.x] = bad;
}

// ---------------------------------------------------------------------------------------
// 2. the planner (one workgroup of kPlanThreads)
// ---------------------------------------------------------------------------------------

// Does expert a come before expert b in (load descending, id ascending) order?
__device__ __forceinline__ bool before(int la, int a, int lb, int b) {
  return la > lb || (la == lb && a < b);
}

__global__ __launch_bounds__(kPlanThreads) void planner_kernel(int32_t* __restrict__ plan,
                                                               int32_t* __restrict__ ws,
                                                               const moonep_sizes s) {
  extern __shared__ int32_t lds[];
  const int E = s.E, R = s.R, E_loc = s.E_loc, C = s.C, slots = s.slots, G = s.G;
  const int NvS = s.NvS;
  int32_t* load_s = lds;            // [E]
  int32_t* shed_s = load_s + E;     // [E]
  int32_t* keep_s = shed_s + E;     // [E]
  int32_t* order_s = keep_s + E;    // [E] shedding experts, plan order
  int32_t* pfirst_s = order_s + E;  // [E]
  int32_t* pnum_s = pfirst_s + E;   // [E]
  __shared__ int32_t X_s[64], D_s[64], used_s[64], fb_s[64], nfb_s[64];
  __shared__ int bad_s, nshed_s, npieces_s, maxload_s, err_s, nred_s;

  int32_t* hdr = plan + s.o_hdr;
  int32_t* pieces = plan + s.o_pieces;
  int32_t* slot_expert = plan + s.o_slot_expert;
  int32_t* off = plan + s.o_off;
  int32_t* home_row = plan + s.o_home_row;
  int32_t* slot_cnt = ws + ws_slotcnt(s);
  const int tid = threadIdx.x;

  // ---- expert loads: column sums of the per-block counts --------------------------------
  for (int e = tid; e < E; e += kPlanThreads) load_s[e] = 0;
  if (tid == 0) { bad_s = INT_MAX; nshed_s = 0; maxload_s = 0; err_s = 0; }
  __syncthreads();
  {
    const int64_t n = (int64_t)s.nblk * E;
    for (int64_t f = tid; f < n; f += kPlanThreads) {
      const int v = ws[f];
      if (v) atomicAdd(&load_s[(int)(f % E)], v);
    }
    for (int b = tid; b < s.nblk; b += kPlanThreads) atomicMin(&bad_s, ws[ws_bad(s) + b]);
  }
  __syncthreads();

  if (bad_s != INT_MAX) {
    // an expert id outside [0, E): publish an empty plan that maps nothing
    for (int e = tid; e < E; e += kPlanThreads) {
      plan[s.o_load + e] = 0; plan[s.o_shed + e] = 0; plan[s.o_keep + e] = 0;
      plan[s.o_pfirst + e] = 0; plan[s.o_pnum + e] = 0; home_row[e] = -1;
    }
    if (tid < H_WORDS) hdr[tid] = 0;
    __syncthreads();
    if (tid == 0) {
      hdr[H_MAGIC] = (int32_t)kMagic; hdr[H_STATUS] = 1; hdr[H_BADIDX] = bad_s;
      hdr[H_R] = R; hdr[H_E] = E; hdr[H_K] = s.K; hdr[H_S] = s.S; hdr[H_SLOTS] = slots;
      hdr[H_NVS] = NvS;
    }
    return;
  }

  // ---- home loads, excess and deficit per rank --------------------------------------------
  if (tid < 64) {
    int hl = 0;
    if (tid < R)
      for (int g = 0; g < E_loc; ++g) hl += load_s[tid * E_loc + g];
    X_s[tid] = tid < R ? max(0, hl - C) : 0;
    D_s[tid] = tid < R ? max(0, C - hl) : 0;
    used_s[tid] = 0; fb_s[tid] = 0; nfb_s[tid] = 0;
  }
  for (int e = tid; e < E; e += kPlanThreads) atomicMax(&maxload_s, load_s[e]);
  __syncthreads();

  // ---- shed: an overloaded home gives away its heaviest experts first -----------------
  for (int e = tid; e < E; e += kPlanThreads) {
    const int h = e / E_loc;
    const int X = X_s[h];
    const int le = load_s[e];
    int sh = 0;
    if (X > 0) {
      int ahead = 0;   // load of the home's experts that come before e
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

  // ---- shedding experts in (load desc, id asc) order ---------------------------------------
  for (int e = tid; e < E; e += kPlanThreads) {
    if (shed_s[e] > 0) {
      const int le = load_s[e];
      int pos = 0;
      for (int e2 = 0; e2 < E; ++e2)
        if (shed_s[e2] > 0 && before(load_s[e2], e2, le, e)) ++pos;
      order_s[pos] = e;
      atomicAdd(&nshed_s, 1);
    }
  }
  __syncthreads();

  // ---- placement: one wave, lane r holds rank r ------------------------------------------
  // For one expert, the lowest-id ranks that are short and have a free slot are filled in
  // id order until the expert's shed count is used up (each piece fills its receiver
  // except possibly the last); any rest goes, again in id order, to ranks that are short
  // but have no free slot (fallback pieces).  This is the one-assignment-at-a-time greedy
  // done one expert at a time.
  if (tid < 64) {
    const int lane = tid;
    int D = D_s[lane];
    int used = 0, fbrows = 0, nfb = 0;
    int np = 0;
    const int nshed = nshed_s;
    const uint64_t lt = lanemask_lt();
    for (int q = 0; q < nshed; ++q) {
      const int e = order_s[q];
      int rem = shed_s[e];
      int start = keep_s[e];
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
          int32_t* pc = pieces + (int64_t)min(p, s.P_max - 1) * kPieceInts;
          if (p >= s.P_max) err_s = 1;
          pc[P_E] = e; pc[P_R] = lane; pc[P_SLOT] = used; pc[P_CNT] = take;
          pc[P_START] = start + excl; pc[P_FBPOS] = 0;
          slot_expert[lane * slots + used] = e;
          slot_cnt[lane * slots + used] = take;
          used += 1;
          D -= take;
        }
        const int moved = min(rem, __shfl(incl, 63, 64));
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
          int32_t* pc = pieces + (int64_t)min(p, s.P_max - 1) * kPieceInts;
          if (p >= s.P_max) err_s = 1;
          pc[P_E] = e; pc[P_R] = lane; pc[P_SLOT] = -1; pc[P_CNT] = take;
          pc[P_START] = start + excl; pc[P_FBPOS] = fbrows;
          fbrows += take;
          nfb += 1;
          D -= take;
        }
        const int moved = min(rem, __shfl(incl, 63, 64));
        np += __popcll(m);
        rem -= moved;
        start += moved;
      }
      if (lane == 0) {
        pfirst_s[e] = first;
        pnum_s[e] = np - first;
        if (rem != 0) err_s = 1;
      }
    }
    used_s[lane] = used;
    fb_s[lane] = fbrows;
    nfb_s[lane] = nfb;
    if (lane < R && D != 0) err_s = 1;
    if (lane == 0) npieces_s = min(np, s.P_max);
  }
  __syncthreads();

  // ---- layout of each rank's buffer: home groups, slot groups, fallback region -----------
  if (tid < R) {
    const int r = tid;
    int32_t* o = off + (int64_t)r * (G + 1);
    int pos = 0;
    for (int g = 0; g < E_loc; ++g) {
      const int e = r * E_loc + g;
      o[g] = pos;
      home_row[e] = r * NvS + pos;
      pos = (pos + keep_s[e] + kRowAlign - 1) / kRowAlign * kRowAlign;
    }
    const int u = used_s[r];
    for (int sl = 0; sl < slots; ++sl) {
      o[E_loc + sl] = pos;
      int size = 0;
      if (sl < u) size = slot_cnt[r * slots + sl];
      else slot_expert[r * slots + sl] = -1;
      pos = (pos + size + kRowAlign - 1) / kRowAlign * kRowAlign;
    }
    o[G] = pos;
    if (pos + fb_s[r] > NvS) err_s = 1;
  }
  __syncthreads();

  // ---- first row of every piece; per-expert tables -----------------------------------------
  const int np = npieces_s;
  for (int p = tid; p < np; p += kPlanThreads) {
    int32_t* pc = pieces + (int64_t)p * kPieceInts;
    const int r = pc[P_R], slot = pc[P_SLOT];
    const int32_t* o = off + (int64_t)r * (G + 1);
    pc[P_ROW0] = r * NvS + (slot >= 0 ? o[E_loc + slot] : o[G] + pc[P_FBPOS]);
    pc[7] = 0;
  }
  for (int e = tid; e < E; e += kPlanThreads) {
    plan[s.o_load + e] = load_s[e];
    plan[s.o_shed + e] = shed_s[e];
    plan[s.o_keep + e] = keep_s[e];
    plan[s.o_pfirst + e] = pfirst_s[e];
    plan[s.o_pnum + e] = pnum_s[e];
  }
  // experts with slot replicas, in plan order (the reduce work list)
  if (tid < 64) {
    const int lane = tid;
    const uint64_t lt = lanemask_lt();
    int n = 0;
    const int nshed = nshed_s;
    for (int q0 = 0; q0 < nshed; q0 += 64) {
      const int q = q0 + lane;
      bool has = false;
      int e = 0;
      if (q < nshed) {
        e = order_s[q];
        has = pnum_s[e] > 0 && pieces[(int64_t)pfirst_s[e] * kPieceInts + P_SLOT] >= 0;
      }
      const uint64_t m = __ballot(has);
      if (has) plan[s.o_red + n + __popcll(m & lt)] = e;
      n += __popcll(m);
    }
    if (lane == 0) nred_s = n;
  }
  __syncthreads();

  if (tid == 0) {
    int nrep = 0, nfb = 0, maxppr = 0;
    for (int r = 0; r < R; ++r) {
      nrep += used_s[r];
      nfb += nfb_s[r];
      maxppr = max(maxppr, used_s[r] + nfb_s[r]);
    }
    for (int w = 0; w < H_WORDS; ++w) hdr[w] = 0;
    hdr[H_MAGIC] = (int32_t)kMagic;
    hdr[H_STATUS] = err_s ? 2 : 0;
    hdr[H_NPIECES] = np;
    hdr[H_NREPLICAS] = nrep;
    hdr[H_NFALLBACK] = nfb;
    hdr[H_MAXPPR] = maxppr;
    hdr[H_NRED] = err_s ? 0 : nred_s;
    hdr[H_BADIDX] = -1;
    hdr[H_NSHED] = nshed_s;
    hdr[H_MAXLOAD] = maxload_s;
    hdr[H_R] = R; hdr[H_E] = E; hdr[H_K] = s.K; hdr[H_S] = s.S; hdr[H_SLOTS] = slots;
    hdr[H_NVS] = NvS;
  }
}

// ---------------------------------------------------------------------------------------
// 3. token -> row map
// ---------------------------------------------------------------------------------------

// M = chunks of 64 assignments per wave; a block is kMapThreads * M assignments.
template <int M>
__global__ __launch_bounds__(kMapThreads) void map_kernel(const int32_t* __restrict__ ids,
                                                          const float* __restrict__ w,
                                                          int32_t* __restrict__ plan,
                                                          const int32_t* __restrict__ ws,
                                                          const moonep_sizes s) {
  extern __shared__ int32_t lds[];
  const int E = s.E;
  const int P = s.P_max;
  int32_t* run = lds;                       // [kMapWaves][E]
  int32_t* keep_s = run + kMapWaves * E;    // [E]
  int32_t* home_s = keep_s + E;             // [E]
  int32_t* pfirst_s = home_s + E;           // [E]
  int32_t* pnum_s = pfirst_s + E;           // [E]
  int32_t* pstart_s = pnum_s + E;           // [P]
  int32_t* pcnt_s = pstart_s + P;           // [P]
  int32_t* prow_s = pcnt_s + P;             // [P]

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int64_t A = s.A;
  const int64_t i_wave = (int64_t)blockIdx.x * s.blk + (int64_t)wave * (64 * M);
  int32_t* dst = plan + s.o_dst_row;
  float* wout = reinterpret_cast<float*>(plan + s.o_w);

  if (plan[s.o_hdr + H_STATUS] != 0) {
    // invalid plan: map nothing
#pragma unroll
    for (int c = 0; c < M; ++c) {
      const int64_t i = i_wave + c * 64 + lane;
      if (i < A) { dst[i] = -1; wout[i] = 0.f; }
    }
    return;
  }

  int idv[M];
  float wv[M];
#pragma unroll
  for (int c = 0; c < M; ++c) {
    const int64_t i = i_wave + c * 64 + lane;
    idv[c] = i < A ? ids[i] : E;    // E marks lanes past the end
    wv[c] = i < A ? w[i] : 0.f;
  }

  for (int e = lane; e < E; e += 64) run[wave * E + e] = 0;
  for (int e = tid; e < E; e += kMapThreads) {
    keep_s[e] = plan[s.o_keep + e];
    home_s[e] = plan[s.o_home_row + e];
    pfirst_s[e] = plan[s.o_pfirst + e];
    pnum_s[e] = plan[s.o_pnum + e];
  }
  const int np = plan[s.o_hdr + H_NPIECES];
  for (int p = tid; p < np; p += kMapThreads) {
    const int32_t* pc = plan + s.o_pieces + (int64_t)p * kPieceInts;
    pstart_s[p] = pc[P_START];
    pcnt_s[p] = pc[P_CNT];
    prow_s[p] = pc[P_ROW0];
  }
  // the wave's own counters are zeroed by the wave itself; LDS is in order per wave
  const int nbits = 32 - __clz(E);
  const uint64_t lt = lanemask_lt();
  int loc[M];
  int32_t* myrun = run + wave * E;
#pragma unroll
  for (int c = 0; c < M; ++c) {
    const int id = idv[c];
    uint64_t peers = ~0ull;
    for (int bit = 0; bit < nbits; ++bit) {
      const bool on = (id >> bit) & 1;
      const uint64_t bl = __ballot(on);
      peers &= on ? bl : ~bl;
    }
    const int below = __popcll(peers & lt);
    int base = 0;
    if (id < E) base = myrun[id];
    loc[c] = base + below;
    if (below == 0 && id < E) myrun[id] = base + __popcll(peers);
  }
  __syncthreads();

  // per expert: block prefix (earlier blocks) + earlier waves of this block
  for (int e = tid; e < E; e += kMapThreads) {
    int acc = 0;
    const int nb = blockIdx.x;
    int b = 0;
    for (; b + 4 <= nb; b += 4) {
      const int c0 = ws[(int64_t)(b + 0) * E + e];
      const int c1 = ws[(int64_t)(b + 1) * E + e];
      const int c2 = ws[(int64_t)(b + 2) * E + e];
      const int c3 = ws[(int64_t)(b + 3) * E + e];
      acc += c0 + c1 + c2 + c3;
    }
    for (; b < nb; ++b) acc += ws[(int64_t)b * E + e];
#pragma unroll
    for (int v = 0; v < kMapWaves; ++v) {
      const int c = run[v * E + e];
      run[v * E + e] = acc;
      acc += c;
    }
  }
  __syncthreads();

#pragma unroll
  for (int c = 0; c < M; ++c) {
    const int64_t i = i_wave + c * 64 + lane;
    if (i < A) {
      const int id = idv[c];
      int row = -1;
      if ((unsigned)id >= (unsigned)E) {
        // cannot happen for ids the histogram saw; never index with it
      } else if (const int j = myrun[id] + loc[c]; j < keep_s[id]) {
        row = home_s[id] + j;
      } else {
        const int q1 = pfirst_s[id] + pnum_s[id];
        for (int q = pfirst_s[id]; q < q1; ++q) {
          const int st = pstart_s[q];
          if (j < st + pcnt_s[q]) { row = prow_s[q] + (j - st); break; }
        }
      }
      dst[i] = row;
      wout[i] = wv[c];
    }
  }
}

template <int M>
hipError_t launch_map(const moonep_sizes& s, const int32_t* ids, const float* w, int32_t* plan,
                      const int32_t* ws, hipStream_t st) {
  const size_t lds = (size_t)(kMapWaves * s.E + 4 * s.E + 3 * s.P_max) * sizeof(int32_t);
  hipLaunchKernelGGL(map_kernel<M>, dim3(s.nblk), dim3(kMapThreads), lds, st, ids, w, plan,
                     ws, s);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_plan(const moonep_sizes& s, const int32_t* ids, const float* w,
                       int32_t* plan, int32_t* ws, hipStream_t st) {
  hipLaunchKernelGGL(hist_kernel, dim3(s.nblk), dim3(kMapThreads),
                     (size_t)s.E * sizeof(int32_t), st, ids, ws, s);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(planner_kernel, dim3(1), dim3(kPlanThreads),
                     (size_t)6 * s.E * sizeof(int32_t), st, plan, ws, s);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  switch (s.blk / kMapThreads) {
    case 1: return launch_map<1>(s, ids, w, plan, ws, st);
    case 2: return launch_map<2>(s, ids, w, plan, ws, st);
    case 4: return launch_map<4>(s, ids, w, plan, ws, st);
    case 8: return launch_map<8>(s, ids, w, plan, ws, st);
    case 16: return launch_map<16>(s, ids, w, plan, ws, st);
    case 32: return launch_map<32>(s, ids, w, plan, ws, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace moonep
