// Internal layout of the plan blob and the plan workspace, shared by the kernels and the
// C ABI.  Everything is int32 elements; each array starts on a 64-element (256-byte)
// boundary.
#pragma once

#include <stdint.h>
#include <algorithm>
#include <hip/hip_runtime.h>

#include "moonep.h"

namespace moonep {

constexpr uint32_t kMagic = 0x4D4F4E45u;   // plan descriptor / blob tag
constexpr int kRowAlign = MOONEP_ROW_ALIGN;
constexpr int kMapWaves = 8;                // waves per workgroup of the hist/map kernels
constexpr int kMapThreads = kMapWaves * 64;
constexpr int kPlanThreads = 1024;          // the single planner workgroup
constexpr int kPieceInts = 8;               // e, r, slot, cnt, start, fbpos, row0, pad
constexpr int kColumnBudget = 32768;        // blocks x experts the planner scans in registers
constexpr int kMapChunks = 8;               // 64-assignment chunks per map wave, at most
constexpr int kWsCtl = 64;                  // control words at the head of the plan workspace

// header words
enum Hdr : int {
  H_MAGIC = 0, H_STATUS, H_NPIECES, H_NREPLICAS, H_NFALLBACK, H_MAXPPR, H_NRED, H_BADIDX,
  H_NSHED, H_MAXLOAD,
  H_R = 16, H_E, H_K, H_S, H_SLOTS, H_NVS,
  H_WORDS = 64
};

// piece fields
enum Piece : int { P_E = 0, P_R, P_SLOT, P_CNT, P_START, P_FBPOS, P_ROW0 };

__host__ __device__ inline int64_t align64(int64_t n) { return (n + 63) / 64 * 64; }

// Fills every derived field of `s` from R, E, K, S, slots; returns MOONEP_OK or an error.
inline int fill_sizes(int R, int E, int K, int S, int slots, moonep_sizes* s) {
  if (R < 1 || E < 1 || K < 1 || S < 1 || slots < 0 || E % R != 0 || K > E)
    return MOONEP_EINVAL;
  if (R > MOONEP_MAX_R || E > MOONEP_MAX_E || K > MOONEP_MAX_K || slots > MOONEP_MAX_SLOTS)
    return MOONEP_ELIMIT;
  s->R = R; s->E = E; s->K = K; s->S = S; s->slots = slots;
  s->E_loc = E / R;
  const int64_t C = (int64_t)S * K;
  const int64_t G = (int64_t)s->E_loc + slots;
  const int64_t NvS = (C + G * (kRowAlign - 1) + kRowAlign - 1) / kRowAlign * kRowAlign;
  const int64_t T = (int64_t)R * S;
  const int64_t A = T * K;
  if (C > INT32_MAX || NvS * R > INT32_MAX || A > INT32_MAX) return MOONEP_ELIMIT;
  s->C = (int32_t)C; s->G = (int32_t)G; s->NvS = (int32_t)NvS;
  s->P_max = E + R;
  s->T = T; s->A = A;
  s->recv_rows = NvS * R;
  // assignment blocks: kMapThreads * m assignments each, m a power of two in [1, 32],
  // aiming at no more than 32768 / E blocks: the planner then scans at most 32 block
  // counts per thread (1024 threads, E columns), held in registers.
  const int64_t target = std::max<int64_t>(1, kColumnBudget / E);
  int64_t m = 1;
  while (m < 32 && (int64_t)kMapThreads * m * target < A) m *= 2;
  s->blk = (int32_t)(kMapThreads * m);
  s->nblk = (int32_t)((A + s->blk - 1) / s->blk);
  int64_t o = 0;
  s->o_hdr = o;         o += align64(H_WORDS);
  s->o_load = o;        o += align64(E);
  s->o_shed = o;        o += align64(E);
  s->o_keep = o;        o += align64(E);
  s->o_home_row = o;    o += align64(E);
  s->o_pfirst = o;      o += align64(E);
  s->o_pnum = o;        o += align64(E);
  s->o_pieces = o;      o += align64((int64_t)s->P_max * kPieceInts);
  s->o_slot_expert = o; o += align64((int64_t)R * (slots > 0 ? slots : 1));
  s->o_off = o;         o += align64((int64_t)R * (G + 1));
  s->o_red = o;         o += align64(E);
  s->o_xtab = o;        o += align64((int64_t)4 * E);            // int4 per expert
  s->o_ptab = o;        o += align64((int64_t)4 * s->P_max);     // int4 per piece
  s->o_dst_row = o;     o += align64(A);
  s->o_w = o;           o += align64(A);
  s->plan_bytes = o * 4;
  // workspace: kWsCtl control words (word 0: the histogram workgroups' arrival count,
  // zero between calls), then per-block expert counts [nblk][E] (overwritten by the
  // planner with per-block bases), per-block first bad index [nblk], per-wave prefixes
  // inside each block [nblk][kMapWaves][E], and, when a histogram wave's 64*m assignments
  // are split into Q > 1 map sub-blocks, the wave's running counts at each inner
  // sub-block boundary [nblk][kMapWaves][Q-1][E].  The offsets below count from the end
  // of the control words.
  const int64_t Q = m > kMapChunks ? m / kMapChunks : 1;
  s->workspace_bytes = (kWsCtl + align64((int64_t)s->nblk * E) + align64(s->nblk) +
                        align64((int64_t)s->nblk * kMapWaves * E) +
                        align64((int64_t)s->nblk * kMapWaves * (Q - 1) * E)) * 4;
  return MOONEP_OK;
}

// chunks per map wave and map sub-blocks per histogram wave
__host__ __device__ inline int map_chunks(const moonep_sizes& s) {
  const int m = s.blk / kMapThreads;
  return m < kMapChunks ? m : kMapChunks;
}
__host__ __device__ inline int map_split(const moonep_sizes& s) {
  return s.blk / kMapThreads / map_chunks(s);
}

// workspace offsets (int32 elements)
__host__ __device__ inline int64_t ws_bad(const moonep_sizes& s) { return align64((int64_t)s.nblk * s.E); }
__host__ __device__ inline int64_t ws_sub(const moonep_sizes& s) { return ws_bad(s) + align64(s.nblk); }
__host__ __device__ inline int64_t ws_snap(const moonep_sizes& s) {
  return ws_sub(s) + align64((int64_t)s.nblk * kMapWaves * s.E);
}

// Launchers (defined in the .hip files).  Each returns the launch status of what it
// enqueued; the C ABI clears any earlier, unrelated error of the thread before calling.
// Whether the dispatch/combine grids (one workgroup per token and row chunk) fit the
// launch limit for rows of H bf16 elements:
bool move_grid_fits(const moonep_sizes& s, int H);
hipError_t launch_plan(const moonep_sizes& s, const int32_t* ids, const float* w,
                       int32_t* plan, int32_t* ws, hipStream_t st);
hipError_t launch_dispatch(const moonep_sizes& s, const int32_t* plan, const uint16_t* x,
                           int H, uint16_t* recv, hipStream_t st);
hipError_t launch_combine(const moonep_sizes& s, const int32_t* plan, const uint16_t* y,
                          int H, uint16_t* out, hipStream_t st);
hipError_t launch_dispatch_staged(const moonep_sizes& s, const int32_t* plan, const uint16_t* x,
                                  int H, uint16_t* stage, uint16_t* recv, hipStream_t st);
hipError_t launch_combine_staged(const moonep_sizes& s, const int32_t* plan, const uint16_t* y,
                                 int H, uint16_t* stage, uint16_t* out, hipStream_t st);
hipError_t launch_dispatch_bwd(const moonep_sizes& s, const int32_t* plan, const uint16_t* g_recv,
                               int H, uint16_t* gx, hipStream_t st);
hipError_t launch_combine_bwd(const moonep_sizes& s, const int32_t* plan, const uint16_t* dout,
                              const uint16_t* y, int H, uint16_t* g_y, float* dw,
                              hipStream_t st);
hipError_t launch_prefetch(const moonep_sizes& s, const int32_t* plan, const uint16_t* home_w,
                           int64_t W_el, uint16_t* slot_w, hipStream_t st);
hipError_t launch_expert_stub(const moonep_sizes& s, const int32_t* plan, const int32_t* ids,
                              const uint16_t* recv, const uint16_t* home_w,
                              const uint16_t* slot_w, int64_t W_el, int H, uint16_t* y,
                              hipStream_t st);
hipError_t launch_reduce(const moonep_sizes& s, const int32_t* plan, float* home,
                         const float* rep, int64_t G_el, hipStream_t st);

}  // namespace moonep
