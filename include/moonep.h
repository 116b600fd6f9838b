/*
 * moonep.h -- C ABI of the balanced expert-parallel hot path on one MI355X (gfx950).
 *
 * R expert-parallel ranks are simulated as partitions of one GPU's HBM.  One MoE layer
 * step runs four calls, in the order the pages give for a forward and backward pass
 * ("MoonshotAI/MoonEP 딥다이브" (fiv.co.kr), section 5: planning -> dispatch -> expert
 * compute -> combine -> grad_reduce):
 *
 *   moonep_plan        live top-K router output -> replica plan + token->row map
 *   moonep_dispatch    zero-copy scatter of bf16 token rows into static per-rank buffers
 *   moonep_combine     weighted gather of expert outputs back to token order
 *   moonep_reduce_grad replica gradients summed into their home experts
 *
 * Notation.  T = R*S tokens; token t comes from rank t / S.  Assignment i = t*K + k.
 * E_loc = E/R experts per rank; expert e is homed on rank e / E_loc.  C = S*K is every
 * rank's exact quota ("Moonshot AI Open-Sources MoonEP" (tldrocket.com), paragraph 3).
 * G = E_loc + slots groups per rank.  NvS = align16(C + G*15) rows per rank buffer
 * (S*K plus alignment padding: deep dive, section 4, design pattern 2).
 *
 * Conventions for every call:
 *   - Device pointers are plain HIP device addresses; the caller owns and allocates all
 *     memory.  The library never allocates, frees or synchronises (except
 *     moonep_plan_status, which waits on `stream`).  moonep_plan_noalloc alone uses
 *     library-owned device memory: a static per-GPU workspace array.
 *   - All GPU work is enqueued on `stream` (0 = the null stream) and is asynchronous.
 *   - Return value: MOONEP_OK (0) or a negative MOONEP_E* code.  Argument errors
 *     (EINVAL, ELIMIT, EALIGN, EPLAN) are found on the host and nothing is enqueued; an
 *     EHIP from a call that launches several kernels (moonep_plan, the staged calls) can
 *     follow launches of that call that were already enqueued.  Each call clears the
 *     thread's earlier HIP error before launching, so an EHIP is its own.  Data errors
 *     found on the device (an expert id outside [0, E)) are never reported by a return
 *     code: they set the plan's status word, read with moonep_plan_status; such a plan
 *     maps nothing (every dst_row is -1), dispatch then writes nothing, combine writes
 *     zero rows and reduce adds nothing.
 *   - Calls are thread-safe; the library has no global mutable state apart from
 *     moonep_plan_noalloc's per-GPU workspace array (see there).
 */
#ifndef MOONEP_H_
#define MOONEP_H_

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOONEP_ROW_ALIGN 16      /* rows: each home/slot group starts on a multiple */
#define MOONEP_MAX_R 64          /* the planner keeps one wave64 lane per rank      */
#define MOONEP_MAX_E 1024
#define MOONEP_MAX_K 32
#define MOONEP_MAX_SLOTS 256
/* largest planning workspace moonep_plan_noalloc serves from its static device array */
#define MOONEP_NOALLOC_WORKSPACE_MAX (8 << 20)

enum {
  MOONEP_OK = 0,
  MOONEP_EINVAL = -1,   /* a size or pointer argument is invalid                       */
  MOONEP_ELIMIT = -2,   /* sizes beyond MOONEP_MAX_* or int32 row indexing              */
  MOONEP_EPLAN = -3,    /* the plan descriptor is not initialised or does not match     */
  MOONEP_EHIP = -4,     /* a HIP launch or copy failed                                  */
  MOONEP_EALIGN = -5    /* a data pointer is not 16-byte aligned                        */
};

/* Sizes of one (R, E, K, S, slots) problem; filled by moonep_query (host only). */
typedef struct moonep_sizes {
  int32_t R, E, K, S, slots;
  int32_t E_loc, C, G, NvS, P_max;
  int64_t T, A;
  int64_t recv_rows;        /* R * NvS: rows of the dispatch buffer [R, NvS, H]          */
  int64_t plan_bytes;       /* device bytes of the plan blob                             */
  int64_t workspace_bytes;  /* device bytes of the transient workspace of moonep_plan    */
  int32_t nblk, blk;        /* assignment blocks used by the plan kernels                */
  /* int32-element offsets of the plan blob's arrays (for inspection and tests):        */
  int64_t o_hdr, o_load, o_shed, o_keep, o_home_row, o_pfirst, o_pnum, o_pieces,
          o_slot_expert, o_off, o_red, o_xtab, o_ptab, o_dst_row, o_w;
} moonep_sizes;

/* Host-side handle of a plan: sizes plus the caller's device blob.  Filled by
 * moonep_plan; read by the other calls.  Copying the struct copies the handle. */
typedef struct moonep_plan_desc {
  uint32_t magic;
  moonep_sizes sz;
  void* dev;                /* device blob of sz.plan_bytes, 256-byte aligned            */
} moonep_plan_desc;

/* Plan statistics, copied from the device by moonep_plan_status. */
typedef struct moonep_plan_stats {
  int32_t status;           /* 0 = valid plan; 1 = an expert id was outside [0, E)       */
  int32_t bad_index;        /* smallest assignment index with a bad id, else -1          */
  int32_t n_pieces;         /* replica pieces (slot-backed + fallback)                   */
  int32_t n_replicas;       /* slot-backed pieces = prefetch slots in use                */
  int32_t n_fallback;       /* pieces served by cross-partition weight reads             */
  int32_t max_pieces_per_rank;
  int32_t n_red;            /* experts with at least one slot replica                    */
  int32_t n_shed;           /* experts that shed assignments                             */
  int32_t max_load;         /* largest per-expert load                                   */
} moonep_plan_stats;

/* Sizes for a problem, host only ("MoonshotAI/MoonEP 딥다이브", section 4, design
 * pattern 2: per-rank buffers have a static size, S*K rows plus alignment padding, fixed
 * before any routing is seen; section 2, point 3: so the host never waits for the device
 * to learn how much to allocate).  Every buffer the other calls take is sized from here.
 * EINVAL unless R>=1, E%R==0, 1<=K<=E, S>=1, slots>=0; ELIMIT beyond R<=64, E<=1024,
 * K<=32, slots<=256, or when R*NvS or T*K exceeds int32. */
int moonep_query(int R, int E, int K, int S, int slots, moonep_sizes* out);

/* Planning ("Moonshot AI Open-Sources MoonEP", paragraph 3: duplicate a few overloaded
 * experts, planned from live router output, so every rank receives exactly S*K; deep
 * dive, section 4, design pattern 1: plan once, reuse).
 *
 *   topk_ids   device int32 [T, K] row-major, ranks contiguous (token t from rank t/S)
 *   topk_w     device fp32  [T, K]; copied into the plan, so combine needs no weights
 *   plan_dev   device blob of moonep_sizes.plan_bytes, 256-byte aligned
 *   workspace  device scratch of moonep_sizes.workspace_bytes, 256-byte aligned,
 *              zero-filled before its first use: its first word counts the planning
 *              workgroups as they finish, and every call leaves it at zero again, so a
 *              workspace reused call after call (for any sizes) needs no clearing.  A
 *              workspace whose first word is not zero leaves the plan undefined; every
 *              kernel that reads a plan still keeps its accesses inside the plan and the
 *              buffers it was given, whatever the plan holds.  Free for other use
 *              once the plan's kernels have run on `stream`; two calls whose kernels
 *              overlap in time must not share a workspace
 *   desc       host handle, filled synchronously (sizes + plan_dev)
 *
 * Boundary note.  The plan is a device blob, as in a blob-only signature, but the call also
 * fills `desc`, a host copy of the problem's sizes plus the blob's address, and every
 * later call takes `desc` instead of the bare blob.  The sizes of every launch (grid,
 * rows, K) are then known on the host without reading the device, so no call ever waits
 * for the plan (the deep dive's section 2, point 3: no per-layer host synchronisation);
 * the blob itself stays on the device and is what the kernels read.
 *
 * Errors: EINVAL, ELIMIT and EALIGN are found on the host before anything is enqueued;
 * EHIP means a launch failed, in which case kernels launched before it by this call may
 * already be enqueued (the plan is then unusable until a later call succeeds).
 *
 * The plan rule: experts are taken by (load descending, id ascending); an expert on a
 * home whose load exceeds S*K sheds min(load, remaining excess); each shed assignment
 * goes to the lowest-id rank still short of S*K that has a free prefetch slot, else
 * (slots exhausted) to the lowest-id rank still short, as a fallback piece whose expert
 * weights are read across partitions ("Moonshot AI Open-Sources MoonEP", paragraph 5).
 * Within an expert, assignments are taken in increasing i: the home keeps the first
 * `keep`, replica pieces take the rest in creation order.  Each rank's buffer holds its
 * home experts, then its slots (each group 16-row aligned), then a fallback region.
 * Deterministic: the same ids give a bit-identical plan. */
int moonep_plan(const int32_t* topk_ids, const float* topk_w, int R, int E, int K, int S,
                int slots, void* plan_dev, void* workspace, moonep_plan_desc* desc,
                hipStream_t stream);

/* moonep_plan for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Same arguments, result
 * and errors as moonep_plan, without `workspace`: the planning kernels use a file-scope
 * device array of MOONEP_NOALLOC_WORKSPACE_MAX bytes (8 MiB; enough for every
 * (R, E, K, S, slots) whose moonep_sizes.workspace_bytes is at most that), one copy per GPU,
 * held until the process ends.  The call allocates and frees nothing; the caller still
 * provides topk_ids, topk_w and the plan blob.
 *   ELIMIT  when workspace_bytes exceeds MOONEP_NOALLOC_WORKSPACE_MAX (nothing enqueued)
 *   EINVAL  when `stream` does not belong to the current device (the array used is the
 *           current device's)
 * Every call on one GPU shares that GPU's array: two of these calls whose kernels overlap
 * in time on the same GPU (different streams, or different host threads without ordering)
 * race and may both produce wrong plans.  Calls ordered on one stream are safe.  The array
 * is zero when the library is loaded; every call leaves its first word (the planning
 * workgroups' arrival count) at zero again and the rest holding the last call's
 * contents. */
int moonep_plan_noalloc(const int32_t* topk_ids, const float* topk_w, int R, int E, int K, int S,
                        int slots, void* plan_dev, moonep_plan_desc* desc, hipStream_t stream);

/* Zero-copy dispatch ("MoonshotAI/MoonEP 딥다이브", section 2, point 2: each token row
 * is written straight into its final expert position; no permute, no staging copy):
 *   recv[dst_row[t, k], :] = x[t, :]  (bit copy) for every assignment.
 *   x     device bf16 [T, H] (raw 16-bit patterns)      recv  device bf16 [R*NvS, H]
 * H % 8 == 0; x and recv 16-byte aligned.  Padding rows of recv are not written. */
int moonep_dispatch(const moonep_plan_desc* plan, const uint16_t* x, int H, uint16_t* recv,
                    hipStream_t stream);

/* Weighted combine (deep dive, section 1: dispatch -> expert compute -> combine):
 *   out[t, :] = bf16_rne( sum_{k=0..K-1} w[t,k] * float(y[dst_row[t,k], :]) )
 * accumulated in fp32, k ascending, each product and sum rounded separately (no fused
 * multiply-add), one round-to-nearest-even to bf16 at the end.
 *   y     device bf16 [R*NvS, H] (expert outputs, laid out like recv)
 *   out   device bf16 [T, H]
 * H % 8 == 0; y and out 16-byte aligned; out must not overlap y. */
int moonep_combine(const moonep_plan_desc* plan, const uint16_t* y, int H, uint16_t* out,
                   hipStream_t stream);

/* Staged (non-zero-copy) dispatch, the A/B baseline for zero-copy ("MoonshotAI/MoonEP
 * 딥다이브", section 2, point 2: the conventional scheme receives tokens into a
 * communication buffer, then permutes and copies them into the user buffer; section 8,
 * exercise D measures that copy):
 *   stage[t*K + k, :] = x[t, :]                  (arrival order)
 *   recv[dst_row[t,k], :] = stage[t*K + k, :]    (the epilogue copy)
 * recv ends bit-identical to moonep_dispatch's.  stage: device bf16 [T*K, H]. */
int moonep_dispatch_staged(const moonep_plan_desc* plan, const uint16_t* x, int H,
                           uint16_t* stage, uint16_t* recv, hipStream_t stream);

/* Staged combine (same passage): the prologue copy stage[t*K + k, :] = y[dst_row[t,k], :],
 * then out[t] as in moonep_combine, read from the staging buffer.  out ends bit-identical
 * to moonep_combine's.  stage: device bf16 [T*K, H]. */
int moonep_combine_staged(const moonep_plan_desc* plan, const uint16_t* y, int H,
                          uint16_t* stage, uint16_t* out, hipStream_t stream);

/* Backward of dispatch, reusing the forward plan ("MoonshotAI/MoonEP 딥다이브", section 4,
 * design pattern 1: the plan serves both backward passes).  Dispatch copied x[t] into
 * its K rows, so
 *   gx[t, :] = bf16_rne( sum_{k=0..K-1} float(g_recv[dst_row[t,k], :]) )
 * summed in fp32, k ascending.
 *   g_recv  device bf16 [R*NvS, H] (gradient w.r.t. the dispatched rows)
 *   gx      device bf16 [T, H]
 * H % 8 == 0; both 16-byte aligned; gx must not overlap g_recv. */
int moonep_dispatch_bwd(const moonep_plan_desc* plan, const uint16_t* g_recv, int H,
                        uint16_t* gx, hipStream_t stream);

/* Backward of combine, reusing the forward plan (same passage).  For
 * out[t] = sum_k w[t,k] * y[dst_row[t,k]]:
 *   g_y[dst_row[t,k], :] = bf16_rne( w[t,k] * float(dout[t, :]) )   (fp32 product)
 *   dw[t, k]             = sum_h float(dout[t,h]) * float(y[dst_row[t,k], h])   (fp32, fused
 *                          multiply-add, summation order unspecified)
 *   dout  device bf16 [T, H];  y  device bf16 [R*NvS, H] (the forward expert outputs)
 *   g_y   device bf16 [R*NvS, H], may be y itself (in place); padding rows untouched
 *   dw    device fp32 [T, K]
 * H % 8 == 0; dout, y, g_y 16-byte aligned. */
int moonep_combine_bwd(const moonep_plan_desc* plan, const uint16_t* dout, const uint16_t* y,
                       int H, uint16_t* g_y, float* dw, hipStream_t stream);

/* Replica-gradient reduce (deep dive, section 4, design pattern 3: a replica's gradient
 * is kept apart and added to its home expert, so training equals no replication):
 *   for each expert e, for its slot pieces in creation order:
 *       home_grad[e, :] += rep_grad[rank, slot, :]      (fp32 adds, in that order)
 *   home_grad  device fp32 [E, G_el], updated in place
 *   rep_grad   device fp32 [R, slots, G_el]
 * G_el % 4 == 0; both 16-byte aligned.  Fallback pieces own no slot and add nothing. */
int moonep_reduce_grad(const moonep_plan_desc* plan, float* home_grad, const float* rep_grad,
                       int64_t G_el, hipStream_t stream);

/* Replica weight prefetch ("Moonshot AI Open-Sources MoonEP", paragraph 3: the duplicated
 * experts are prefetched before computation starts; "MoonshotAI/MoonEP 딥다이브", section 3:
 * Buffer.prefetch_weight):
 *   for every slot piece p of the plan:  slot_w[r_p, slot_p, :] = home_w[e_p, :]  (bit copy)
 *   home_w  device bf16 [E, W_el] (each expert's weights, any layout, W_el elements)
 *   slot_w  device bf16 [R, slots, W_el]; slots no piece uses are not written
 * W_el % 8 == 0; both 16-byte aligned; slot_w must not overlap home_w.  Fallback pieces
 * own no slot: their rank reads home_w directly (see moonep_expert_stub). */
int moonep_prefetch_weight(const moonep_plan_desc* plan, const uint16_t* home_w, int64_t W_el,
                           uint16_t* slot_w, hipStream_t stream);

/* A toy expert that checks which weights each buffer group reads ("Moonshot AI
 * Open-Sources MoonEP", paragraph 5: without a free slot the rank falls back to remote
 * reads of the home expert):
 *   y[row, h] = bf16_rne( float(recv[row, h]) * float(W[h]) ),  h < H,
 * for every mapped row, where W is home_w[e] for a home group, slot_w[r, slot] for a slot
 * group and home_w[e] (read across partitions) for a fallback piece.  The row's expert e
 * comes from the caller's topk_ids (the same array given to moonep_plan).
 *   topk_ids int32 [T, K];  recv, y  bf16 [R*NvS, H];  home_w bf16 [E, W_el];
 *   slot_w bf16 [R, slots, W_el]  (W_el >= H, W_el % 8 == 0, H % 8 == 0)
 * Padding rows of y are not written. */
int moonep_expert_stub(const moonep_plan_desc* plan, const int32_t* topk_ids,
                       const uint16_t* recv, const uint16_t* home_w, const uint16_t* slot_w,
                       int64_t W_el, int H, uint16_t* y, hipStream_t stream);

/* Waits for `stream`, then copies the plan's statistics to the host.  The only call
 * that synchronises: the hot path itself never reads the plan back ("MoonshotAI/MoonEP
 * 딥다이브", section 2, point 3: static buffers remove the per-layer host sync), so data
 * errors found on the device (status 1: an expert id outside [0, E); status 2: an
 * internal invariant of the plan failed) are reported here, when the caller asks, and
 * meanwhile make the plan map nothing. */
int moonep_plan_status(const moonep_plan_desc* plan, moonep_plan_stats* out,
                       hipStream_t stream);

const char* moonep_strerror(int code);

#ifdef __cplusplus
}
#endif
#endif /* MOONEP_H_ */
