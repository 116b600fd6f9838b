// Data movement of the balanced expert-parallel step: zero-copy dispatch, weighted
// combine, replica-gradient reduce, and the backward, prefetch and staged variants.  All
// are HBM-bound streams with no reuse between workgroups: 16-byte vector loads and
// stores, many bytes in flight per CU, and cache hints chosen by measurement (each
// kernel's comment gives them).
//
// "MoonshotAI/MoonEP 딥다이브" (fiv.co.kr), section 2, point 2: token rows go straight
// to their final expert position and the buffer is handed to expert compute as a view,
// with no permute or staging copy; section 4, pattern 3: replica gradients are summed
// into their home expert.
#include "moonep_internal.h"

namespace moonep {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf_lo(unsigned int v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf_hi(unsigned int v) { return __uint_as_float(v & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even; NaN -> 0x7FC0.
__device__ __forceinline__ unsigned int to_bf16(float f) {
  const unsigned int u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Counts and piece ranges read from a plan are clamped to the tables they index: a blob
// that no plan call finished writing can hold anything, and every read stays inside it.
__device__ __forceinline__ int clamp_count(int n, int max_n) { return min(max(n, 0), max_n); }
__device__ __forceinline__ void piece_range(int first, int count, int pmax, int* q0, int* q1) {
  *q0 = clamp_count(first, pmax);
  *q1 = *q0 + clamp_count(count, pmax - *q0);
}

// Threads per workgroup (a multiple of 64, at most 1024) and vectors per thread (at most
// umax) for a row of nvec 16-byte vectors: the fewest idle lanes first, then the vectors
// per thread closest to upref, then the most threads.
void row_shape(int nvec, int umax, int upref, int* threads, int* u) {
  long best[3] = {-1, 0, 0};
  for (int t = 64; t <= 1024; t += 64) {
    for (int uu = 1; uu <= umax; ++uu) {
      const long cover = (long)t * uu;
      const long waste = (nvec + cover - 1) / cover * cover - nvec;
      const long d = uu > upref ? uu - upref : upref - uu;
      const bool better = best[0] < 0 || waste < best[0] ||
                          (waste == best[0] && (d < best[1] || (d == best[1] && t > *threads)));
      if (better) { best[0] = waste; best[1] = d; *threads = t; *u = uu; }
    }
  }
}

// ---------------------------------------------------------------------------------------
// dispatch: recv[dst_row[t, k]] = x[t]
// ---------------------------------------------------------------------------------------
// One single-wave workgroup per (token, chunk of kDispChunk 16-byte vectors): each lane
// loads kDispU vectors of the chunk (64 vectors apart, so every load and store of the
// wave covers 1 KB contiguous), then stores each of them to the token's K destination
// rows, vector by vector, with non-temporal stores.  Measured on MI355X, interleaved A/B
// in one process on DeepSeek-V3-, Kimi- and decode-shaped routing: one wave per 2 KB
// chunk is 2-5% faster than one 448-thread workgroup per token, and a token-major launch
// order beats chunk-major or XCD-local orders.  Plain stores run within 1% of
// non-temporal ones here, but leave dirty lines in the caches that cost the following
// combine 2-7%.  A workgroup of one wave starts as soon as any wave slot of a CU frees,
// so the CUs stay full of short-lived waves; larger workgroups wait for several free
// slots at once (2-, 7-wave workgroups and 2-3 tokens per wave measured 2-20% slower).
//
// One explicit wait separates the loads from the stores.  gfx9 counts stores in the
// same vmcnt counter as loads, and the loads and stores here sit under conditions (a
// partial last chunk, an unmapped row), so without it the compiler cannot tell how many
// operations follow a load on a given path and places a vmcnt(0) before every store:
// each of the K*kDispU stores of a wave then waits for the previous one's write
// acknowledgement.  With the single wait the stores issue back to back: +2-3% at
// DeepSeek-V3 shape and Kimi scale in the step at the same residency cap, and the best
// cap moved from 6 to 5 workgroups per CU.  Waiting per vector instead (branch-free code
// lets the compiler count exactly) measured 6% slower than waiting once for both.
//
// KT = K when K is a compile-time constant (the rows are then held in registers), else 0.
// STAGED: the destination is row t*K + k of a [T*K, H] staging buffer (the non-zero-copy
// A/B baseline), not the plan's row; it has its own instantiation so that profiles keep
// the zero-copy kernel's figures apart.
constexpr int kWave = 64;
constexpr int kDispU = 2;
constexpr int kDispChunk = kWave * kDispU;     // 128 vectors = 2 KB of a bf16 row
constexpr int kCombChunk = kWave;              // 64 vectors = 1 KB of a bf16 row
// s_waitcnt vmcnt(0) in the gfx9 encoding, with expcnt and lgkmcnt left at their maximum
constexpr int kWaitVmcnt0 = 0x0F70;

// Residency caps.  Each launch requests dynamic LDS that the kernels never touch, so that
// at most floor(160 KB / request) of their single-wave workgroups sit on a CU at once
// (gfx950: 160 KB of LDS per CU): fewer tokens in flight, fewer rows of the big buffer
// open at once.  Chosen on MI355X inside the real step (plan -> dispatch -> combine,
// cycling through the routing batches, interleaved variants of the library in one
// process), which is where it counts: the cache and memory state the previous kernel
// leaves behind moves the optimum against back-to-back launches of one kernel.
//   combine, 9 per CU: +8% over no cap at DeepSeek-V3 shape, +11% at Kimi scale, and
//     7, 8, 10 or 11 per CU all lose to 9 there and at decode; but -7% when the gathered rows
//     fit in the 256 MB last-level cache (more rows in flight then win), so the cap
//     applies only to larger buffers;
//   dispatch, 5 per CU: at DeepSeek-V3 shape and Kimi scale +2-4% over 6 per CU, +6-7%
//     over 7 per CU and +3-9% over 4 per CU; within 1% of them at decode; with no cap
//     the kernel loses 11%.
// Each request sits mid-interval, clear of the LDS allocation granularity.
constexpr int kDispLdsBytes = 29 * 1024;       // 5 dispatch workgroups per CU
constexpr int kCombLdsBytes = 17 * 1024;       // 9 combine workgroups per CU
constexpr int64_t kLastLevelCacheBytes = 256ll << 20;   // MI355X Infinity Cache

template <int KT, bool STAGED>
__global__ __launch_bounds__(kWave) void dispatch_kernel(const int32_t* __restrict__ dst,
                                                         const u32x4* __restrict__ x,
                                                         u32x4* __restrict__ recv, int Krt,
                                                         int nvec, int nch, int nrows) {
  const int K = KT > 0 ? KT : Krt;
  const int64_t t = blockIdx.x / nch;
  const int c0 = (int)(blockIdx.x - t * nch) * kDispChunk + (int)threadIdx.x;
  const int32_t* d = STAGED ? nullptr : dst + t * K;
  const u32x4* src = x + t * nvec;
  u32x4 buf[kDispU];
  if constexpr (KT > 0) {
    int rows[KT];
#pragma unroll
    for (int k = 0; k < KT; ++k) rows[k] = STAGED ? (int)(t * K + k) : d[k];
#pragma unroll
    for (int u = 0; u < kDispU; ++u) {
      const int v = c0 + u * kWave;
      if (v < nvec) buf[u] = src[v];
    }
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
#pragma unroll
    for (int u = 0; u < kDispU; ++u) {
      const int v = c0 + u * kWave;
      if (v < nvec) {
#pragma unroll
        for (int k = 0; k < KT; ++k)
          if ((unsigned)rows[k] < (unsigned)nrows)   // -1: unmapped
            __builtin_nontemporal_store(buf[u], recv + (int64_t)rows[k] * nvec + v);
      }
    }
  } else {
#pragma unroll
    for (int u = 0; u < kDispU; ++u) {
      const int v = c0 + u * kWave;
      if (v < nvec) buf[u] = src[v];
    }
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    for (int k = 0; k < K; ++k) {
      const int row = STAGED ? (int)(t * K + k) : d[k];
      if ((unsigned)row >= (unsigned)nrows) continue;   // -1: unmapped
      u32x4* o = recv + (int64_t)row * nvec;
#pragma unroll
      for (int u = 0; u < kDispU; ++u) {
        const int v = c0 + u * kWave;
        if (v < nvec) __builtin_nontemporal_store(buf[u], o + v);
      }
    }
  }
}

// ---------------------------------------------------------------------------------------
// combine: out[t] = bf16( sum_k w[t,k] * y[dst_row[t,k]] ), fp32, k ascending, no FMA
// ---------------------------------------------------------------------------------------
// One single-wave workgroup per (token, chunk of 64 vectors): each lane issues its K row
// loads (non-temporal) before any arithmetic, then acc = acc + w*y per element with a
// separate fp32 multiply and add, in k order, one round-to-nearest-even to bf16, and a
// non-temporal store.  Measured on MI355X against one 448-thread workgroup per token
// (interleaved A/B): 2-6% faster; plain loads or a plain store lose 6-10%.
// An assignment whose plan row is -1 (an invalid plan) adds nothing, so such a token's
// output is a zero row.  STAGED: the K rows are read from staging rows t*K + k (the
// non-zero-copy prologue filled them); the plan's row still decides whether an
// assignment is mapped.  WEIGHTED = false is the gradient of dispatch:
// gx[t] = bf16(sum_k g_recv[dst_row[t,k]]).
template <int KT, bool WEIGHTED, bool STAGED>
__global__ __launch_bounds__(kWave) void combine_kernel(const int32_t* __restrict__ dst,
                                                        const float* __restrict__ wts,
                                                        const u32x4* __restrict__ y,
                                                        u32x4* __restrict__ out, int Krt,
                                                        int nvec, int nch, int nrows) {
  const int K = KT > 0 ? KT : Krt;
  const int64_t t = blockIdx.x / nch;
  const int v = (int)(blockIdx.x - t * nch) * kCombChunk + (int)threadIdx.x;
  const int32_t* d = dst + t * K;
  const float* wt = wts + t * K;
  if (v >= nvec) return;
  float acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.f;
  auto add = [&](const u32x4 yv, float wk) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float p0 = WEIGHTED ? wk * bf_lo(yv[q]) : bf_lo(yv[q]);
      const float p1 = WEIGHTED ? wk * bf_hi(yv[q]) : bf_hi(yv[q]);
      acc[2 * q] = acc[2 * q] + p0;
      acc[2 * q + 1] = acc[2 * q + 1] + p1;
    }
  };
  if constexpr (KT > 0) {
    int rows[KT];
    bool ok[KT];
#pragma unroll
    for (int k = 0; k < KT; ++k) {
      const int r = d[k];
      ok[k] = (unsigned)r < (unsigned)nrows;       // -1: unmapped
      rows[k] = STAGED ? (int)(t * K + k) : r;
    }
    u32x4 yv[KT];
#pragma unroll
    for (int k = 0; k < KT; ++k)
      yv[k] = ok[k] ? __builtin_nontemporal_load(y + (int64_t)rows[k] * nvec + v)
                    : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int k = 0; k < KT; ++k)
      if (ok[k]) add(yv[k], WEIGHTED ? wt[k] : 1.f);
  } else {
    for (int k = 0; k < K; ++k) {
      const int r = d[k];
      if ((unsigned)r >= (unsigned)nrows) continue;   // -1: unmapped
      const int64_t row = STAGED ? t * K + k : r;
      add(__builtin_nontemporal_load(y + row * nvec + v), WEIGHTED ? wt[k] : 1.f);
    }
  }
  u32x4 o;
#pragma unroll
  for (int q = 0; q < 4; ++q) o[q] = to_bf16(acc[2 * q]) | (to_bf16(acc[2 * q + 1]) << 16);
  __builtin_nontemporal_store(o, out + t * nvec + v);
}

// ---------------------------------------------------------------------------------------
// combine backward: g_y[dst_row[t,k]] = bf16(w[t,k] * dout[t]);
//                   dw[t,k] = sum_h dout[t,h] * y[dst_row[t,k],h]   (fp32, fused multiply-add)
// ---------------------------------------------------------------------------------------
// One workgroup per token.  Each thread holds U vectors of dout and takes the K rows of y
// in groups: it loads the same vectors of every row of the group, waits once, then keeps
// a partial dot product per row and writes the scaled dout vectors to the group's rows of
// g_y back to back (g_y may be y itself: each element is read before it is written by
// the same thread).  Without the single wait the compiler places a wait for every
// earlier memory operation before each store (vmcnt counts loads and stores alike), and
// the row-by-row load, wait, store sequence ran at 5.1 TB/s.  The K partials are summed
// over the wave with lane shuffles, then over the waves in LDS.  KMAX = K when K is a
// compile-time constant, else MOONEP_MAX_K with the loop bounded by the runtime K.
constexpr int kBwdGroup = 8;    // rows of y per group (fewer when U > 2 or K is not a constant)

template <int KMAX, int U>
__global__ __launch_bounds__(1024) void combine_bwd_kernel(const int32_t* __restrict__ dst,
                                                           const float* __restrict__ wts,
                                                           const u32x4* __restrict__ dout,
                                                           const u32x4* y, u32x4* g_y,
                                                           float* __restrict__ dw, int K,
                                                           int nvec, int nrows) {
  __shared__ float red[16][KMAX];
  const int64_t t = blockIdx.x;
  const int32_t* d = dst + t * K;
  const float* wt = wts + t * K;
  float part[KMAX];
#pragma unroll
  for (int k = 0; k < KMAX; ++k) part[k] = 0.f;
  for (int v0 = threadIdx.x; v0 < nvec; v0 += blockDim.x * U) {
    u32x4 dv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int v = v0 + u * blockDim.x;
      dv[u] = v < nvec ? __builtin_nontemporal_load(dout + t * nvec + v) : u32x4{0u, 0u, 0u, 0u};
    }
    // groups of up to 8 rows: every load of the group, one wait, then the group's stores
    // back to back (a row is read before it is overwritten when g_y is y)
    constexpr int NG = KMAX <= kBwdGroup && U <= 2 ? KMAX
                       : KMAX < 4 ? KMAX : KMAX > kBwdGroup && U > 2 ? 2 : 4;
#pragma unroll
    for (int k0 = 0; k0 < KMAX; k0 += NG) {
      if (k0 >= K) break;
      int row[NG];
      bool ok[NG];
      float wk[NG];
      u32x4 yv[NG][U];
#pragma unroll
      for (int j = 0; j < NG; ++j) {
        const int k = k0 + j;
        row[j] = k < K ? d[k] : -1;
        ok[j] = (unsigned)row[j] < (unsigned)nrows;      // -1: unmapped, or past K
        wk[j] = k < K ? wt[k] : 0.f;
      }
#pragma unroll
      for (int j = 0; j < NG; ++j)
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int v = v0 + u * blockDim.x;
          yv[j][u] = ok[j] && v < nvec ? __builtin_nontemporal_load(y + (int64_t)row[j] * nvec + v)
                                       : u32x4{0u, 0u, 0u, 0u};
        }
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
#pragma unroll
      for (int j = 0; j < NG; ++j) {
        if (!ok[j]) continue;
        u32x4* gdst = g_y + (int64_t)row[j] * nvec;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int v = v0 + u * blockDim.x;
          if (v >= nvec) continue;
          u32x4 g;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float d0 = bf_lo(dv[u][q]), d1 = bf_hi(dv[u][q]);
            part[k0 + j] = __builtin_fmaf(d0, bf_lo(yv[j][u][q]), part[k0 + j]);
            part[k0 + j] = __builtin_fmaf(d1, bf_hi(yv[j][u][q]), part[k0 + j]);
            g[q] = to_bf16(wk[j] * d0) | (to_bf16(wk[j] * d1) << 16);
          }
          __builtin_nontemporal_store(g, gdst + v);
        }
      }
    }
  }
  // sum the partial dot products over the workgroup
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    if (k >= K) break;
    float v = part[k];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    if (lane == 0) red[wave][k] = v;
  }
  __syncthreads();
  if ((int)threadIdx.x < K) {
    const int k = threadIdx.x;
    float v = 0.f;
    const int nw = (blockDim.x + 63) >> 6;
    for (int w = 0; w < nw; ++w) v += red[w][k];
    dw[t * K + k] = d[k] >= 0 ? v : 0.f;
  }
}

template <int KMAX>
void launch_combine_bwd_k(const moonep_sizes& s, const int32_t* dst, const float* w,
                          const uint16_t* dout, const uint16_t* y, uint16_t* g_y, float* dw,
                          int nvec, int threads, int u, hipStream_t st) {
  const dim3 grid((unsigned)s.T), block(threads);
  const u32x4* dv = reinterpret_cast<const u32x4*>(dout);
  const u32x4* yv = reinterpret_cast<const u32x4*>(y);
  u32x4* gv = reinterpret_cast<u32x4*>(g_y);
  const int nrows = (int)s.recv_rows;
  switch (u) {
    case 1: hipLaunchKernelGGL((combine_bwd_kernel<KMAX, 1>), grid, block, 0, st, dst, w, dv, yv, gv, dw, s.K, nvec, nrows); break;
    case 2: hipLaunchKernelGGL((combine_bwd_kernel<KMAX, 2>), grid, block, 0, st, dst, w, dv, yv, gv, dw, s.K, nvec, nrows); break;
    case 3: hipLaunchKernelGGL((combine_bwd_kernel<KMAX, 3>), grid, block, 0, st, dst, w, dv, yv, gv, dw, s.K, nvec, nrows); break;
    default: hipLaunchKernelGGL((combine_bwd_kernel<KMAX, 4>), grid, block, 0, st, dst, w, dv, yv, gv, dw, s.K, nvec, nrows); break;
  }
}

// ---------------------------------------------------------------------------------------
// staged (non-zero-copy) mode: the row copies zero-copy removes
// ---------------------------------------------------------------------------------------
// EPILOGUE: recv[dst_row[t,k]] = stage[t*K + k]  (staging buffer -> final rows)
// PROLOGUE: stage[t*K + k] = y[dst_row[t,k]]     (final rows -> staging buffer)
// The dispatch kernel's shape and residency, so that the baseline is as well built as the
// path it is compared with: one single-wave workgroup per (token, 2 KB chunk); for each
// group of up to 8 of the token's rows, every load, one wait, then the non-temporal
// stores back to back.
template <int KT, bool EPILOGUE>
__global__ __launch_bounds__(kWave) void copy_rows_kernel(const int32_t* __restrict__ dst,
                                                          const u32x4* __restrict__ src,
                                                          u32x4* __restrict__ out, int Krt,
                                                          int nvec, int nch, int nrows) {
  const int K = KT > 0 ? KT : Krt;
  const int64_t t = blockIdx.x / nch;
  const int c0 = (int)(blockIdx.x - t * nch) * kDispChunk + (int)threadIdx.x;
  const int32_t* d = dst + t * K;
  constexpr int G = KT > 0 && KT < 8 ? KT : 8;
  for (int k0 = 0; k0 < K; k0 += G) {
    int64_t srow[G], drow[G];
    bool ok[G];
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const int k = k0 + j;
      const int r = k < K ? d[k] : -1;
      ok[j] = (unsigned)r < (unsigned)nrows;          // -1: unmapped, or past K
      srow[j] = EPILOGUE ? t * K + k : r;
      drow[j] = EPILOGUE ? r : t * K + k;
    }
    u32x4 buf[G][kDispU];
#pragma unroll
    for (int j = 0; j < G; ++j)
#pragma unroll
      for (int u = 0; u < kDispU; ++u) {
        const int v = c0 + u * kWave;
        if (ok[j] && v < nvec) buf[j][u] = src[srow[j] * nvec + v];
      }
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
#pragma unroll
    for (int j = 0; j < G; ++j)
#pragma unroll
      for (int u = 0; u < kDispU; ++u) {
        const int v = c0 + u * kWave;
        if (ok[j] && v < nvec) __builtin_nontemporal_store(buf[j][u], out + drow[j] * nvec + v);
      }
  }
}

template <int KT, bool EPILOGUE>
void launch_copy_rows_k(const moonep_sizes& s, const int32_t* dst, const uint16_t* src,
                        uint16_t* out, int nvec, int nch, hipStream_t st) {
  hipLaunchKernelGGL((copy_rows_kernel<KT, EPILOGUE>), dim3((unsigned)(s.T * nch)), dim3(kWave),
                     kDispLdsBytes, st, dst, reinterpret_cast<const u32x4*>(src),
                     reinterpret_cast<u32x4*>(out), s.K, nvec, nch, (int)s.recv_rows);
}

template <bool EPILOGUE>
void launch_copy_rows(const moonep_sizes& s, const int32_t* dst, const uint16_t* src, uint16_t* out,
                      int nvec, hipStream_t st) {
  const int nch = (nvec + kDispChunk - 1) / kDispChunk;
  switch (s.K) {
    case 1: launch_copy_rows_k<1, EPILOGUE>(s, dst, src, out, nvec, nch, st); break;
    case 2: launch_copy_rows_k<2, EPILOGUE>(s, dst, src, out, nvec, nch, st); break;
    case 4: launch_copy_rows_k<4, EPILOGUE>(s, dst, src, out, nvec, nch, st); break;
    case 6: launch_copy_rows_k<6, EPILOGUE>(s, dst, src, out, nvec, nch, st); break;
    case 8: launch_copy_rows_k<8, EPILOGUE>(s, dst, src, out, nvec, nch, st); break;
    default: launch_copy_rows_k<0, EPILOGUE>(s, dst, src, out, nvec, nch, st); break;
  }
}

// ---------------------------------------------------------------------------------------
// replica weight prefetch: slot_w[r_p][slot_p] = home_w[e_p] for every slot piece p
// ---------------------------------------------------------------------------------------
// Persistent grid over (piece, 16 KB chunk) items; the piece count comes from the plan
// header, so the host never waits for the plan.  Fallback pieces own no slot: skipped.
constexpr int kCopyThreads = 256;
constexpr int kCopyU = 4;
constexpr int kCopyChunk = kCopyThreads * kCopyU;     // 16-byte vectors per item

__global__ __launch_bounds__(kCopyThreads) void prefetch_kernel(const int32_t* __restrict__ plan,
                                                                const u32x4* __restrict__ home,
                                                                u32x4* __restrict__ slotw,
                                                                int64_t wv, const moonep_sizes s) {
  const int np = plan[s.o_hdr + H_STATUS] == 0 ? clamp_count(plan[s.o_hdr + H_NPIECES], s.P_max) : 0;
  const int64_t nchunk = (wv + kCopyChunk - 1) / kCopyChunk;
  const int64_t items = (int64_t)np * nchunk;
  const int32_t* pieces = plan + s.o_pieces;
  for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
    const int p = (int)(it / nchunk);
    const int64_t c = it - (int64_t)p * nchunk;
    const int32_t* pc = pieces + (int64_t)p * kPieceInts;
    const int slot = pc[P_SLOT], r = pc[P_R], e = pc[P_E];
    if (slot < 0 || slot >= s.slots || (unsigned)r >= (unsigned)s.R || (unsigned)e >= (unsigned)s.E)
      continue;
    const u32x4* src = home + (int64_t)e * wv;
    u32x4* dstp = slotw + ((int64_t)r * s.slots + slot) * wv;
    u32x4 v[kCopyU];
#pragma unroll
    for (int u = 0; u < kCopyU; ++u) {
      const int64_t i = c * kCopyChunk + u * kCopyThreads + threadIdx.x;
      if (i < wv) v[u] = __builtin_nontemporal_load(src + i);
    }
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);     // then the stores issue back to back
#pragma unroll
    for (int u = 0; u < kCopyU; ++u) {
      const int64_t i = c * kCopyChunk + u * kCopyThreads + threadIdx.x;
      if (i < wv) __builtin_nontemporal_store(v[u], dstp + i);
    }
  }
}

// ---------------------------------------------------------------------------------------
// expert stub: y[row, h] = bf16(recv[row, h] * W[h]) for h < H, with W the weight slab the
// row's group uses (home group: home_w[e]; slot group: the rank's prefetched slot_w copy;
// fallback piece: home_w[e], read across partitions)
// ---------------------------------------------------------------------------------------
// One workgroup per token; each assignment's row and expert come from dst_row and the
// caller's topk_ids, its weight source from the packed expert and piece tables.
__global__ __launch_bounds__(256) void expert_stub_kernel(const int32_t* __restrict__ plan,
                                                          const int32_t* __restrict__ ids,
                                                          const u32x4* __restrict__ recv,
                                                          const u32x4* __restrict__ home,
                                                          const u32x4* __restrict__ slotw,
                                                          int64_t wv, u32x4* __restrict__ y,
                                                          int nvec, const moonep_sizes s) {
  typedef int i32x4 __attribute__((ext_vector_type(4)));
  const int64_t t = blockIdx.x;
  const int32_t* dst = plan + s.o_dst_row;
  const i32x4* xtab = reinterpret_cast<const i32x4*>(plan + s.o_xtab);
  const int32_t* pieces = plan + s.o_pieces;
  const int nrows = (int)s.recv_rows;
  for (int k = 0; k < s.K; ++k) {
    const int row = dst[t * s.K + k];
    const int e = ids[t * s.K + k];
    if ((unsigned)row >= (unsigned)nrows || (unsigned)e >= (unsigned)s.E) continue;
    const i32x4 xt = xtab[e];                    // keep, home row, first piece, count
    const u32x4* w = home + (int64_t)e * wv;     // home group, or fallback (remote read)
    if (row < xt.y || row >= xt.y + xt.x) {
      int q0, q1;
      piece_range(xt.z, xt.w, s.P_max, &q0, &q1);
      for (int q = q0; q < q1; ++q) {
        const int32_t* pc = pieces + (int64_t)q * kPieceInts;
        if (row >= pc[P_ROW0] && row < pc[P_ROW0] + pc[P_CNT]) {
          if (pc[P_SLOT] >= 0 && pc[P_SLOT] < s.slots && (unsigned)pc[P_R] < (unsigned)s.R)
            w = slotw + ((int64_t)pc[P_R] * s.slots + pc[P_SLOT]) * wv;
          break;
        }
      }
    }
    const u32x4* src = recv + (int64_t)row * nvec;
    u32x4* out = y + (int64_t)row * nvec;
    for (int v = threadIdx.x; v < nvec; v += blockDim.x) {
      const u32x4 a = src[v], b = w[v];
      u32x4 o;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float lo = bf_lo(a[q]) * bf_lo(b[q]);
        const float hi = bf_hi(a[q]) * bf_hi(b[q]);
        o[q] = to_bf16(lo) | (to_bf16(hi) << 16);
      }
      out[v] = o;
    }
  }
}

// ---------------------------------------------------------------------------------------
// reduce: home[e] += rep[r_p][slot_p] for each slot piece p of e, in creation order
// ---------------------------------------------------------------------------------------
// A persistent grid walks (expert with replicas, chunk) items; the item count lives on
// the device (plan header), so the host never waits for the plan.
constexpr int kRedThreads = 256;
constexpr int kRedU = 4;                       // float4 per thread per item
constexpr int kRedChunk = kRedThreads * kRedU; // float4 per item

__global__ __launch_bounds__(kRedThreads) void reduce_kernel(const int32_t* __restrict__ plan,
                                                             f32x4* __restrict__ home,
                                                             const f32x4* __restrict__ rep,
                                                             int64_t g4, const moonep_sizes s) {
  const int nred = plan[s.o_hdr + H_STATUS] == 0 ? clamp_count(plan[s.o_hdr + H_NRED], s.E) : 0;
  const int64_t nchunk = (g4 + kRedChunk - 1) / kRedChunk;
  const int64_t items = (int64_t)nred * nchunk;
  const int32_t* red = plan + s.o_red;
  const int32_t* pieces = plan + s.o_pieces;
  for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
    const int ri = (int)(it / nchunk);
    const int64_t c = it - (int64_t)ri * nchunk;
    const int e = red[ri];
    if ((unsigned)e >= (unsigned)s.E) continue;
    int q0, q1;
    piece_range(plan[s.o_pfirst + e], plan[s.o_pnum + e], s.P_max, &q0, &q1);
    f32x4* h = home + (int64_t)e * g4;
    f32x4 acc[kRedU];
#pragma unroll
    for (int u = 0; u < kRedU; ++u) {
      const int64_t v = c * kRedChunk + u * kRedThreads + threadIdx.x;
      acc[u] = v < g4 ? h[v] : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    for (int q = q0; q < q1; ++q) {
      const int slot = pieces[(int64_t)q * kPieceInts + P_SLOT];
      if (slot < 0) break;                 // an expert's fallback pieces come last
      const int r = pieces[(int64_t)q * kPieceInts + P_R];
      if (slot >= s.slots || (unsigned)r >= (unsigned)s.R) break;
      const f32x4* src = rep + ((int64_t)r * s.slots + slot) * g4;
#pragma unroll
      for (int u = 0; u < kRedU; ++u) {
        const int64_t v = c * kRedChunk + u * kRedThreads + threadIdx.x;
        if (v < g4) acc[u] = acc[u] + __builtin_nontemporal_load(src + v);
      }
    }
#pragma unroll
    for (int u = 0; u < kRedU; ++u) {
      const int64_t v = c * kRedChunk + u * kRedThreads + threadIdx.x;
      if (v < g4) h[v] = acc[u];
    }
  }
}


template <int KT, bool STAGED>
void launch_dispatch_k(const moonep_sizes& s, const int32_t* dst, int nrows, const uint16_t* x,
                       uint16_t* recv, int nvec, int nch, hipStream_t st) {
  hipLaunchKernelGGL((dispatch_kernel<KT, STAGED>), dim3((unsigned)(s.T * nch)), dim3(kWave),
                     kDispLdsBytes, st,
                     dst, reinterpret_cast<const u32x4*>(x), reinterpret_cast<u32x4*>(recv), s.K, nvec,
                     nch, nrows);
}

template <bool STAGED>
void dispatch_rows(const moonep_sizes& s, const int32_t* dst, int nrows, const uint16_t* x, int H,
                   uint16_t* recv, hipStream_t st) {
  const int nvec = H / 8;
  const int nch = (nvec + kDispChunk - 1) / kDispChunk;
  switch (s.K) {
    case 1: launch_dispatch_k<1, STAGED>(s, dst, nrows, x, recv, nvec, nch, st); break;
    case 2: launch_dispatch_k<2, STAGED>(s, dst, nrows, x, recv, nvec, nch, st); break;
    case 4: launch_dispatch_k<4, STAGED>(s, dst, nrows, x, recv, nvec, nch, st); break;
    case 6: launch_dispatch_k<6, STAGED>(s, dst, nrows, x, recv, nvec, nch, st); break;
    case 8: launch_dispatch_k<8, STAGED>(s, dst, nrows, x, recv, nvec, nch, st); break;
    default: launch_dispatch_k<0, STAGED>(s, dst, nrows, x, recv, nvec, nch, st); break;
  }
}

template <int KT, bool WEIGHTED, bool STAGED>
void launch_combine_k(const moonep_sizes& s, const int32_t* dst, const float* w, const uint16_t* y,
                      uint16_t* out, int nvec, int nch, hipStream_t st) {
  // the rows gathered: the receive-shaped buffer, or the [T*K, H] staging buffer
  const int64_t src_bytes = (STAGED ? s.A : s.recv_rows) * (int64_t)nvec * 16;
  const int lds = src_bytes > kLastLevelCacheBytes ? kCombLdsBytes : 0;
  hipLaunchKernelGGL((combine_kernel<KT, WEIGHTED, STAGED>), dim3((unsigned)(s.T * nch)), dim3(kWave),
                     lds, st, dst, w, reinterpret_cast<const u32x4*>(y), reinterpret_cast<u32x4*>(out),
                     s.K, nvec, nch, (int)s.recv_rows);
}

template <bool WEIGHTED, bool STAGED>
void gather_sum(const moonep_sizes& s, const int32_t* plan, const uint16_t* y, int H, uint16_t* out,
                hipStream_t st) {
  const int nvec = H / 8;
  const int nch = (nvec + kCombChunk - 1) / kCombChunk;
  const int32_t* dst = plan + s.o_dst_row;
  const float* w = reinterpret_cast<const float*>(plan + s.o_w);
  switch (s.K) {
    case 1: launch_combine_k<1, WEIGHTED, STAGED>(s, dst, w, y, out, nvec, nch, st); break;
    case 2: launch_combine_k<2, WEIGHTED, STAGED>(s, dst, w, y, out, nvec, nch, st); break;
    case 4: launch_combine_k<4, WEIGHTED, STAGED>(s, dst, w, y, out, nvec, nch, st); break;
    case 6: launch_combine_k<6, WEIGHTED, STAGED>(s, dst, w, y, out, nvec, nch, st); break;
    case 8: launch_combine_k<8, WEIGHTED, STAGED>(s, dst, w, y, out, nvec, nch, st); break;
    default: launch_combine_k<0, WEIGHTED, STAGED>(s, dst, w, y, out, nvec, nch, st); break;
  }
}

}  // namespace

bool move_grid_fits(const moonep_sizes& s, int H) {
  const int64_t nvec = H / 8;
  const int64_t nch = (nvec + kCombChunk - 1) / kCombChunk;   // the finer of the two chunkings
  return s.T * nch <= INT32_MAX;
}

hipError_t launch_dispatch(const moonep_sizes& s, const int32_t* plan, const uint16_t* x,
                           int H, uint16_t* recv, hipStream_t st) {
  dispatch_rows<false>(s, plan + s.o_dst_row, (int)s.recv_rows, x, H, recv, st);
  return hipGetLastError();
}

hipError_t launch_dispatch_staged(const moonep_sizes& s, const int32_t* plan, const uint16_t* x,
                                  int H, uint16_t* stage, uint16_t* recv, hipStream_t st) {
  dispatch_rows<true>(s, nullptr, (int)s.A, x, H, stage, st);
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  launch_copy_rows<true>(s, plan + s.o_dst_row, stage, recv, H / 8, st);
  return hipGetLastError();
}

hipError_t launch_combine(const moonep_sizes& s, const int32_t* plan, const uint16_t* y,
                          int H, uint16_t* out, hipStream_t st) {
  gather_sum<true, false>(s, plan, y, H, out, st);
  return hipGetLastError();
}

hipError_t launch_combine_staged(const moonep_sizes& s, const int32_t* plan, const uint16_t* y,
                                 int H, uint16_t* stage, uint16_t* out, hipStream_t st) {
  launch_copy_rows<false>(s, plan + s.o_dst_row, y, stage, H / 8, st);
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  gather_sum<true, true>(s, plan, stage, H, out, st);
  return hipGetLastError();
}

hipError_t launch_dispatch_bwd(const moonep_sizes& s, const int32_t* plan, const uint16_t* g_recv,
                               int H, uint16_t* gx, hipStream_t st) {
  gather_sum<false, false>(s, plan, g_recv, H, gx, st);
  return hipGetLastError();
}

hipError_t launch_combine_bwd(const moonep_sizes& s, const int32_t* plan, const uint16_t* dout,
                              const uint16_t* y, int H, uint16_t* g_y, float* dw,
                              hipStream_t st) {
  const int nvec = H / 8;
  int threads = 64, u = 1;
  row_shape(nvec, 4, 2, &threads, &u);
  const int32_t* dst = plan + s.o_dst_row;
  const float* w = reinterpret_cast<const float*>(plan + s.o_w);
  switch (s.K) {
    case 1: launch_combine_bwd_k<1>(s, dst, w, dout, y, g_y, dw, nvec, threads, u, st); break;
    case 2: launch_combine_bwd_k<2>(s, dst, w, dout, y, g_y, dw, nvec, threads, u, st); break;
    case 4: launch_combine_bwd_k<4>(s, dst, w, dout, y, g_y, dw, nvec, threads, u, st); break;
    case 6: launch_combine_bwd_k<6>(s, dst, w, dout, y, g_y, dw, nvec, threads, u, st); break;
    case 8: launch_combine_bwd_k<8>(s, dst, w, dout, y, g_y, dw, nvec, threads, u, st); break;
    default: launch_combine_bwd_k<MOONEP_MAX_K>(s, dst, w, dout, y, g_y, dw, nvec, threads, u, st); break;
  }
  return hipGetLastError();
}

hipError_t launch_prefetch(const moonep_sizes& s, const int32_t* plan, const uint16_t* home_w,
                           int64_t W_el, uint16_t* slot_w, hipStream_t st) {
  hipLaunchKernelGGL(prefetch_kernel, dim3(2048), dim3(kCopyThreads), 0, st, plan,
                     reinterpret_cast<const u32x4*>(home_w), reinterpret_cast<u32x4*>(slot_w),
                     W_el / 8, s);
  return hipGetLastError();
}

hipError_t launch_expert_stub(const moonep_sizes& s, const int32_t* plan, const int32_t* ids,
                              const uint16_t* recv, const uint16_t* home_w,
                              const uint16_t* slot_w, int64_t W_el, int H, uint16_t* y,
                              hipStream_t st) {
  hipLaunchKernelGGL(expert_stub_kernel, dim3((unsigned)s.T), dim3(256), 0, st, plan, ids,
                     reinterpret_cast<const u32x4*>(recv), reinterpret_cast<const u32x4*>(home_w),
                     reinterpret_cast<const u32x4*>(slot_w), W_el / 8,
                     reinterpret_cast<u32x4*>(y), H / 8, s);
  return hipGetLastError();
}

hipError_t launch_reduce(const moonep_sizes& s, const int32_t* plan, float* home,
                         const float* rep, int64_t G_el, hipStream_t st) {
  const int64_t g4 = G_el / 4;
  hipLaunchKernelGGL(reduce_kernel, dim3(2048), dim3(kRedThreads), 0, st, plan,
                     reinterpret_cast<f32x4*>(home), reinterpret_cast<const f32x4*>(rep), g4,
                     s);
  return hipGetLastError();
}

}  // namespace moonep
