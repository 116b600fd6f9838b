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

constexpr int64_t kLastLevelCacheBytes = 256ll << 20;   // MI355X Infinity Cache

__device__ __forceinline__ float bf_lo(unsigned int v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf_hi(unsigned int v) { return __uint_as_float(v & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even; NaN -> 0x7FC0.
__device__ __forceinline__ unsigned int to_bf16(float f) {
  const unsigned int u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
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
// One workgroup per token: each thread loads U vectors of the row, then stores each of
// them to the token's K destination rows in turn.  Measured on MI355X: storing one
// vector to all K rows before the next is about 1.5% faster than writing the rows one
// after another, and non-temporal loads of x are 2% slower.  Stores: when the whole
// destination buffer fits the 256 MB last-level cache, plain stores leave it dirty there
// and the next kernel pays for the write-back (a combine reading it right after took 45%
// longer), so the stores are non-temporal (NTS); for larger buffers non-temporal stores
// are 5-8% slower and plain stores are used.
// KT = K when K is a compile-time constant (the rows are then held in registers), else 0.
template <int KT, int U, bool NTS>
__global__ __launch_bounds__(1024) void dispatch_kernel(const int32_t* __restrict__ dst,
                                                       const u32x4* __restrict__ x,
                                                       u32x4* __restrict__ recv, int Krt,
                                                       int nvec, int nrows) {
  const int K = KT > 0 ? KT : Krt;
  const int64_t t = blockIdx.x;
  const int32_t* d = dst ? dst + t * K : nullptr;   // null: staging row t*K + k
  const u32x4* src = x + t * nvec;
  const int step = blockDim.x * U;
  if constexpr (KT > 0) {
    int rows[KT];
#pragma unroll
    for (int k = 0; k < KT; ++k) rows[k] = d ? d[k] : (int)(t * K + k);
    for (int v0 = threadIdx.x; v0 < nvec; v0 += step) {
      u32x4 buf[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int v = v0 + u * blockDim.x;
        if (v < nvec) buf[u] = src[v];
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int v = v0 + u * blockDim.x;
        if (v < nvec) {
#pragma unroll
          for (int k = 0; k < KT; ++k)
            if ((unsigned)rows[k] < (unsigned)nrows) {    // -1: unmapped
              u32x4* o = recv + (int64_t)rows[k] * nvec + v;
              if constexpr (NTS) __builtin_nontemporal_store(buf[u], o); else *o = buf[u];
            }
        }
      }
    }
  } else {
    for (int v0 = threadIdx.x; v0 < nvec; v0 += step) {
      u32x4 buf[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int v = v0 + u * blockDim.x;
        if (v < nvec) buf[u] = src[v];
      }
      for (int k = 0; k < K; ++k) {
        const int row = d ? d[k] : (int)(t * K + k);
        if ((unsigned)row >= (unsigned)nrows) continue;   // -1: unmapped
        u32x4* o = recv + (int64_t)row * nvec;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int v = v0 + u * blockDim.x;
          if (v < nvec) {
            if constexpr (NTS) __builtin_nontemporal_store(buf[u], o + v); else o[v] = buf[u];
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------------------
// combine: out[t] = bf16( sum_k w[t,k] * y[dst_row[t,k]] ), fp32, k ascending, no FMA
// ---------------------------------------------------------------------------------------
// acc += w * y[row, v0 + u*blockDim.x] for the thread's U vectors (8 bf16 each): a
// separate fp32 multiply and add per element, in the caller's k order.  The rows are
// read with non-temporal loads (about 9% faster than plain loads), and the output row is
// written with a non-temporal store.
template <int U, bool WEIGHTED>
__device__ __forceinline__ void combine_accumulate(float (&acc)[U][8], const u32x4* __restrict__ y,
                                                   int row, float wk, int v0, int nvec,
                                                   int nrows) {
  if ((unsigned)row >= (unsigned)nrows) return;    // -1: unmapped
  const u32x4* src = y + (int64_t)row * nvec;
  u32x4 yv[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int v = v0 + u * blockDim.x;
    yv[u] = v < nvec ? __builtin_nontemporal_load(src + v) : u32x4{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const unsigned int bits = yv[u][q];
      const float p0 = WEIGHTED ? wk * bf_lo(bits) : bf_lo(bits);
      const float p1 = WEIGHTED ? wk * bf_hi(bits) : bf_hi(bits);
      acc[u][2 * q] = acc[u][2 * q] + p0;
      acc[u][2 * q + 1] = acc[u][2 * q + 1] + p1;
    }
  }
}

// WEIGHTED = false is the gradient of dispatch: gx[t] = bf16(sum_k g_recv[dst_row[t,k]]).
template <int KT, int U, bool WEIGHTED>
__global__ __launch_bounds__(1024) void combine_kernel(const int32_t* __restrict__ dst,
                                                      const float* __restrict__ wts,
                                                      const u32x4* __restrict__ y,
                                                      u32x4* __restrict__ out, int Krt,
                                                      int nvec, int nrows) {
  const int K = KT > 0 ? KT : Krt;
  const int64_t t = blockIdx.x;
  const int32_t* d = dst ? dst + t * K : nullptr;   // null: staging row t*K + k
  const float* wt = wts + t * K;
  const int step = blockDim.x * U;
  for (int v0 = threadIdx.x; v0 < nvec; v0 += step) {
    float acc[U][8];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[u][j] = 0.f;
    if constexpr (KT > 0) {
#pragma unroll
      for (int k = 0; k < KT; ++k)
        combine_accumulate<U, WEIGHTED>(acc, y, d ? d[k] : (int)(t * K + k),
                                        WEIGHTED ? wt[k] : 1.f, v0, nvec, nrows);
    } else {
      for (int k = 0; k < K; ++k)
        combine_accumulate<U, WEIGHTED>(acc, y, d ? d[k] : (int)(t * K + k),
                                        WEIGHTED ? wt[k] : 1.f, v0, nvec, nrows);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int v = v0 + u * blockDim.x;
      if (v < nvec) {
        u32x4 o;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          o[q] = to_bf16(acc[u][2 * q]) | (to_bf16(acc[u][2 * q + 1]) << 16);
        __builtin_nontemporal_store(o, out + t * nvec + v);
      }
    }
  }
}

// ---------------------------------------------------------------------------------------
// combine backward: g_y[dst_row[t,k]] = bf16(w[t,k] * dout[t]);
//                   dw[t,k] = sum_h dout[t,h] * y[dst_row[t,k],h]   (fp32, fused multiply-add)
// ---------------------------------------------------------------------------------------
// One workgroup per token.  Each thread holds U vectors of dout, reads the same vectors of
// each of the K rows of y, keeps K partial dot products, and writes the scaled dout
// vectors to the K rows of g_y (g_y may be y itself: each element is read before it is
// written by the same thread).  The K partials are summed over the wave with lane
// shuffles, then over the waves in LDS.  KMAX = K when K is a compile-time
// constant, else MOONEP_MAX_K with the loop bounded by the runtime K.
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
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
      if (k >= K) break;
      const int row = d[k];
      if ((unsigned)row >= (unsigned)nrows) continue;     // -1: unmapped
      const float wk = wt[k];
      const u32x4* ysrc = y + (int64_t)row * nvec;
      u32x4* gdst = g_y + (int64_t)row * nvec;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int v = v0 + u * blockDim.x;
        if (v < nvec) {
          const u32x4 yv = __builtin_nontemporal_load(ysrc + v);
          u32x4 g;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float d0 = bf_lo(dv[u][q]), d1 = bf_hi(dv[u][q]);
            part[k] = __builtin_fmaf(d0, bf_lo(yv[q]), part[k]);
            part[k] = __builtin_fmaf(d1, bf_hi(yv[q]), part[k]);
            const float g0 = wk * d0;
            const float g1 = wk * d1;
            g[q] = to_bf16(g0) | (to_bf16(g1) << 16);
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
template <int U, bool EPILOGUE>
__global__ __launch_bounds__(1024) void copy_rows_kernel(const int32_t* __restrict__ dst,
                                                         const u32x4* __restrict__ src,
                                                         u32x4* __restrict__ out, int K,
                                                         int nvec, int nrows) {
  const int64_t t = blockIdx.x;
  const int32_t* d = dst + t * K;
  for (int k = 0; k < K; ++k) {
    const int r = d[k];
    if ((unsigned)r >= (unsigned)nrows) continue;      // -1: unmapped
    const int64_t srow = EPILOGUE ? t * K + k : r;
    const int64_t drow = EPILOGUE ? r : t * K + k;
    const u32x4* sp = src + srow * nvec;
    u32x4* op = out + drow * nvec;
    for (int v0 = threadIdx.x; v0 < nvec; v0 += blockDim.x * U) {
      u32x4 buf[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int v = v0 + u * blockDim.x;
        if (v < nvec) buf[u] = sp[v];
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int v = v0 + u * blockDim.x;
        if (v < nvec) op[v] = buf[u];
      }
    }
  }
}

template <bool EPILOGUE>
void launch_copy_rows(const moonep_sizes& s, const int32_t* dst, const uint16_t* src, uint16_t* out,
                      int nvec, hipStream_t st) {
  int threads = 64, u = 1;
  row_shape(nvec, 8, 7, &threads, &u);
  const dim3 grid((unsigned)s.T), block(threads);
  const u32x4* sv = reinterpret_cast<const u32x4*>(src);
  u32x4* ov = reinterpret_cast<u32x4*>(out);
  const int nrows = (int)s.recv_rows;
  switch (u) {
    case 1: hipLaunchKernelGGL((copy_rows_kernel<1, EPILOGUE>), grid, block, 0, st, dst, sv, ov, s.K, nvec, nrows); break;
    case 2: hipLaunchKernelGGL((copy_rows_kernel<2, EPILOGUE>), grid, block, 0, st, dst, sv, ov, s.K, nvec, nrows); break;
    case 3: hipLaunchKernelGGL((copy_rows_kernel<3, EPILOGUE>), grid, block, 0, st, dst, sv, ov, s.K, nvec, nrows); break;
    case 4: hipLaunchKernelGGL((copy_rows_kernel<4, EPILOGUE>), grid, block, 0, st, dst, sv, ov, s.K, nvec, nrows); break;
    case 5: hipLaunchKernelGGL((copy_rows_kernel<5, EPILOGUE>), grid, block, 0, st, dst, sv, ov, s.K, nvec, nrows); break;
    case 6: hipLaunchKernelGGL((copy_rows_kernel<6, EPILOGUE>), grid, block, 0, st, dst, sv, ov, s.K, nvec, nrows); break;
    case 7: hipLaunchKernelGGL((copy_rows_kernel<7, EPILOGUE>), grid, block, 0, st, dst, sv, ov, s.K, nvec, nrows); break;
    default: hipLaunchKernelGGL((copy_rows_kernel<8, EPILOGUE>), grid, block, 0, st, dst, sv, ov, s.K, nvec, nrows); break;
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
  const int np = plan[s.o_hdr + H_STATUS] == 0 ? plan[s.o_hdr + H_NPIECES] : 0;
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
      for (int q = xt.z; q < xt.z + xt.w; ++q) {
        const int32_t* pc = pieces + (int64_t)q * kPieceInts;
        if (row >= pc[P_ROW0] && row < pc[P_ROW0] + pc[P_CNT]) {
          if (pc[P_SLOT] >= 0 && pc[P_SLOT] < s.slots)
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
  const int nred = plan[s.o_hdr + H_STATUS] == 0 ? plan[s.o_hdr + H_NRED] : 0;
  const int64_t nchunk = (g4 + kRedChunk - 1) / kRedChunk;
  const int64_t items = (int64_t)nred * nchunk;
  const int32_t* red = plan + s.o_red;
  const int32_t* pieces = plan + s.o_pieces;
  for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
    const int ri = (int)(it / nchunk);
    const int64_t c = it - (int64_t)ri * nchunk;
    const int e = red[ri];
    if ((unsigned)e >= (unsigned)s.E) continue;
    const int q0 = plan[s.o_pfirst + e];
    const int q1 = q0 + plan[s.o_pnum + e];
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


template <int KT, int U>
void launch_dispatch_ku(const moonep_sizes& s, const int32_t* dst, int nrows, const uint16_t* x,
                        uint16_t* recv, int nvec, int threads, hipStream_t st) {
  const bool fits_llc = (int64_t)nrows * nvec * 16 <= kLastLevelCacheBytes;
  if (fits_llc)
    hipLaunchKernelGGL((dispatch_kernel<KT, U, true>), dim3((unsigned)s.T), dim3(threads), 0, st,
                       dst, reinterpret_cast<const u32x4*>(x), reinterpret_cast<u32x4*>(recv), s.K,
                       nvec, nrows);
  else
    hipLaunchKernelGGL((dispatch_kernel<KT, U, false>), dim3((unsigned)s.T), dim3(threads), 0, st,
                       dst, reinterpret_cast<const u32x4*>(x), reinterpret_cast<u32x4*>(recv), s.K,
                       nvec, nrows);
}

template <int KT>
void launch_dispatch_k(const moonep_sizes& s, const int32_t* dst, int nrows, const uint16_t* x,
                       uint16_t* recv, int nvec, int threads, int u, hipStream_t st) {
  switch (u) {
    case 1: launch_dispatch_ku<KT, 1>(s, dst, nrows, x, recv, nvec, threads, st); break;
    case 2: launch_dispatch_ku<KT, 2>(s, dst, nrows, x, recv, nvec, threads, st); break;
    case 3: launch_dispatch_ku<KT, 3>(s, dst, nrows, x, recv, nvec, threads, st); break;
    default: launch_dispatch_ku<KT, 4>(s, dst, nrows, x, recv, nvec, threads, st); break;
  }
}

template <int KT, int U, bool WEIGHTED>
void launch_combine_ku(const moonep_sizes& s, const int32_t* dst, const float* w,
                       const uint16_t* y, uint16_t* out, int nvec, int threads, hipStream_t st) {
  hipLaunchKernelGGL((combine_kernel<KT, U, WEIGHTED>), dim3((unsigned)s.T), dim3(threads), 0, st, dst,
                     w, reinterpret_cast<const u32x4*>(y), reinterpret_cast<u32x4*>(out), s.K,
                     nvec, dst ? (int)s.recv_rows : (int)s.A);
}

template <int KT, bool WEIGHTED>
void launch_combine_k(const moonep_sizes& s, const int32_t* dst, const float* w,
                      const uint16_t* y, uint16_t* out, int nvec, int threads, int u,
                      hipStream_t st) {
  switch (u) {
    case 1: launch_combine_ku<KT, 1, WEIGHTED>(s, dst, w, y, out, nvec, threads, st); break;
    case 2: launch_combine_ku<KT, 2, WEIGHTED>(s, dst, w, y, out, nvec, threads, st); break;
    case 3: launch_combine_ku<KT, 3, WEIGHTED>(s, dst, w, y, out, nvec, threads, st); break;
    default: launch_combine_ku<KT, 4, WEIGHTED>(s, dst, w, y, out, nvec, threads, st); break;
  }
}

}  // namespace

// rows from the plan's dst_row, or (staged) row t*K + k of a [T*K, H] staging buffer
hipError_t dispatch_rows(const moonep_sizes& s, const int32_t* dst, int nrows, const uint16_t* x,
                         int H, uint16_t* recv, hipStream_t st) {
  const int nvec = H / 8;
  int threads = 64, u = 1;
  row_shape(nvec, 4, 2, &threads, &u);
  switch (s.K) {
    case 1: launch_dispatch_k<1>(s, dst, nrows, x, recv, nvec, threads, u, st); break;
    case 2: launch_dispatch_k<2>(s, dst, nrows, x, recv, nvec, threads, u, st); break;
    case 4: launch_dispatch_k<4>(s, dst, nrows, x, recv, nvec, threads, u, st); break;
    case 6: launch_dispatch_k<6>(s, dst, nrows, x, recv, nvec, threads, u, st); break;
    case 8: launch_dispatch_k<8>(s, dst, nrows, x, recv, nvec, threads, u, st); break;
    default: launch_dispatch_k<0>(s, dst, nrows, x, recv, nvec, threads, u, st); break;
  }
  return hipGetLastError();
}

hipError_t launch_dispatch(const moonep_sizes& s, const int32_t* plan, const uint16_t* x,
                           int H, uint16_t* recv, hipStream_t st) {
  return dispatch_rows(s, plan + s.o_dst_row, (int)s.recv_rows, x, H, recv, st);
}

hipError_t launch_dispatch_staged(const moonep_sizes& s, const int32_t* plan, const uint16_t* x,
                                  int H, uint16_t* stage, uint16_t* recv, hipStream_t st) {
  const hipError_t err = dispatch_rows(s, nullptr, (int)s.A, x, H, stage, st);
  if (err != hipSuccess) return err;
  launch_copy_rows<true>(s, plan + s.o_dst_row, stage, recv, H / 8, st);
  return hipGetLastError();
}

template <bool WEIGHTED>
hipError_t launch_gather_sum(const moonep_sizes& s, const int32_t* plan, const uint16_t* y,
                             int H, uint16_t* out, hipStream_t st, bool staged = false) {
  const int nvec = H / 8;
  int threads = 64, u = 1;
  row_shape(nvec, 4, 2, &threads, &u);
  const int32_t* dst = staged ? nullptr : plan + s.o_dst_row;
  const float* w = reinterpret_cast<const float*>(plan + s.o_w);
  switch (s.K) {
    case 1: launch_combine_k<1, WEIGHTED>(s, dst, w, y, out, nvec, threads, u, st); break;
    case 2: launch_combine_k<2, WEIGHTED>(s, dst, w, y, out, nvec, threads, u, st); break;
    case 4: launch_combine_k<4, WEIGHTED>(s, dst, w, y, out, nvec, threads, u, st); break;
    case 6: launch_combine_k<6, WEIGHTED>(s, dst, w, y, out, nvec, threads, u, st); break;
    case 8: launch_combine_k<8, WEIGHTED>(s, dst, w, y, out, nvec, threads, u, st); break;
    default: launch_combine_k<0, WEIGHTED>(s, dst, w, y, out, nvec, threads, u, st); break;
  }
  return hipGetLastError();
}

hipError_t launch_combine(const moonep_sizes& s, const int32_t* plan, const uint16_t* y,
                          int H, uint16_t* out, hipStream_t st) {
  return launch_gather_sum<true>(s, plan, y, H, out, st);
}

hipError_t launch_combine_staged(const moonep_sizes& s, const int32_t* plan, const uint16_t* y,
                                 int H, uint16_t* stage, uint16_t* out, hipStream_t st) {
  launch_copy_rows<false>(s, plan + s.o_dst_row, y, stage, H / 8, st);
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  return launch_gather_sum<true>(s, plan, stage, H, out, st, true);
}

hipError_t launch_dispatch_bwd(const moonep_sizes& s, const int32_t* plan, const uint16_t* g_recv,
                               int H, uint16_t* gx, hipStream_t st) {
  return launch_gather_sum<false>(s, plan, g_recv, H, gx, st);
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
