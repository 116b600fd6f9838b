// Plain 16-byte memory streams: the ceilings the hot path's kernels are measured against
// (declared in moonep_streams.h).  Not part of the hot path.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moonep_streams.h"

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kEInval = -1, kEHip = -4;

// s_waitcnt vmcnt(0) in the gfx9 encoding, with expcnt and lgkmcnt left at their maximum
constexpr int kWaitVmcnt0 = 0x0F70;

// The row streams use the hot path kernels' residency caps (dynamic LDS they never touch,
// so that at most floor(160 KB / request) single-wave workgroups sit on a CU): 5 per CU
// for the fan-out, 9 per CU for the gather when its source exceeds the 256 MB last-level
// cache.
constexpr int kFanoutLdsBytes = 29 * 1024;
constexpr int kGatherLdsBytes = 17 * 1024;
constexpr int64_t kLastLevelCacheBytes = 256ll << 20;

template <int POL>
__device__ __forceinline__ u32x4 load16(const u32x4* p) {
  if constexpr (POL == 1) return __builtin_nontemporal_load(p); else return *p;
}
template <int POL>
__device__ __forceinline__ void store16(u32x4* p, u32x4 v) {
  if constexpr (POL == 1) __builtin_nontemporal_store(v, p); else *p = v;
}

// A pattern the XOR of real data never equals in practice; the store behind it keeps the
// loads alive.
__device__ __forceinline__ bool unlikely_pattern(u32x4 a) {
  return a.x == 0x9E3779B9u && a.y == 0x7F4A7C15u && a.z == 0x94D049BBu && a.w == 0x2545F491u;
}

// One workgroup per blockDim*U vectors: U = 2 with 64 lanes (2 KB) or U = 1 with 256 lanes
// (4 KB), each lane's vectors blockDim apart.
template <int U, int POL>
__global__ __launch_bounds__(256) void read_kernel(const u32x4* __restrict__ src, int64_t nvec,
                                                   u32x4* sink) {
  const int64_t base = (int64_t)blockIdx.x * blockDim.x * U + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t v = base + (int64_t)u * blockDim.x;
    if (v < nvec) acc ^= load16<POL>(src + v);
  }
  if (unlikely_pattern(acc)) sink[0] = acc;
}

template <int U, int POL>
__global__ __launch_bounds__(256) void write_kernel(u32x4* __restrict__ dst, int64_t nvec) {
  const int64_t base = (int64_t)blockIdx.x * blockDim.x * U + threadIdx.x;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t v = base + (int64_t)u * blockDim.x;
    if (v < nvec) store16<POL>(dst + v, u32x4{(unsigned)v, 0x5A5A5A5Au, 0x3C3C3C3Cu, 0u});
  }
}

template <int U, int POL>
__global__ __launch_bounds__(256) void copy_kernel(const u32x4* __restrict__ src,
                                                   u32x4* __restrict__ dst, int64_t nvec) {
  const int64_t base = (int64_t)blockIdx.x * blockDim.x * U + threadIdx.x;
  u32x4 b[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t v = base + (int64_t)u * blockDim.x;
    if (v < nvec) b[u] = load16<POL>(src + v);
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t v = base + (int64_t)u * blockDim.x;
    if (v < nvec) store16<POL>(dst + v, b[u]);
  }
}

// dispatch's mix: one wave per (source row, 128-vector chunk), the dispatch kernel's
// shape: the row indices and the two loads first, one wait for the loads (without it the
// compiler waits for every earlier store before each store: vmcnt counts both), then the
// stores back to back
__global__ __launch_bounds__(64) void fanout_kernel(const int32_t* __restrict__ rows,
                                                    const u32x4* __restrict__ src,
                                                    u32x4* __restrict__ dst, int K, int nvec,
                                                    int nch, int64_t dst_rows, int read_src) {
  const int64_t i = blockIdx.x / nch;
  const int c0 = (int)(blockIdx.x - i * nch) * 128 + (int)threadIdx.x;
  u32x4 b[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int v = c0 + u * 64;
    if (v < nvec)
      b[u] = read_src ? src[i * nvec + v] : u32x4{(unsigned)i, (unsigned)v, 0x77777777u, 1u};
  }
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  for (int k0 = 0; k0 < K; k0 += 8) {
    int64_t r[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) r[j] = k0 + j < K ? rows[i * K + k0 + j] : -1;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int v = c0 + u * 64;
      if (v >= nvec) continue;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (r[j] >= 0 && r[j] < dst_rows) __builtin_nontemporal_store(b[u], dst + r[j] * nvec + v);
    }
  }
}

// combine's mix: one wave per (destination row, 64-vector chunk); the K loads are issued
// eight at a time before they are combined
__global__ __launch_bounds__(64) void gather_kernel(const int32_t* __restrict__ rows,
                                                    const u32x4* __restrict__ src, int64_t src_rows,
                                                    u32x4* __restrict__ dst, int K, int nvec,
                                                    int nch, int write_dst) {
  const int64_t i = blockIdx.x / nch;
  const int v = (int)(blockIdx.x - i * nch) * 64 + (int)threadIdx.x;
  if (v >= nvec) return;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int k0 = 0; k0 < K; k0 += 8) {
    u32x4 y[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t r = k0 + j < K ? rows[i * K + k0 + j] : -1;
      y[j] = (r >= 0 && r < src_rows) ? __builtin_nontemporal_load(src + r * nvec + v)
                                      : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) acc ^= y[j];
  }
  if (write_dst || unlikely_pattern(acc)) __builtin_nontemporal_store(acc, dst + i * nvec + v);
}

// the combine backward's mix: one workgroup per source row i, its threads holding two
// vectors of row i and taking its K listed rows in groups of up to 8: every load of the
// group, one wait, then the group's stores
__global__ __launch_bounds__(1024) void update_kernel(const int32_t* __restrict__ rows,
                                                      const u32x4* __restrict__ src,
                                                      const u32x4* __restrict__ a,
                                                      u32x4* __restrict__ b, int K, int nvec,
                                                      int64_t rows_ab) {
  const int64_t i = blockIdx.x;
  for (int v0 = threadIdx.x; v0 < nvec; v0 += blockDim.x * 2) {
    u32x4 sv[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int v = v0 + u * blockDim.x;
      sv[u] = v < nvec ? src[i * nvec + v] : u32x4{0u, 0u, 0u, 0u};
    }
    for (int k0 = 0; k0 < K; k0 += 8) {
      int64_t r[8];
      u32x4 y[8][2];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        r[j] = k0 + j < K ? rows[i * K + k0 + j] : -1;
        if (r[j] >= rows_ab) r[j] = -1;
      }
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int v = v0 + u * blockDim.x;
          y[j][u] = r[j] >= 0 && v < nvec ? __builtin_nontemporal_load(a + r[j] * nvec + v)
                                          : u32x4{0u, 0u, 0u, 0u};
        }
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int v = v0 + u * blockDim.x;
          if (r[j] >= 0 && v < nvec) __builtin_nontemporal_store(y[j][u] ^ sv[u], b + r[j] * nvec + v);
        }
    }
  }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

int status() { return hipGetLastError() == hipSuccess ? 0 : kEHip; }

// grid of one linear stream: workgroups of `threads` lanes x U vectors
bool linear_grid(int64_t nbytes, int shape, int64_t* nvec, unsigned* grid, int* threads) {
  if (nbytes <= 0 || nbytes % 16 != 0) return false;
  if (shape != MOONEP_SHAPE_WAVE_2K && shape != MOONEP_SHAPE_BLOCK_4K) return false;
  *nvec = nbytes / 16;
  *threads = shape == MOONEP_SHAPE_WAVE_2K ? 64 : 256;
  const int64_t per = shape == MOONEP_SHAPE_WAVE_2K ? 128 : 256;
  const int64_t g = (*nvec + per - 1) / per;
  if (g > INT32_MAX) return false;
  *grid = (unsigned)g;
  return true;
}

}  // namespace

extern "C" {

int moonep_stream_read(const void* src, int64_t nbytes, int shape, int policy, void* sink,
                       hipStream_t stream) {
  int64_t nvec;
  unsigned grid;
  int threads;
  if (!src || !sink || !aligned16(src) || !aligned16(sink) || (policy != 0 && policy != 1) ||
      !linear_grid(nbytes, shape, &nvec, &grid, &threads))
    return kEInval;
  (void)hipGetLastError();
  const u32x4* s = static_cast<const u32x4*>(src);
  u32x4* k = static_cast<u32x4*>(sink);
  if (shape == MOONEP_SHAPE_WAVE_2K) {
    if (policy) hipLaunchKernelGGL((read_kernel<2, 1>), dim3(grid), dim3(threads), 0, stream, s, nvec, k);
    else hipLaunchKernelGGL((read_kernel<2, 0>), dim3(grid), dim3(threads), 0, stream, s, nvec, k);
  } else {
    if (policy) hipLaunchKernelGGL((read_kernel<1, 1>), dim3(grid), dim3(threads), 0, stream, s, nvec, k);
    else hipLaunchKernelGGL((read_kernel<1, 0>), dim3(grid), dim3(threads), 0, stream, s, nvec, k);
  }
  return status();
}

int moonep_stream_write(void* dst, int64_t nbytes, int shape, int policy, hipStream_t stream) {
  int64_t nvec;
  unsigned grid;
  int threads;
  if (!dst || !aligned16(dst) || (policy != 0 && policy != 1) ||
      !linear_grid(nbytes, shape, &nvec, &grid, &threads))
    return kEInval;
  (void)hipGetLastError();
  u32x4* d = static_cast<u32x4*>(dst);
  if (shape == MOONEP_SHAPE_WAVE_2K) {
    if (policy) hipLaunchKernelGGL((write_kernel<2, 1>), dim3(grid), dim3(threads), 0, stream, d, nvec);
    else hipLaunchKernelGGL((write_kernel<2, 0>), dim3(grid), dim3(threads), 0, stream, d, nvec);
  } else {
    if (policy) hipLaunchKernelGGL((write_kernel<1, 1>), dim3(grid), dim3(threads), 0, stream, d, nvec);
    else hipLaunchKernelGGL((write_kernel<1, 0>), dim3(grid), dim3(threads), 0, stream, d, nvec);
  }
  return status();
}

int moonep_stream_copy(const void* src, void* dst, int64_t nbytes, int shape, int policy,
                       hipStream_t stream) {
  int64_t nvec;
  unsigned grid;
  int threads;
  if (!src || !dst || !aligned16(src) || !aligned16(dst) || (policy != 0 && policy != 1) ||
      !linear_grid(nbytes, shape, &nvec, &grid, &threads))
    return kEInval;
  (void)hipGetLastError();
  const u32x4* s = static_cast<const u32x4*>(src);
  u32x4* d = static_cast<u32x4*>(dst);
  if (shape == MOONEP_SHAPE_WAVE_2K) {
    if (policy) hipLaunchKernelGGL((copy_kernel<2, 1>), dim3(grid), dim3(threads), 0, stream, s, d, nvec);
    else hipLaunchKernelGGL((copy_kernel<2, 0>), dim3(grid), dim3(threads), 0, stream, s, d, nvec);
  } else {
    if (policy) hipLaunchKernelGGL((copy_kernel<1, 1>), dim3(grid), dim3(threads), 0, stream, s, d, nvec);
    else hipLaunchKernelGGL((copy_kernel<1, 0>), dim3(grid), dim3(threads), 0, stream, s, d, nvec);
  }
  return status();
}

int moonep_rows_fanout(const int32_t* rows, int64_t n, int K, const void* src, void* dst,
                       int64_t dst_rows, int row_bytes, int read_src, hipStream_t stream) {
  if (!rows || !dst || (read_src && !src) || n <= 0 || K < 1 || dst_rows <= 0 || row_bytes <= 0 ||
      row_bytes % 16 != 0 || !aligned16(dst) || (src && !aligned16(src)))
    return kEInval;
  const int nvec = row_bytes / 16;
  const int nch = (nvec + 127) / 128;
  if (n * nch > INT32_MAX) return kEInval;
  (void)hipGetLastError();
  hipLaunchKernelGGL(fanout_kernel, dim3((unsigned)(n * nch)), dim3(64), kFanoutLdsBytes, stream,
                     rows, static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), K, nvec, nch,
                     dst_rows, read_src);
  return status();
}

int moonep_rows_gather(const int32_t* rows, int64_t n, int K, const void* src, int64_t src_rows,
                       void* dst, int row_bytes, int write_dst, hipStream_t stream) {
  if (!rows || !src || !dst || n <= 0 || K < 1 || src_rows <= 0 || row_bytes <= 0 ||
      row_bytes % 16 != 0 || !aligned16(dst) || !aligned16(src))
    return kEInval;
  const int nvec = row_bytes / 16;
  const int nch = (nvec + 63) / 64;
  if (n * nch > INT32_MAX) return kEInval;
  (void)hipGetLastError();
  const int lds = src_rows * (int64_t)row_bytes > kLastLevelCacheBytes ? kGatherLdsBytes : 0;
  hipLaunchKernelGGL(gather_kernel, dim3((unsigned)(n * nch)), dim3(64), lds, stream, rows,
                     static_cast<const u32x4*>(src), src_rows, static_cast<u32x4*>(dst), K, nvec,
                     nch, write_dst);
  return status();
}

int moonep_rows_update(const int32_t* rows, int64_t n, int K, const void* src, const void* a,
                       void* b, int64_t rows_ab, int row_bytes, hipStream_t stream) {
  if (!rows || !src || !a || !b || n <= 0 || K < 1 || rows_ab <= 0 || row_bytes <= 0 ||
      row_bytes % 16 != 0 || !aligned16(src) || !aligned16(a) || !aligned16(b) || n > INT32_MAX)
    return kEInval;
  const int nvec = row_bytes / 16;
  const int half = (nvec + 1) / 2;
  const int threads = half >= 1024 ? 1024 : (half + 63) / 64 * 64;
  (void)hipGetLastError();
  hipLaunchKernelGGL(update_kernel, dim3((unsigned)n), dim3(threads), 0, stream, rows,
                     static_cast<const u32x4*>(src), static_cast<const u32x4*>(a),
                     static_cast<u32x4*>(b), K, nvec, rows_ab);
  return status();
}

}  // extern "C"
