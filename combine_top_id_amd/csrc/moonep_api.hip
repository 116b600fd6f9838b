// The C ABI: argument checks, sizes, and the launches on the caller's stream.
#include <cstring>
#include <mutex>

#include "moonep_internal.h"

using namespace moonep;

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_desc(const moonep_plan_desc* d) {
  if (!d || d->magic != kMagic || !d->dev) return MOONEP_EPLAN;
  moonep_sizes s;
  if (fill_sizes(d->sz.R, d->sz.E, d->sz.K, d->sz.S, d->sz.slots, &s) != MOONEP_OK)
    return MOONEP_EPLAN;
  if (std::memcmp(&s, &d->sz, sizeof(s)) != 0) return MOONEP_EPLAN;
  return MOONEP_OK;
}

// hipGetLastError() returns, and clears, the last error of the calling thread, whichever
// call caused it.  Each entry point clears it right before its launches, so the status it
// reads afterwards belongs to its own launches only.
void clear_error() { (void)hipGetLastError(); }

// The planning workspace of moonep_plan_noalloc: a file-scope device array, one copy per
// GPU the library runs on, held until the process ends.  Host code never uses the name
// `scratch` as an address (on the host it is only a stand-in for the symbol); each
// device's own address comes from hipGetSymbolAddress, looked up once per device with that
// device current, and is what the kernels receive.  Nothing in the planning kernels needs
// the workspace to start at zero: every word they read was written earlier in the same
// plan.
constexpr int64_t kNoAllocWorkspaceBytes = MOONEP_NOALLOC_WORKSPACE_MAX;
__device__ __align__(256) int32_t scratch[kNoAllocWorkspaceBytes / 4];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch` (nullptr on a HIP error).
void* device_scratch(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

int moonep_query(int R, int E, int K, int S, int slots, moonep_sizes* out) {
  if (!out) return MOONEP_EINVAL;
  moonep_sizes s;
  std::memset(&s, 0, sizeof(s));
  const int rc = fill_sizes(R, E, K, S, slots, &s);
  if (rc != MOONEP_OK) return rc;
  *out = s;
  return MOONEP_OK;
}

int moonep_plan(const int32_t* topk_ids, const float* topk_w, int R, int E, int K, int S,
                int slots, void* plan_dev, void* workspace, moonep_plan_desc* desc,
                hipStream_t stream) {
  if (!topk_ids || !topk_w || !plan_dev || !workspace || !desc) return MOONEP_EINVAL;
  moonep_sizes s;
  std::memset(&s, 0, sizeof(s));
  const int rc = fill_sizes(R, E, K, S, slots, &s);
  if (rc != MOONEP_OK) return rc;
  if (!aligned(plan_dev, 256) || !aligned(workspace, 256) || !aligned(topk_ids, 4) ||
      !aligned(topk_w, 4))
    return MOONEP_EALIGN;
  desc->magic = kMagic;
  desc->sz = s;
  desc->dev = plan_dev;
  clear_error();
  const hipError_t err = launch_plan(s, topk_ids, topk_w, static_cast<int32_t*>(plan_dev),
                                     static_cast<int32_t*>(workspace), stream);
  return err == hipSuccess ? MOONEP_OK : MOONEP_EHIP;
}

int moonep_plan_noalloc(const int32_t* topk_ids, const float* topk_w, int R, int E, int K, int S,
                        int slots, void* plan_dev, moonep_plan_desc* desc, hipStream_t stream) {
  if (!topk_ids || !topk_w || !plan_dev || !desc) return MOONEP_EINVAL;
  moonep_sizes s;
  std::memset(&s, 0, sizeof(s));
  const int rc = fill_sizes(R, E, K, S, slots, &s);
  if (rc != MOONEP_OK) return rc;
  if (s.workspace_bytes > kNoAllocWorkspaceBytes) return MOONEP_ELIMIT;
  if (!aligned(plan_dev, 256) || !aligned(topk_ids, 4) || !aligned(topk_w, 4)) return MOONEP_EALIGN;
  int dev = -1, sdev = -1;
  if (hipGetDevice(&dev) != hipSuccess || hipStreamGetDevice(stream, &sdev) != hipSuccess)
    return MOONEP_EHIP;
  if (sdev != dev) return MOONEP_EINVAL;      // the stream must belong to the current device
  void* ws = device_scratch(dev);
  if (!ws) return MOONEP_EHIP;
  desc->magic = kMagic;
  desc->sz = s;
  desc->dev = plan_dev;
  clear_error();
  const hipError_t err = launch_plan(s, topk_ids, topk_w, static_cast<int32_t*>(plan_dev),
                                     static_cast<int32_t*>(ws), stream);
  return err == hipSuccess ? MOONEP_OK : MOONEP_EHIP;
}

int moonep_dispatch(const moonep_plan_desc* plan, const uint16_t* x, int H, uint16_t* recv,
                    hipStream_t stream) {
  const int rc = check_desc(plan);
  if (rc != MOONEP_OK) return rc;
  if (!x || !recv || H <= 0 || H % 8 != 0) return MOONEP_EINVAL;
  if (!aligned(x, 16) || !aligned(recv, 16)) return MOONEP_EALIGN;
  if (!move_grid_fits(plan->sz, H)) return MOONEP_ELIMIT;
  clear_error();
  const hipError_t err = launch_dispatch(plan->sz, static_cast<const int32_t*>(plan->dev), x,
                                         H, recv, stream);
  return err == hipSuccess ? MOONEP_OK : MOONEP_EHIP;
}

int moonep_combine(const moonep_plan_desc* plan, const uint16_t* y, int H, uint16_t* out,
                   hipStream_t stream) {
  const int rc = check_desc(plan);
  if (rc != MOONEP_OK) return rc;
  if (!y || !out || H <= 0 || H % 8 != 0) return MOONEP_EINVAL;
  if (!aligned(y, 16) || !aligned(out, 16)) return MOONEP_EALIGN;
  if (!move_grid_fits(plan->sz, H)) return MOONEP_ELIMIT;
  clear_error();
  const hipError_t err = launch_combine(plan->sz, static_cast<const int32_t*>(plan->dev), y, H,
                                        out, stream);
  return err == hipSuccess ? MOONEP_OK : MOONEP_EHIP;
}

int moonep_dispatch_staged(const moonep_plan_desc* plan, const uint16_t* x, int H,
                           uint16_t* stage, uint16_t* recv, hipStream_t stream) {
  const int rc = check_desc(plan);
  if (rc != MOONEP_OK) return rc;
  if (!x || !stage || !recv || H <= 0 || H % 8 != 0) return MOONEP_EINVAL;
  if (!aligned(x, 16) || !aligned(stage, 16) || !aligned(recv, 16)) return MOONEP_EALIGN;
  if (!move_grid_fits(plan->sz, H)) return MOONEP_ELIMIT;
  clear_error();
  const hipError_t err = launch_dispatch_staged(plan->sz, static_cast<const int32_t*>(plan->dev),
                                                x, H, stage, recv, stream);
  return err == hipSuccess ? MOONEP_OK : MOONEP_EHIP;
}

int moonep_combine_staged(const moonep_plan_desc* plan, const uint16_t* y, int H,
                          uint16_t* stage, uint16_t* out, hipStream_t stream) {
  const int rc = check_desc(plan);
  if (rc != MOONEP_OK) return rc;
  if (!y || !stage || !out || H <= 0 || H % 8 != 0) return MOONEP_EINVAL;
  if (!aligned(y, 16) || !aligned(stage, 16) || !aligned(out, 16)) return MOONEP_EALIGN;
  if (!move_grid_fits(plan->sz, H)) return MOONEP_ELIMIT;
  clear_error();
  const hipError_t err = launch_combine_staged(plan->sz, static_cast<const int32_t*>(plan->dev),
                                               y, H, stage, out, stream);
  return err == hipSuccess ? MOONEP_OK : MOONEP_EHIP;
}

int moonep_dispatch_bwd(const moonep_plan_desc* plan, const uint16_t* g_recv, int H,
                        uint16_t* gx, hipStream_t stream) {
  const int rc = check_desc(plan);
  if (rc != MOONEP_OK) return rc;
  if (!g_recv || !gx || H <= 0 || H % 8 != 0) return MOONEP_EINVAL;
  if (!aligned(g_recv, 16) || !aligned(gx, 16)) return MOONEP_EALIGN;
  if (!move_grid_fits(plan->sz, H)) return MOONEP_ELIMIT;
  clear_error();
  const hipError_t err = launch_dispatch_bwd(plan->sz, static_cast<const int32_t*>(plan->dev),
                                             g_recv, H, gx, stream);
  return err == hipSuccess ? MOONEP_OK : MOONEP_EHIP;
}

int moonep_combine_bwd(const moonep_plan_desc* plan, const uint16_t* dout, const uint16_t* y,
                       int H, uint16_t* g_y, float* dw, hipStream_t stream) {
  const int rc = check_desc(plan);
  if (rc != MOONEP_OK) return rc;
  if (!dout || !y || !g_y || !dw || H <= 0 || H % 8 != 0) return MOONEP_EINVAL;
  if (!aligned(dout, 16) || !aligned(y, 16) || !aligned(g_y, 16) || !aligned(dw, 4))
    return MOONEP_EALIGN;
  clear_error();
  const hipError_t err = launch_combine_bwd(plan->sz, static_cast<const int32_t*>(plan->dev),
                                            dout, y, H, g_y, dw, stream);
  return err == hipSuccess ? MOONEP_OK : MOONEP_EHIP;
}

int moonep_reduce_grad(const moonep_plan_desc* plan, float* home_grad, const float* rep_grad,
                       int64_t G_el, hipStream_t stream) {
  const int rc = check_desc(plan);
  if (rc != MOONEP_OK) return rc;
  if (!home_grad || G_el < 0 || G_el % 4 != 0) return MOONEP_EINVAL;
  if (plan->sz.slots > 0 && !rep_grad) return MOONEP_EINVAL;
  if (!aligned(home_grad, 16) || (rep_grad && !aligned(rep_grad, 16))) return MOONEP_EALIGN;
  if (G_el == 0 || plan->sz.slots == 0) return MOONEP_OK;
  clear_error();
  const hipError_t err = launch_reduce(plan->sz, static_cast<const int32_t*>(plan->dev),
                                       home_grad, rep_grad, G_el, stream);
  return err == hipSuccess ? MOONEP_OK : MOONEP_EHIP;
}

int moonep_prefetch_weight(const moonep_plan_desc* plan, const uint16_t* home_w, int64_t W_el,
                           uint16_t* slot_w, hipStream_t stream) {
  const int rc = check_desc(plan);
  if (rc != MOONEP_OK) return rc;
  if (!home_w || W_el <= 0 || W_el % 8 != 0) return MOONEP_EINVAL;
  if (plan->sz.slots > 0 && !slot_w) return MOONEP_EINVAL;
  if (!aligned(home_w, 16) || (slot_w && !aligned(slot_w, 16))) return MOONEP_EALIGN;
  if (plan->sz.slots == 0) return MOONEP_OK;
  clear_error();
  const hipError_t err = launch_prefetch(plan->sz, static_cast<const int32_t*>(plan->dev), home_w,
                                         W_el, slot_w, stream);
  return err == hipSuccess ? MOONEP_OK : MOONEP_EHIP;
}

int moonep_expert_stub(const moonep_plan_desc* plan, const int32_t* topk_ids,
                       const uint16_t* recv, const uint16_t* home_w, const uint16_t* slot_w,
                       int64_t W_el, int H, uint16_t* y, hipStream_t stream) {
  const int rc = check_desc(plan);
  if (rc != MOONEP_OK) return rc;
  if (!topk_ids || !recv || !home_w || !y || H <= 0 || H % 8 != 0 || W_el < H || W_el % 8 != 0)
    return MOONEP_EINVAL;
  if (plan->sz.slots > 0 && !slot_w) return MOONEP_EINVAL;
  if (!aligned(recv, 16) || !aligned(home_w, 16) || !aligned(y, 16) || !aligned(topk_ids, 4) ||
      (slot_w && !aligned(slot_w, 16)))
    return MOONEP_EALIGN;
  clear_error();
  const hipError_t err = launch_expert_stub(plan->sz, static_cast<const int32_t*>(plan->dev),
                                            topk_ids, recv, home_w, slot_w, W_el, H, y, stream);
  return err == hipSuccess ? MOONEP_OK : MOONEP_EHIP;
}

int moonep_plan_status(const moonep_plan_desc* plan, moonep_plan_stats* out,
                       hipStream_t stream) {
  const int rc = check_desc(plan);
  if (rc != MOONEP_OK) return rc;
  if (!out) return MOONEP_EINVAL;
  if (hipStreamSynchronize(stream) != hipSuccess) return MOONEP_EHIP;
  int32_t hdr[H_WORDS];
  if (hipMemcpy(hdr, static_cast<const int32_t*>(plan->dev) + plan->sz.o_hdr, sizeof(hdr),
                hipMemcpyDeviceToHost) != hipSuccess)
    return MOONEP_EHIP;
  out->status = hdr[H_STATUS];
  out->bad_index = hdr[H_STATUS] == 1 ? hdr[H_BADIDX] : -1;
  out->n_pieces = hdr[H_NPIECES];
  out->n_replicas = hdr[H_NREPLICAS];
  out->n_fallback = hdr[H_NFALLBACK];
  out->max_pieces_per_rank = hdr[H_MAXPPR];
  out->n_red = hdr[H_NRED];
  out->n_shed = hdr[H_NSHED];
  out->max_load = hdr[H_MAXLOAD];
  return MOONEP_OK;
}

const char* moonep_strerror(int code) {
  switch (code) {
    case MOONEP_OK: return "ok";
    case MOONEP_EINVAL: return "invalid argument";
    case MOONEP_ELIMIT: return "sizes beyond the library's limits";
    case MOONEP_EPLAN: return "plan descriptor missing, uninitialised or inconsistent";
    case MOONEP_EHIP: return "HIP launch or copy failed";
    case MOONEP_EALIGN: return "pointer not aligned (16 bytes for data, 256 for plan/workspace)";
    default: return "unknown error";
  }
}

}  // extern "C"
