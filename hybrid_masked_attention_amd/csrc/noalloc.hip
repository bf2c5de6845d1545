// The serving candidate pass for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops): the same launches as
// mtfm_serve_targets, with the workspace taken from a file-scope device array
// instead of a caller buffer.
//
// The array is per GPU (each device that loads the library holds its own copy
// until the process ends).  Its device address is looked up once per device
// with hipGetSymbolAddress, with that device current, and kept; host code
// never passes the array's name itself to a kernel (on the host that name is
// only a stand-in, not a device address).  Nothing in the array must start at
// zero: every byte a call reads was written earlier in the same call.  Calls
// that overlap on one GPU share the array and race.

#include <mutex>

#include "api_internal.h"

namespace {

constexpr size_t kScratchBytes = (size_t)64 << 20;   // 64 MiB per GPU
constexpr int kMaxDevices = 64;

__device__ __align__(256) char scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of this device's scratch array (looked up on first use).
mtfm_status scratch_address(hipStream_t stream, char** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "mtfm_serve_targets_noalloc: hipGetDevice");
  if (stream) {
    int sdev = -1;
    e = hipStreamGetDevice(stream, &sdev);
    if (e != hipSuccess) return hip_fail(e, "mtfm_serve_targets_noalloc: hipStreamGetDevice");
    if (sdev != dev) {
      set_last_error("mtfm_serve_targets_noalloc: the stream belongs to another device than the current one");
      return MTFM_E_UNSUPPORTED;
    }
  }
  if (dev < 0 || dev >= kMaxDevices) {
    set_last_error("mtfm_serve_targets_noalloc: device index out of range");
    return MTFM_E_UNSUPPORTED;
  }
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "mtfm_serve_targets_noalloc: hipGetSymbolAddress(scratch)");
    if (!p) {
      set_last_error("mtfm_serve_targets_noalloc: hipGetSymbolAddress returned a null address");
      return MTFM_E_HIP;
    }
    g_scratch[dev] = p;
  }
  *out = (char*)g_scratch[dev];
  return MTFM_OK;
}

}  // namespace

extern "C" size_t mtfm_serve_targets_noalloc_max_bytes(void) { return kScratchBytes; }

extern "C" mtfm_status mtfm_serve_targets_noalloc(const mtfm_batch* batch, const mtfm_dims* dims, int32_t n_blocks,
                                                  int32_t k_target, const void* meta_d, const mtfm_full_w* full,
                                                  const mtfm_target_w* tgt, const void* kv_cache, size_t cache_bytes,
                                                  void* x_t, void* stream) {
  Ctx c;
  TRY(serve_targets_check(batch, dims, n_blocks, k_target, meta_d, full, tgt, kv_cache, cache_bytes, x_t, &c));
  const int64_t need = serve_targets_ws_bytes(c.plan, dims);
  if (need > (int64_t)kScratchBytes) {
    set_last_error("mtfm_serve_targets_noalloc: the candidate batch needs more scratch than the static array "
                   "holds (mtfm_serve_targets_noalloc_max_bytes); split the batch or use mtfm_serve_targets");
    return MTFM_E_WORKSPACE;
  }
  if (c.plan.n_t_rows == 0 || n_blocks == 0) return MTFM_OK;
  c.s = (hipStream_t)stream;
  char* ws = nullptr;
  TRY(scratch_address(c.s, &ws));
  TimingOff no_events;
  return serve_targets_run(c, dims, n_blocks, k_target, full, tgt, kv_cache, x_t, ws);
}
