// Host-side helpers shared by the C ABI and the backward orchestration (internal).
#pragma once
#include <cmath>

#include "attn.h"
#include "common.h"
#include "gemm.h"
#include "gln.h"

#define TRY(x)                          \
  do {                                  \
    mtfm_status _s = (x);               \
    if (_s != MTFM_OK) return _s;       \
  } while (0)

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;

inline int elem_size(int dtype) { return dtype == MTFM_BF16 ? 2 : 4; }
inline RowMap identity_map() { return RowMap{nullptr, 1, 0}; }
// Q is stored times log2(e) / sqrt(dh) so the attention kernels evaluate SiLU with exp2.
inline float q_scale(int dh) { return kLog2e / std::sqrt((float)dh); }

int64_t align_up(int64_t x, int64_t a);

struct LayerWs {
  int64_t xt = 0, z = 0, kv = 0, vt = 0, a = 0, y = 0, total = 0;
  int64_t ldvt = 0;   // row length of the transposed values (bf16 path)
};
// Row length of the transposed value copy: every packed row, rounded up to 64.
inline int64_t vt_ld(int64_t n_rows) { return (n_rows + 63) / 64 * 64; }
LayerWs layer_ws(const MetaPlan& p, const mtfm_dims* d, int op);

struct Ctx {
  const mtfm_batch* b = nullptr;
  MetaPlan plan;
  MetaPtrs meta{};
  hipStream_t s = nullptr;
  bool write_a = false;   // the bf16 forward also stores A in the workspace (single-layer calls: the probe reads it)
};

mtfm_status check_dims(const mtfm_dims* d);
mtfm_status prepare(const mtfm_batch* b, const mtfm_dims* d, const void* meta_d, const void* x0, const void* x1,
                    void* ws, size_t ws_bytes, int op, Ctx* c, void* stream);
// Where a layer puts the K (row-major, [rows][G*dh]) and V^T ([G*dh][ldvt]) of
// its rows when they are kept beyond the layer (bf16 serving cache).
struct KvOut {
  void* k = nullptr;
  void* vt = nullptr;
  int64_t ldvt = 0;
};
// Intermediates of one layer's forward pass kept for its backward (bf16,
// caller-placed).  Full layer: X~ [R][d], Z = U|Q'|K|V [R][zw] and its
// pre-activations [R][zw], A [R][H*dh].  Target layer: X~ [R][d], K|V and
// pre-activations [R][2 G*dh] (every packed row), Z_T and pre-activations
// [T][zw], A_T [T][H*dh].  A forward given one writes them there (and the
// pre-activations, which it otherwise does not produce); a backward given one
// reads them instead of recomputing GLN1, the projections and the attention.
// Both passes use the same kernels and shapes, so the values are the same.
struct FwdKeep {
  char* xt = nullptr;
  char* z = nullptr;
  char* hpre = nullptr;
  char* kv = nullptr;
  char* kvpre = nullptr;
  char* a = nullptr;
};
mtfm_status run_full(const Ctx& c, const mtfm_dims* d, const mtfm_full_w* w, const void* x_in, void* x_out, char* ws,
                     const KvOut* kv = nullptr, const FwdKeep* keep = nullptr);
mtfm_status run_target(const Ctx& c, const mtfm_dims* d, const mtfm_target_w* w, const void* x_in, void* x_out,
                       char* ws, const FwdKeep* keep = nullptr);

// backward (bwd.hip)
int64_t bwd_ws_bytes(const MetaPlan& p, const mtfm_dims* d, int op);
mtfm_status run_full_bwd(const Ctx& c, const mtfm_dims* d, const mtfm_full_w* w, const void* x_in, const void* dy,
                         void* dx, const mtfm_full_grad* g, char* ws, const FwdKeep* keep = nullptr);
mtfm_status run_target_bwd(const Ctx& c, const mtfm_dims* d, const mtfm_target_w* w, const void* x_in,
                           const void* dy, void* dx, const mtfm_target_grad* g, char* ws,
                           const FwdKeep* keep = nullptr);

// RAII bracket of one launch with HIP events when its kernel class is enabled
// (see mtfm_timing_enable); a no-op otherwise.
class TimedLaunch {
 public:
  TimedLaunch(int kclass, hipStream_t s);
  ~TimedLaunch();
  TimedLaunch(const TimedLaunch&) = delete;
  TimedLaunch& operator=(const TimedLaunch&) = delete;

 private:
  int cls_;
  hipStream_t stream_;
  hipEvent_t start_ = nullptr, stop_ = nullptr;
};

// While one of these lives, launches on this thread are not timed (no events
// are created or recorded): for the entry point that must not allocate.
class TimingOff {
 public:
  TimingOff();
  ~TimingOff();
  TimingOff(const TimingOff&) = delete;
  TimingOff& operator=(const TimingOff&) = delete;
};

// Serving candidate pass (api.hip): argument checks without the workspace,
// the workspace size, and the pass itself on checked arguments.
mtfm_status serve_targets_check(const mtfm_batch* batch, const mtfm_dims* dims, int32_t n_blocks, int32_t k_target,
                                const void* meta_d, const mtfm_full_w* full, const mtfm_target_w* tgt,
                                const void* kv_cache, size_t cache_bytes, const void* x_t, Ctx* c);
int64_t serve_targets_ws_bytes(const MetaPlan& p, const mtfm_dims* d);
mtfm_status serve_targets_run(const Ctx& c, const mtfm_dims* dims, int32_t n_blocks, int32_t k_target,
                              const mtfm_full_w* full, const mtfm_target_w* tgt, const void* kv_cache, void* x_t,
                              char* ws);

// Launch helpers that time themselves under a kernel class.
inline mtfm_status timed_gemm(int kclass, const GemmArgs& g, int dt, hipStream_t s) {
  TimedLaunch t(kclass, s);
  return launch_gemm(g, dt, s);
}
inline mtfm_status timed_attention(int kclass, const AttnArgs& a, int dt, hipStream_t s) {
  TimedLaunch t(kclass, s);
  return launch_attention(a, dt, s);
}
inline mtfm_status timed_gln(const GlnArgs& a, int dt, hipStream_t s, int kclass = MTFM_K_GLN) {
  TimedLaunch t(kclass, s);
  return launch_gln(a, dt, s);
}
