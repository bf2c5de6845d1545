// Internal definitions shared by the libmtfm translation units (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mtfm.h"

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

#define MTFM_DEV __device__ __forceinline__

// Debug builds (MTFM_DEBUG, build.py --debug) check the indexing assumptions
// of the kernels.  MTFM_DCHECK_UNIFORM is for conditions every thread of the
// workgroup evaluates alike (read from a tile descriptor, say): a violation is
// reported and the whole workgroup leaves before any barrier, reading nothing
// out of bounds.  MTFM_DCHECK_LANE only reports (the caller keeps the access
// in bounds).  Release builds compile both away.
#ifdef MTFM_DEBUG
#define MTFM_DCHECK_UNIFORM(cond, what)                                                     \
  do {                                                                                      \
    if (!(cond)) {                                                                          \
      if (threadIdx.x == 0) printf("mtfm debug: %s failed (%s:%d, block %u)\n", what, __FILE__, __LINE__, \
                                   blockIdx.x);                                             \
      return;                                                                               \
    }                                                                                       \
  } while (0)
#define MTFM_DCHECK_LANE(cond, what)                                                        \
  do {                                                                                      \
    if (!(cond)) printf("mtfm debug: %s failed (%s:%d, block %u thread %u)\n", what, __FILE__, __LINE__, \
                        blockIdx.x, threadIdx.x);                                           \
  } while (0)
#else
#define MTFM_DCHECK_UNIFORM(cond, what) do {} while (0)
#define MTFM_DCHECK_LANE(cond, what) do {} while (0)
#endif

// Tile edge of the mask metadata and of the attention kernels.
static constexpr int kTile = MTFM_TILE;

// Rows of the user table inside the metadata buffer (each [n_users + 1]).
enum UserTable { UT_ROW = 0, UT_ACT = 1, UT_PARENT = 2, UT_CTX = 3, UT_FTILE = 4, UT_TTILE = 5, UT_TROW = 6, UT_KTILE = 7,
                 UT_COUNT = 8 };

// Token types, also the row index into the [3][D] group-LayerNorm parameters.
enum TokenType { TT_H = 0, TT_R = 1, TT_T = 2 };

// Tile descriptor fields (int32 x 8), see mtfm.h.
enum TileField { TD_USER = 0, TD_ROW0 = 1, TD_NROWS = 2, TD_FULL_END = 3, TD_END = 4, TD_GROW0 = 5, TD_QROW0 = 6, TD_UROW0 = 7 };

MTFM_DEV float to_f32(float x) { return x; }
MTFM_DEV float to_f32(bf16 x) { return (float)x; }
template <typename T> MTFM_DEV T from_f32(float x);
template <> MTFM_DEV float from_f32<float>(float x) { return x; }
template <> MTFM_DEV bf16 from_f32<bf16>(float x) { return (bf16)x; }

MTFM_DEV float silu_f(float x) { return x / (1.0f + __expf(-x)); }

MTFM_DEV float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
MTFM_DEV int wave_min(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o, 64));
  return v;
}
MTFM_DEV int wave_max(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o, 64));
  return v;
}

// Logical block index such that blocks sharing an XCD get consecutive ids:
// the hardware hands consecutive workgroup ids to the 8 XCDs round-robin, so
// logical neighbours (which share operands) land on one XCD and its L2.
MTFM_DEV int xcd_remap(int bid, int nblocks) {
  const int q = nblocks >> 3, r = nblocks & 7;
  const int x = bid & 7, k = bid >> 3;
  return x * q + min(x, r) + k;
}

// Orders one wave's LDS accesses across lanes: its earlier LDS writes before
// its later reads of what other lanes wrote, and its earlier reads before
// later overwrites.  A wave-scope release / acquire pair around a wave
// barrier; it also keeps the compiler from moving LDS accesses across it.
MTFM_DEV void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Largest i in [0, n) with off[i] <= x (off ascending, off[0] <= x).
MTFM_DEV int upper_index(const int32_t* off, int n, int x) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (off[mid] <= x) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// ---------------------------------------------------------------------------
// Attention work order.  The bf16 attention grids take their 32-row query
// slices in an order that balances the 8 XCDs (each with its own L2; the
// hardware deals consecutive workgroup ids to them round-robin): users ranked
// by estimated work, largest first (ties: lower index first), dealt to the
// XCDs in a boustrophedon 0..7, 7..0, 0..7 ..., each XCD taking its users in
// rank order and a user's slices last first (the later rows see the most
// keys).  A user's slices stay on one XCD, so its K / V tiles are fetched into
// one L2.  The estimate depends on the lengths alone: the host sizes the grid
// with the same integer arithmetic the device uses to write the order.
#define MTFM_HD __host__ __device__ __forceinline__

constexpr int kOrderMaxUsers = 2048;   // larger batches keep the plain XCD-contiguous order (as do
                                        // batches the dealing would leave unbalanced)
constexpr int kTSortMaxRows = 4096;    // users with more T rows keep their own order
enum OrderLayer { OL_FULL = 0, OL_TARGET = 1 };

// 32-row query slices of user u: every packed row (full layer) or its T rows.
MTFM_HD int32_t order_slices(const int32_t* lens, int u, int split, int layer) {
  const int32_t lt = split * lens[3 * u + 2];
  const int32_t rows = layer == OL_FULL ? lens[3 * u] + lens[3 * u + 1] + lt : lt;
  return (rows + 31) / 32;
}

// Work of slice k of user u: key tiles it can visit (a bound from the lengths:
// an H row sees L_H keys, R row j L_H + j + 1, a T row at most L_H + L_R),
// plus one for the slice's fixed cost.
MTFM_HD int32_t order_slice_work(const int32_t* lens, int u, int split, int layer, int k) {
  const int32_t lh = lens[3 * u], ctx = lh + lens[3 * u + 1];
  if (layer == OL_TARGET) return (ctx + 63) / 64 + 1;
  const int32_t rows = ctx + split * lens[3 * u + 2];
  const int32_t last = (32 * k + 32 < rows ? 32 * k + 32 : rows) - 1;
  const int32_t p = last < lh ? lh : (last < ctx ? last + 1 : ctx);
  return (p + 63) / 64 + 1;
}

MTFM_HD int64_t order_user_work(const int32_t* lens, int u, int split, int layer) {
  const int32_t ns = order_slices(lens, u, split, layer);
  int64_t w = 0;
  for (int k = 0; k < ns; ++k) w += order_slice_work(lens, u, split, layer, k);
  return w;
}

// XCD of the user of rank r (boustrophedon over groups of 8 ranks).
MTFM_HD int order_xcd(int r) { return ((r >> 3) & 1) ? 7 - (r & 7) : (r & 7); }

// ---------------------------------------------------------------------------
// Host-side plan of a batch: totals and device pointers into the metadata.
struct MetaPlan {
  int32_t n_users = 0, split = 1;
  int64_t n_rows = 0, n_t_rows = 0, n_parents = 0, n_ctx_rows = 0;
  int64_t n_full_tiles = 0, n_target_tiles = 0, n_key_tiles = 0;
  int32_t max_user_rows = 0, max_t_rows = 0, max_ctx_rows = 0;
  int64_t n_full_order = 0, n_target_order = 0;   // work-order entries (8 x longest XCD list; 0 = none)
  mtfm_meta_layout lay{};
};

struct MetaPtrs {
  const int32_t* user;      // [UT_COUNT][n_users + 1]
  const int32_t* p;
  const int32_t* n;
  const uint8_t* type;
  const int32_t* full_tiles;
  const int32_t* target_tiles;
  const int32_t* ctx_rows;
  const int32_t* parent_row;
  const int32_t* full_order;     // nullptr when the batch has no work order
  const int32_t* target_order;
  // T rows of each user in ascending order of their visible prefix (stable):
  // position k holds T row tsort_q[k] (query space) at packed row tsort_g[k];
  // target_tiles_sorted tiles those positions like target_tiles the T rows
  const int32_t* tsort_q;
  const int32_t* tsort_g;
  const int32_t* target_tiles_sorted;
};

mtfm_status plan_meta(const mtfm_batch* b, MetaPlan* plan);
MetaPtrs meta_ptrs(const MetaPlan& plan, const void* meta_d);

// Records a HIP failure for mtfm_last_error and maps it to a status.
mtfm_status hip_fail(hipError_t e, const char* where);
// Records a message for mtfm_last_error (argument or size checks).
void set_last_error(const char* msg);
#define MTFM_LAUNCH_CHECK(where)                                  \
  do {                                                            \
    hipError_t _e = hipGetLastError();                            \
    if (_e != hipSuccess) return hip_fail(_e, where);             \
  } while (0)

// ---------------------------------------------------------------------------
// Launchers implemented in the kernel translation units.
mtfm_status launch_mask_build(const mtfm_batch* b, const MetaPlan& plan, void* meta_d, hipStream_t s);
