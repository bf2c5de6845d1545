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
// Host-side plan of a batch: totals and device pointers into the metadata.
struct MetaPlan {
  int32_t n_users = 0, split = 1;
  int64_t n_rows = 0, n_t_rows = 0, n_parents = 0, n_ctx_rows = 0;
  int64_t n_full_tiles = 0, n_target_tiles = 0, n_key_tiles = 0;
  int32_t max_user_rows = 0, max_t_rows = 0;
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
