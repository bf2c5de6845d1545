// Projection GEMM interface (internal).
//
// C[m][n] = epilogue( sum_k A[arow(m)][k] * B[n][k] ) for the bias-free
// linear maps f1, f2, f_uq, f_kv of the layer equations ([explainer] §4.1,
// §4.2).  A rows may be gathered and C rows scattered through a row map, so
// the same kernel serves all packed rows, only the H/R rows, or only the
// T rows of one V2 sub-token index ([blog] §3.3.2: per-sub-token Q
// projection) without copying activations.  B is the weight matrix, stored
// [N][K] row-major as up to three stacked segments (e.g. U | Q[k] | K V for
// the target layer's T rows).
#pragma once
#include "common.h"

struct RowMap {
  const int32_t* list;  // if non-null: row = list[m] + add
  int32_t mul;          // else:        row = m * mul + add
  int32_t add;
};

enum GemmEpi {
  EPI_SILU_SPLIT = 0,  // v = SiLU(acc); columns [cend[r-1], cend[r]) -> dst[r] * scale[r] (row-major)
  EPI_RESID = 1,       // out[crow] = acc + resid[crow]
  EPI_STORE_F32 = 2,   // out (fp32) [crow] = acc  (+= if accumulate)
  EPI_STORE = 3        // out (dtype) [crow] = acc
};

struct GemmArgs {
  int32_t M, N, K;
  int32_t groups;                 // grid.z; group z shifts the maps and B pointers below
  const void* A; int64_t lda; RowMap amap; int32_t amap_zadd;
  const void* B[3]; int32_t bn[3]; int64_t bz[3];   // segment rows; per-group element stride
  int64_t ldb;                    // row stride of B (elements), normally K
  RowMap cmap; int32_t cmap_zadd;
  int32_t epi;
  void* dst[4]; int64_t ld[4]; int32_t cend[4]; float scale[4];
  const void* resid; int64_t ldr;
  void* out; int64_t ldo;
  int32_t accumulate;
};

mtfm_status launch_gemm(const GemmArgs& g, int dtype, hipStream_t s);
