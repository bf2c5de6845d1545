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
  const int32_t* list;  // if non-null: row = list[m / div] + m % div + add
  int32_t mul;          // else:        row = m * mul + add
  int32_t add;
  int32_t div;          // 0 or 1: plain list lookup
};

enum GemmEpi {
  EPI_SILU_SPLIT = 0,  // v = SiLU(acc); columns [cend[r-1], cend[r]) -> dst[r] * scale[r] (row-major)
  EPI_RESID = 1,       // out[crow] = acc + resid[crow]
  EPI_STORE_F32 = 2,   // out (fp32) [crow] = acc  (+= if accumulate)
  EPI_STORE = 3,       // out (dtype) [crow] = acc
  EPI_SWIGLU = 4       // bf16: weight rows interleaved in blocks of 32 (gate units [32j, 32j + 32), then up
                       // units [32j, 32j + 32)); out[crow][32j + i] = SiLU(gate) * up, width N / 2
};

struct GemmArgs {
  int32_t M, N, K;
  int32_t groups;                 // grid.z; group z shifts the maps and B pointers below
  const void* A; int64_t lda; RowMap amap; int32_t amap_zadd;
  int64_t a_rows;                 // rows of the A buffer; required (bf16) when amap gathers through a list
  const void* B[3]; int32_t bn[3]; int64_t bz[3];   // segment rows; per-group element stride
  int64_t ldb;                    // row stride of B (elements), normally K
  RowMap cmap; int32_t cmap_zadd;
  int32_t epi;
  void* dst[4]; int64_t ld[4]; int32_t cend[4]; float scale[4];
  const void* resid; int64_t ldr;
  void* out; int64_t ldo;
  int32_t accumulate;
  void* pre; int64_t ldpre;       // EPI_SILU_SPLIT: if set, also store the pre-activation acc here
  // EPI_SILU_SPLIT (bf16): if set, segment 3 is stored only for output rows r
  // with seg3_type[r] == T (a layer's own V is read back only by its T rows)
  const uint8_t* seg3_type;
  // EPI_SILU_SPLIT (bf16, identity row maps): if set, output columns
  // [vt_col0, vt_col0 + vt_cols) are also written transposed,
  //   vt[(n - vt_col0) * ldvt + perm16(m)]  for every m < ldvt,
  // rows past M as zeros; perm16 permutes rows within aligned groups of 16 as
  // {0-3, 8-11, 4-7, 12-15} (the key order of the attention's P V operand).
  void* vt; int64_t ldvt; int32_t vt_col0, vt_cols;
  // with groups > 1: group z's transposed copy at vt + z * vt_zstride (elements)
  int64_t vt_zstride;
  // bf16, dense: if bgroup[0] is set, group z reads its weights (one segment of
  // N rows, stride ldb) from bgroup[z] instead of B (up to 4 groups)
  const void* bgroup[4];
  // bf16 only: if set, B is not read; the weights are 2:4-pruned and packed
  // (mtfm_s24_pack layout) as bs24_rows stacked rows, output column n of
  // group z taking packed row z * bs24_zrows + n; run on the sparse MFMA
  const void* bs24; int32_t bs24_rows, bs24_zrows;
};

mtfm_status launch_gemm(const GemmArgs& g, int dtype, hipStream_t s);

// Weight-gradient GEMM: C[m][n] (fp32, overwritten or accumulated) =
//   sum over r in [0, R) of A[arow(r)][m] * B[brow(r)][n]
// (both operands row-major with the reduced index r as their row), for
// dW = dZ^T X~ style products over all packed rows.  Split over r into
// partial sums that are added in a fixed order (deterministic).
struct GemmTNArgs {
  int32_t M, N, R;
  int32_t groups;                 // grid.z; group z shifts maps and pointers
  const void* A; int64_t lda; RowMap amap; int32_t amap_zadd;
  int64_t a_zoff;                 // element offset per group
  const void* B; int64_t ldb; RowMap bmap; int32_t bmap_zadd;
  int64_t a_rows, b_rows;         // rows of the A and B buffers (bounds the loads); 0 if unknown
  float* C; int64_t ldc; int64_t c_zoff; int32_t accumulate;
  float* partial; int64_t partial_elems;   // workspace for split partial sums
};

int64_t gemm_tn_partial_elems(int32_t M, int32_t N, int32_t R, int32_t groups);
mtfm_status launch_gemm_tn(const GemmTNArgs& g, hipStream_t s);
