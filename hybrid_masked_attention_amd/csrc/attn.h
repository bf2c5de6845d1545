// Masked pointwise-SiLU attention interface (internal).
//
//   A_h[i] = (1 / n_i) * sum_{j visible to i} SiLU(q_ih . k_jg / sqrt(dh)) v_jg,  g = h / r
//
// ([explainer] §4.1 and §4.2 attention equations; [blog] §6.1: one FA2-style
// interface for Full and Target attention with dynamic-mask reads and SiLU
// fused.)  Queries come from a query space (all packed rows for the full
// layer, the T rows for the target layer) tiled by the mask metadata; keys are
// the user's context rows (H then R) plus, for T rows, the row itself.
//
// Q must be stored pre-multiplied by log2(e) / sqrt(dh): then with
// s = q' . k, SiLU(x) = ln2 * s / (1 + 2^-s), so the kernels evaluate
// s * rcp(1 + exp2(-s)) per visible pair and fold ln2 / n_i into the output.
#pragma once
#include <type_traits>

#include "common.h"

struct AttnArgs {
  const void* q; int64_t ldq;    // query rows (query space); head h at column h*dh
  const void* k; int64_t ldk;    // key rows (packed rows); group g at column g*dh
  const void* v; int64_t ldv;    // value rows (fp32 path)
  // bf16 path: values transposed, vt[(g*dh + d) * ldvt + perm16(packed row)]
  // (rows permuted within aligned groups of 16 as {0-3, 8-11, 4-7, 12-15});
  // ldvt a multiple of 64 covering every packed row, slots past the last row zero
  const void* vt; int64_t ldvt;
  int32_t n_key_rows;            // packed rows in k (rows past it read as zero)
  int32_t max_user_rows;         // bf16 path: most packed rows of one user (bounds one user's K resource)
  const void* kd; int64_t ldkd;  // the query rows' own keys / values (query space)
  const void* vd; int64_t ldvd;
  void* a; int64_t lda;          // output [query row][H*dh]; optional on the bf16 path (nullptr: not written)
  const int32_t* tiles; int32_t ntiles;
  // bf16 path, optional work order (mask metadata): entry 8 k + x is the
  // slice id 2 tile + half that XCD x takes k-th, -1 past its list; the grid is
  // n_order (x G with per_group) workgroups.  nullptr: XCD-contiguous order.
  const int32_t* order; int32_t n_order;
  // bf16 path, optional query-row permutation: a tile's query-row field is
  // then a position, and the row at position k is query row qperm[k] at
  // packed row gperm[k] (both or neither)
  const int32_t* qperm; const int32_t* gperm;
  const int32_t* p; const int32_t* n;  // per packed row
  const int32_t* lens;
  int32_t H, G, dh;
  float out_scale;               // ln 2
  // bf16 path, optional fused epilogue (y != nullptr): the gated group
  // LayerNorm after attention, y[row] = (LN(A[row]) * ln_g[t] + ln_b[t]) (.) u[row]
  // over the row's H*dh values, t = type[packed row] (ln_g / ln_b [3][H*dh] fp32)
  void* y; int64_t ldy;
  const void* u; int64_t ldu;
  const float* ln_g; const float* ln_b;
  const uint8_t* type;
  float eps;
  // bf16 path: one workgroup per KV group of a query half instead of one per
  // query half (G times the workgroups; A only, no fused epilogue)
  int32_t per_group;
  // bf16 path with per_group, optional key splits (ksplit > 1): each slice's
  // key tiles are divided into ksplit contiguous runs, one workgroup each
  // (ksplit times the workgroups); run s writes its fp32 partial of A (the
  // 1/n scale applied; the T row's own key in run 0) to
  // a_part + s * part_stride with row stride lda, and A itself is not written.
  // The partials of every run are written, zeros for an empty run.
  int32_t ksplit;
  float* a_part; int64_t part_stride;
};

mtfm_status launch_attention(const AttnArgs& a, int dtype, hipStream_t s);
