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
  const void* kd; int64_t ldkd;  // the query rows' own keys / values (query space)
  const void* vd; int64_t ldvd;
  void* a; int64_t lda;          // output [query row][H*dh]
  const int32_t* tiles; int32_t ntiles;
  const int32_t* p; const int32_t* n;  // per packed row
  const int32_t* lens;
  int32_t H, G, dh;
  float out_scale;               // ln 2
  int32_t half_tiles;            // bf16: 1 = one workgroup per 32-row half tile (more workgroups)
};

mtfm_status launch_attention(const AttnArgs& a, int dtype, hipStream_t s);
