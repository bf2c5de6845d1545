// V2 target-side row kernels (internal): per-parent token mixing and mean
// pooling over the sub-token rows, and the gate/up weight interleave of the
// SwiGLU projection ([blog] §3.3.2).
#pragma once
#include "common.h"

struct TokenRowsArgs {
  bf16* x; int64_t ldx;            // packed rows; parent m's sub-token z at parent_row[m] + z
  const int32_t* parent_row;
  int32_t n_parents, S, D;
  bf16* out; int64_t ldo;          // pooling: [n_parents][D]
};

struct RepackArgs {
  const bf16* gate; const bf16* up;   // [S][F][D] each
  bf16* out;                          // [S][2F][D], rows in blocks of 32: gate units, then up units
  int32_t S, F, D;
};

mtfm_status launch_token_mix(const TokenRowsArgs& a, hipStream_t s);
mtfm_status launch_token_pool(const TokenRowsArgs& a, hipStream_t s);
mtfm_status launch_repack_gate_up(const RepackArgs& a, hipStream_t s);
