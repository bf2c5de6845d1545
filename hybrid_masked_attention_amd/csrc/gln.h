// Group LayerNorm interface (internal).
//
// y[i] = ((x[i] - mean) / sqrt(var + eps)) * gamma[type_i] + beta[type_i]   (* gate[i])
// over a row of width D, biased variance, fp32 statistics.  gamma / beta are
// [3][D] (rows H, R, T), one parameter matrix indexed per token by its type
// ([blog] §6.1: Group LayerNorm with a [G, D] parameter matrix and a per-token
// group id; GLN-MUL fusion = the gate).
#pragma once
#include "common.h"

struct GlnArgs {
  int32_t rows, D;
  const void* x; int64_t ldx;
  void* y; int64_t ldy;
  const void* gate; int64_t ldg;   // optional: y *= gate[i] (the U of the layer)
  const float* gamma; const float* beta;
  const uint8_t* type;             // per row; if null, every row has type `type_const`
  int32_t type_const;
  float eps;
  // optional: input row of output row i is xlist[i / xdiv] + i % xdiv (type from that row)
  const int32_t* xlist; int32_t xdiv;
  // ordinary (cached) stores instead of non-temporal ones, single-output forms
  // only: for small T-row outputs that the next GEMM reads at once (the all-row
  // outputs stream past L2)
  int32_t temporal;
  // optional: up to three more outputs of the same statistics with their own
  // parameters (same stride ldy); rows of type T written as zeros in output o
  // (0 = y, o = y_more[o - 1]) when bit o of zero_t is set (context-only
  // normalisation)
  int32_t n_more;
  void* y_more[3];
  const float* gamma_more[3]; const float* beta_more[3];
  int32_t zero_t;
  // optional (gated form only): the input row is the sum of n_parts fp32
  // rows x_parts + k * part_stride + row * ldx, k = 0, 1, ... in that order
  // (the attention's key-split partials); x is then not read
  const float* x_parts; int32_t n_parts; int64_t part_stride;
};

mtfm_status launch_gln(const GlnArgs& a, int dtype, hipStream_t s);
