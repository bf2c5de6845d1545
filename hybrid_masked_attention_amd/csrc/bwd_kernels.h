// Backward-pass kernel interfaces (internal).  bf16 storage, fp32 math.
#pragma once
#include "common.h"

// Row map of the row-wise backward kernels: packed row = list[m / div] + m % div,
// or m itself when list is null.
struct RowMapB {
  const int32_t* list;
  int32_t div;
};

struct Gln2BwdArgs {
  int32_t rows, D;
  const bf16* a; int64_t lda;       // attention output A (forward input of GLN2)
  const float* gamma; const float* beta;
  const uint8_t* type; int32_t type_const; RowMapB nmap;  // packed row of a row (type, n)
  const int32_t* n;                 // visible-key counts, per packed row
  float eps;
  const bf16* u; int64_t ldu;       // gate U (SiLU output)
  const bf16* hu; int64_t ldhu;     // pre-activation of U
  const float* dy; int64_t lddy;    // dL/dY (fp32)
  bf16* dhu; int64_t lddhu;         // out: dL/d(pre-activation of U)
  bf16* dan; int64_t lddan;         // out: dL/dA divided by n, as bf16 hi + lo (hi = bf16(v),
  bf16* dan_lo;                     //      lo = bf16(v - hi); same stride)
  float* pg;                        // out: [blocks][2][3][D] parameter partials
};

struct Gln1BwdArgs {
  int32_t rows, D;
  const bf16* x; int64_t ldx;       // layer input X
  const float* gamma;
  const uint8_t* type;
  float eps;
  const float* dxt; int64_t lddxt;  // dL/dX~ (fp32)
  const bf16* dres; int64_t lddres; // dL/dX' flowing through the residual
  bf16* dx; int64_t lddx;           // out
  float* pg;                        // out: [blocks][2][3][D]
};

struct TransposeArgs {
  const bf16* in[3];                // row segments stacked along r, each [seg_rows][cols]
  int32_t seg_rows[3];
  int32_t rows, cols;
  bf16* out; int64_t ldo;           // out[c][r]
};

int gln_bwd_grid(int rows);
mtfm_status launch_gln2_bwd(const Gln2BwdArgs& a, hipStream_t s);
mtfm_status launch_gln1_bwd(const Gln1BwdArgs& a, hipStream_t s);
mtfm_status launch_param_reduce(const float* pg, int blocks, int D, float* dgamma, float* dbeta, hipStream_t s);
mtfm_status launch_transpose(const TransposeArgs& a, hipStream_t s);

// Attention backward ([explainer] §4.1 attention, differentiated; [blog]
// §6.1 lists the FA2-style backward of the masked attention).  Inputs are the
// forward's stored bf16 tensors: Q' (= Q log2(e)/sqrt(dh)), K, V, the
// pre-activations of Q, K, V, and dA/n.
struct AttnBwdArgs {
  const bf16* q; int64_t ldq;       // Q' rows (query space), head h at h*dh
  const bf16* k; int64_t ldk;       // context K rows (packed rows), group g at g*dh
  const bf16* v; int64_t ldv;
  const bf16* dan; int64_t lddan;   // dA / n (query space), bf16 hi part
  const bf16* dan_lo;               // and lo part (same stride): dP uses hi + lo
  const int32_t* qtiles;            // query tile descriptors (full or target)
  int32_t nqtiles;
  const int32_t* user;              // user table of the metadata, [8][n_users + 1]
  int32_t n_users;
  int32_t query_tiles_row;          // UT_FTILE or UT_TTILE
  const int32_t* p; const int32_t* n;
  const int32_t* lens;
  int32_t H, G;
  // dQ kernel: dhq = (sum_j dS_ij k_j + self term) / sqrt(dh) * SiLU'(hq), bf16
  float* dq;                        // [query rows][H*dh] fp32: the self kernel's term of T rows
  const bf16* hq; int64_t ldhq;     // pre-activation of Q (query space)
  bf16* dhq; int64_t lddhq;         // out
  float dq_scale;                   // 1 / sqrt(dh)
  // dK / dV kernel (context keys)
  const bf16* hk; int64_t ldhk;     // pre-activations of K, V of context rows (packed rows)
  const bf16* hv; int64_t ldhv;
  bf16* dhk; int64_t lddhk;         // out: dL/d(pre-activation of K), V, context rows
  bf16* dhv; int64_t lddhv;
  // self term of T rows (query space = T rows or packed rows)
  int32_t n_self_rows;              // rows of the query space that are T rows
  RowMapB self_rows;                // query-space row of the i-th T row
  RowMapB self_packed;              // packed row of the i-th T row
  const bf16* ks; int64_t ldks;     // the T rows' own K, V (query space)
  const bf16* vs; int64_t ldvs;
  const bf16* hks; int64_t ldhks;   // their pre-activations
  const bf16* hvs; int64_t ldhvs;
  bf16* dhks; int64_t lddhks;       // out
  bf16* dhvs; int64_t lddhvs;
};

mtfm_status launch_attn_bwd(const AttnBwdArgs& a, int64_t n_key_tiles, hipStream_t s);
