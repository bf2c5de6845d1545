// Row-wise backward kernels of the layers (bf16 storage, fp32 math).
//
// Group LayerNorm backward ([blog] §6.1: the GLN backward reduces the
// parameter gradients block by block before one final sum): for a row x of
// width D with xhat = (x - mean) * rstd and g = dL/d(xhat * gamma + beta),
//   dgamma[type] += g * xhat,  dbeta[type] += g,
//   dx = rstd * (g*gamma - mean(g*gamma) - xhat * mean(g*gamma * xhat)).
// Each workgroup walks a strided set of rows, keeps per-type parameter sums
// in registers, reduces its four waves through LDS and writes one partial;
// a second kernel adds the partials in a fixed order (deterministic).
//
// SiLU'(h) = s (1 + h (1 - s)), s = sigmoid(h), converts gradients of the
// SiLU outputs U, Q, K, V into gradients of the projection pre-activations.

#include "bwd_kernels.h"

namespace {

typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;

template <typename T, int VPL>
MTFM_DEV void load_vec(const T* p, float* v) {
  constexpr int BYTES = VPL * (int)sizeof(T);
  if constexpr (BYTES % 16 == 0) {
    const u32x4* q = reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int c = 0; c < BYTES / 16; ++c) {
      u32x4 w = q[c];
      const T* e = reinterpret_cast<const T*>(&w);
#pragma unroll
      for (int j = 0; j < 16 / (int)sizeof(T); ++j) v[c * (16 / sizeof(T)) + j] = to_f32(e[j]);
    }
  } else {
#pragma unroll
    for (int j = 0; j < VPL; ++j) v[j] = to_f32(p[j]);
  }
}

template <typename T, int VPL>
MTFM_DEV void store_vec(T* p, const float* v) {
  constexpr int BYTES = VPL * (int)sizeof(T);
  if constexpr (BYTES % 16 == 0) {
    u32x4* q = reinterpret_cast<u32x4*>(p);
#pragma unroll
    for (int c = 0; c < BYTES / 16; ++c) {
      u32x4 w;
      T* e = reinterpret_cast<T*>(&w);
#pragma unroll
      for (int j = 0; j < 16 / (int)sizeof(T); ++j) e[j] = from_f32<T>(v[c * (16 / sizeof(T)) + j]);
      q[c] = w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < VPL; ++j) p[j] = from_f32<T>(v[j]);
  }
}

MTFM_DEV float dsilu(float h) {
  const float s = 1.0f / (1.0f + __expf(-h));
  return s * (1.0f + h * (1.0f - s));
}

MTFM_DEV int64_t map_row_b(const RowMapB& r, int m) {
  if (r.list) return (int64_t)r.list[m / r.div] + m % r.div;
  return m;
}

// Common body: normalise row `row` of x, return xhat / rstd; g is dL/d(affine output).
template <int VPL>
MTFM_DEV void gln_stats(const float* v_in, float* xhat, float* rstd_out, int D, float eps) {
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < VPL; ++j) s += v_in[j];
  const float mean = wave_sum(s) / (float)D;
  float q = 0.f;
#pragma unroll
  for (int j = 0; j < VPL; ++j) { xhat[j] = v_in[j] - mean; q += xhat[j] * xhat[j]; }
  const float rstd = rsqrtf(wave_sum(q) / (float)D + eps);
#pragma unroll
  for (int j = 0; j < VPL; ++j) xhat[j] *= rstd;
  *rstd_out = rstd;
}

// Writes the workgroup's per-type parameter partials (pg: [blocks][2][3][D]).
template <int VPL>
MTFM_DEV void flush_param_partials(float (*dg)[VPL], float (*db)[VPL], float* pg, int D, float* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float* out = pg + (int64_t)blockIdx.x * 6 * D;
  for (int which = 0; which < 6; ++which) {
    const int t = which % 3;
    float* src = which < 3 ? dg[t] : db[t];
#pragma unroll
    for (int j = 0; j < VPL; ++j) red[wave * D + lane * VPL + j] = src[j];
    __syncthreads();
    for (int c = threadIdx.x; c < D; c += 256) {
      float a = red[c] + red[D + c] + red[2 * D + c] + red[3 * D + c];
      out[which * D + c] = a;
    }
    __syncthreads();
  }
}

// GLN2 backward with the gate U: y = (xhat gamma + beta) (.) U.
//   du = dy (.) (xhat gamma + beta)        -> dH_U = du (.) SiLU'(h_U)
//   g  = dy (.) U                          -> dA / n written as bf16 (operand of the attention backward)
template <int VPL>
__global__ __launch_bounds__(256) void gln2_bwd_kernel(Gln2BwdArgs a) {
  __shared__ float red[4 * 1024];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float dg[3][VPL] = {}, db[3][VPL] = {};
  for (int row = blockIdx.x * 4 + wave; row < a.rows; row += gridDim.x * 4) {
    float x[VPL], xhat[VPL], rstd;
    load_vec<bf16, VPL>(a.a + (int64_t)row * a.lda + lane * VPL, x);
    gln_stats<VPL>(x, xhat, &rstd, a.D, a.eps);
    const int t = a.type ? a.type[map_row_b(a.nmap, row)] : a.type_const;
    float gm[VPL], bt[VPL], u[VPL], hu[VPL], dyv[VPL];
    load_vec<float, VPL>(a.gamma + t * a.D + lane * VPL, gm);
    load_vec<float, VPL>(a.beta + t * a.D + lane * VPL, bt);
    load_vec<bf16, VPL>(a.u + (int64_t)row * a.ldu + lane * VPL, u);
    load_vec<bf16, VPL>(a.hu + (int64_t)row * a.ldhu + lane * VPL, hu);
    load_vec<float, VPL>(a.dy + (int64_t)row * a.lddy + lane * VPL, dyv);
    float du[VPL], gg[VPL];
    float s1 = 0.f, s2 = 0.f;
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      const float ytil = xhat[j] * gm[j] + bt[j];
      du[j] = dyv[j] * ytil * dsilu(hu[j]);
      const float g = dyv[j] * u[j];
#pragma unroll
      for (int tt = 0; tt < 3; ++tt)
        if (t == tt) { dg[tt][j] += g * xhat[j]; db[tt][j] += g; }
      gg[j] = g * gm[j];
      s1 += gg[j];
      s2 += gg[j] * xhat[j];
    }
    const float m1 = wave_sum(s1) / (float)a.D, m2 = wave_sum(s2) / (float)a.D;
    const float ninv = 1.0f / (float)a.n[map_row_b(a.nmap, row)];
    float dan[VPL], lo[VPL];
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      dan[j] = rstd * (gg[j] - m1 - xhat[j] * m2) * ninv;
      lo[j] = dan[j] - (float)(bf16)dan[j];
    }
    store_vec<bf16, VPL>(a.dhu + (int64_t)row * a.lddhu + lane * VPL, du);
    store_vec<bf16, VPL>(a.dan + (int64_t)row * a.lddan + lane * VPL, dan);
    store_vec<bf16, VPL>(a.dan_lo + (int64_t)row * a.lddan + lane * VPL, lo);
  }
  flush_param_partials<VPL>(dg, db, a.pg, a.D, red);
}

// GLN1 backward plus the residual: dX = dY + LN backward of dX~ (.) gamma.
template <int VPL>
__global__ __launch_bounds__(256) void gln1_bwd_kernel(Gln1BwdArgs a) {
  __shared__ float red[4 * 1024];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float dg[3][VPL] = {}, db[3][VPL] = {};
  for (int row = blockIdx.x * 4 + wave; row < a.rows; row += gridDim.x * 4) {
    float x[VPL], xhat[VPL], rstd;
    load_vec<bf16, VPL>(a.x + (int64_t)row * a.ldx + lane * VPL, x);
    gln_stats<VPL>(x, xhat, &rstd, a.D, a.eps);
    const int t = a.type[row];
    float gm[VPL], dxt[VPL], dres[VPL];
    load_vec<float, VPL>(a.gamma + t * a.D + lane * VPL, gm);
    load_vec<float, VPL>(a.dxt + (int64_t)row * a.lddxt + lane * VPL, dxt);
    load_vec<bf16, VPL>(a.dres + (int64_t)row * a.lddres + lane * VPL, dres);
    float gg[VPL];
    float s1 = 0.f, s2 = 0.f;
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
#pragma unroll
      for (int tt = 0; tt < 3; ++tt)
        if (t == tt) { dg[tt][j] += dxt[j] * xhat[j]; db[tt][j] += dxt[j]; }
      gg[j] = dxt[j] * gm[j];
      s1 += gg[j];
      s2 += gg[j] * xhat[j];
    }
    const float m1 = wave_sum(s1) / (float)a.D, m2 = wave_sum(s2) / (float)a.D;
    float dx[VPL];
#pragma unroll
    for (int j = 0; j < VPL; ++j) dx[j] = dres[j] + rstd * (gg[j] - m1 - xhat[j] * m2);
    store_vec<bf16, VPL>(a.dx + (int64_t)row * a.lddx + lane * VPL, dx);
  }
  flush_param_partials<VPL>(dg, db, a.pg, a.D, red);
}

// out[which][c] = sum over blocks of pg[block][which][c], which in {dgamma x3, dbeta x3}.
// A workgroup owns 64 consecutive outputs; each of its four waves sums a
// contiguous quarter of the blocks, then the four sums are added in order
// (fixed order: deterministic).
__global__ __launch_bounds__(256) void param_reduce_kernel(const float* pg, int blocks, int D, float* dgamma,
                                                           float* dbeta) {
  __shared__ float part[4][64];
  const int l = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int i = blockIdx.x * 64 + l;
  float s = 0.f;
  if (i < 6 * D) {
    const int b0 = w * blocks / 4, b1 = (w + 1) * blocks / 4;
#pragma unroll 8
    for (int b = b0; b < b1; ++b) s += pg[(int64_t)b * 6 * D + i];
  }
  part[w][l] = s;
  __syncthreads();
  if (w != 0 || i >= 6 * D) return;
  const float t = ((part[0][l] + part[1][l]) + part[2][l]) + part[3][l];
  if (i < 3 * D) dgamma[i] = t;
  else dbeta[i - 3 * D] = t;
}

// out[c][r] = in[r][c] for up to three row segments stacked along r.
__global__ __launch_bounds__(256) void transpose_kernel(TransposeArgs a) {
  __shared__ bf16 tile[32][33];
  const int r0 = blockIdx.y * 32, c0 = blockIdx.x * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  for (int k = ty; k < 32; k += 8) {
    const int r = r0 + k, c = c0 + tx;
    bf16 v = (bf16)0.f;
    if (r < a.rows && c < a.cols) {
      int rr = r, s = 0;
      while (s < 2 && rr >= a.seg_rows[s]) { rr -= a.seg_rows[s]; ++s; }
      v = a.in[s][(int64_t)rr * a.cols + c];
    }
    tile[k][tx] = v;
  }
  __syncthreads();
  for (int k = ty; k < 32; k += 8) {
    const int c = c0 + k, r = r0 + tx;
    if (c < a.cols && r < a.rows) a.out[(int64_t)c * a.ldo + r] = tile[tx][k];
  }
}

// dH_Q = dQ * scale * SiLU'(h_Q)   (fp32 accumulator -> bf16 pre-activation gradient)
template <int VPL>
int gln_bwd_blocks(int rows) {
  return std::max(1, std::min(1024, (rows + 3) / 4));
}

}  // namespace

int gln_bwd_grid(int rows) { return gln_bwd_blocks<1>(rows); }

mtfm_status launch_gln2_bwd(const Gln2BwdArgs& a, hipStream_t s) {
  if (a.rows <= 0) return MTFM_OK;
  const int blocks = gln_bwd_grid(a.rows);
  switch (a.D / 64) {
    case 4: gln2_bwd_kernel<4><<<blocks, 256, 0, s>>>(a); break;
    case 8: gln2_bwd_kernel<8><<<blocks, 256, 0, s>>>(a); break;
    case 16: gln2_bwd_kernel<16><<<blocks, 256, 0, s>>>(a); break;
    default: return MTFM_E_UNSUPPORTED;
  }
  MTFM_LAUNCH_CHECK("gln2_bwd");
  return MTFM_OK;
}

mtfm_status launch_gln1_bwd(const Gln1BwdArgs& a, hipStream_t s) {
  if (a.rows <= 0) return MTFM_OK;
  const int blocks = gln_bwd_grid(a.rows);
  switch (a.D / 64) {
    case 4: gln1_bwd_kernel<4><<<blocks, 256, 0, s>>>(a); break;
    case 8: gln1_bwd_kernel<8><<<blocks, 256, 0, s>>>(a); break;
    case 16: gln1_bwd_kernel<16><<<blocks, 256, 0, s>>>(a); break;
    default: return MTFM_E_UNSUPPORTED;
  }
  MTFM_LAUNCH_CHECK("gln1_bwd");
  return MTFM_OK;
}

mtfm_status launch_param_reduce(const float* pg, int blocks, int D, float* dgamma, float* dbeta, hipStream_t s) {
  param_reduce_kernel<<<(6 * D + 63) / 64, 256, 0, s>>>(pg, blocks, D, dgamma, dbeta);
  MTFM_LAUNCH_CHECK("param_reduce");
  return MTFM_OK;
}

mtfm_status launch_transpose(const TransposeArgs& a, hipStream_t s) {
  if (a.rows <= 0 || a.cols <= 0) return MTFM_OK;
  dim3 grid((a.cols + 31) / 32, (a.rows + 31) / 32);
  transpose_kernel<<<grid, 256, 0, s>>>(a);
  MTFM_LAUNCH_CHECK("transpose");
  return MTFM_OK;
}

