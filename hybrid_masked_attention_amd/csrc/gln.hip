// Group LayerNorm kernels: one wave per row, the row held in registers
// (D / 64 contiguous values per lane, moved as 16-byte vectors), two-pass
// mean and variance in fp32, type-indexed affine, optional multiplicative
// gate, optional gathered input rows, and up to four outputs of the same
// statistics with different parameters (the target layers of one block share
// their context rows).  HBM-bound: each row is read once and written once per
// output.

#include "gln.h"

namespace {

typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;

// Load / store VPL contiguous elements through 16-byte vectors when they fill
// whole vectors, element by element otherwise.
template <typename T, int VPL>
MTFM_DEV void load_row(const T* p, float* v) {
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
MTFM_DEV void store_row(T* p, const float* v) {
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

template <typename T, int VPL, int NOUT>
__global__ __launch_bounds__(256) void gln_kernel(GlnArgs a) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= a.rows) return;
  const int64_t xrow = a.xlist ? (int64_t)a.xlist[row / a.xdiv] + row % a.xdiv : row;
  float v[VPL];
  load_row<T, VPL>((const T*)a.x + xrow * a.ldx + lane * VPL, v);
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < VPL; ++j) s += v[j];
  const float mean = wave_sum(s) / (float)a.D;
  float q = 0.f;
#pragma unroll
  for (int j = 0; j < VPL; ++j) { v[j] -= mean; q += v[j] * v[j]; }
  const float rstd = rsqrtf(wave_sum(q) / (float)a.D + a.eps);
  const int t = a.type ? a.type[xrow] : a.type_const;
  const bool zero = a.zero_t && t == TT_T;
  float g[VPL];
  if (a.gate) load_row<T, VPL>((const T*)a.gate + (int64_t)row * a.ldg + lane * VPL, g);
#pragma unroll
  for (int o = 0; o < NOUT; ++o) {
    const float* gamma = o ? a.gamma_more[o - 1] : a.gamma;
    const float* beta = o ? a.beta_more[o - 1] : a.beta;
    T* y = (T*)(o ? a.y_more[o - 1] : a.y);
    float gm[VPL], bt[VPL], w[VPL];
    load_row<float, VPL>(gamma + t * a.D + lane * VPL, gm);
    load_row<float, VPL>(beta + t * a.D + lane * VPL, bt);
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      w[j] = zero ? 0.f : v[j] * rstd * gm[j] + bt[j];
      if (a.gate) w[j] *= g[j];
    }
    store_row<T, VPL>(y + (int64_t)row * a.ldy + lane * VPL, w);
  }
}

template <typename T, int NOUT>
mtfm_status launch_n(const GlnArgs& a, hipStream_t s) {
  const unsigned blocks = (unsigned)((a.rows + 3) / 4);
  switch (a.D / 64) {
    case 1: gln_kernel<T, 1, NOUT><<<blocks, 256, 0, s>>>(a); break;
    case 2: gln_kernel<T, 2, NOUT><<<blocks, 256, 0, s>>>(a); break;
    case 4: gln_kernel<T, 4, NOUT><<<blocks, 256, 0, s>>>(a); break;
    case 8: gln_kernel<T, 8, NOUT><<<blocks, 256, 0, s>>>(a); break;
    case 16: gln_kernel<T, 16, NOUT><<<blocks, 256, 0, s>>>(a); break;
    default: return MTFM_E_UNSUPPORTED;
  }
  MTFM_LAUNCH_CHECK("gln");
  return MTFM_OK;
}

template <typename T>
mtfm_status launch_t(const GlnArgs& a, hipStream_t s) {
  switch (a.n_more) {
    case 0: return launch_n<T, 1>(a, s);
    case 1: return launch_n<T, 2>(a, s);
    case 2: return launch_n<T, 3>(a, s);
    case 3: return launch_n<T, 4>(a, s);
    default: return MTFM_E_UNSUPPORTED;
  }
}

}  // namespace

mtfm_status launch_gln(const GlnArgs& a, int dtype, hipStream_t s) {
  if (a.rows <= 0) return MTFM_OK;
  if (a.D % 64 != 0 || a.n_more < 0 || a.n_more > 3 || (a.xlist && a.xdiv < 1)) return MTFM_E_UNSUPPORTED;
  for (int o = 0; o < a.n_more; ++o)
    if (!a.y_more[o] || !a.gamma_more[o] || !a.beta_more[o]) return MTFM_E_NULL;
  return dtype == MTFM_BF16 ? launch_t<bf16>(a, s) : launch_t<float>(a, s);
}
