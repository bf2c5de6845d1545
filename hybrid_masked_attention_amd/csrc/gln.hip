// Group LayerNorm kernels: one wave per row, the row held in registers
// (D / 64 contiguous values per lane, moved as 16-byte vectors), two-pass
// mean and variance in fp32, type-indexed affine, optional multiplicative
// gate.  HBM-bound: each row is read once and written once.

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

template <typename T, int VPL>
__global__ __launch_bounds__(256) void gln_kernel(GlnArgs a) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= a.rows) return;
  float v[VPL];
  load_row<T, VPL>((const T*)a.x + (int64_t)row * a.ldx + lane * VPL, v);
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < VPL; ++j) s += v[j];
  const float mean = wave_sum(s) / (float)a.D;
  float q = 0.f;
#pragma unroll
  for (int j = 0; j < VPL; ++j) { v[j] -= mean; q += v[j] * v[j]; }
  const float rstd = rsqrtf(wave_sum(q) / (float)a.D + a.eps);
  const int t = a.type ? a.type[row] : a.type_const;
  float gm[VPL], bt[VPL];
  load_row<float, VPL>(a.gamma + t * a.D + lane * VPL, gm);
  load_row<float, VPL>(a.beta + t * a.D + lane * VPL, bt);
#pragma unroll
  for (int j = 0; j < VPL; ++j) v[j] = v[j] * rstd * gm[j] + bt[j];
  if (a.gate) {
    float g[VPL];
    load_row<T, VPL>((const T*)a.gate + (int64_t)row * a.ldg + lane * VPL, g);
#pragma unroll
    for (int j = 0; j < VPL; ++j) v[j] *= g[j];
  }
  store_row<T, VPL>((T*)a.y + (int64_t)row * a.ldy + lane * VPL, v);
}

template <typename T>
mtfm_status launch_t(const GlnArgs& a, hipStream_t s) {
  const unsigned blocks = (unsigned)((a.rows + 3) / 4);
  switch (a.D / 64) {
    case 1: gln_kernel<T, 1><<<blocks, 256, 0, s>>>(a); break;
    case 2: gln_kernel<T, 2><<<blocks, 256, 0, s>>>(a); break;
    case 4: gln_kernel<T, 4><<<blocks, 256, 0, s>>>(a); break;
    case 8: gln_kernel<T, 8><<<blocks, 256, 0, s>>>(a); break;
    case 16: gln_kernel<T, 16><<<blocks, 256, 0, s>>>(a); break;
    default: return MTFM_E_UNSUPPORTED;
  }
  MTFM_LAUNCH_CHECK("gln");
  return MTFM_OK;
}

}  // namespace

mtfm_status launch_gln(const GlnArgs& a, int dtype, hipStream_t s) {
  if (a.rows <= 0) return MTFM_OK;
  if (a.D % 64 != 0) return MTFM_E_UNSUPPORTED;
  return dtype == MTFM_BF16 ? launch_t<bf16>(a, s) : launch_t<float>(a, s);
}
