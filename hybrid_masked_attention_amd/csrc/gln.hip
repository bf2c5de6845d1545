// Group LayerNorm kernels: one wave per row, the row held in registers
// (D / 64 contiguous values per lane, loaded as vectors), two-pass mean and
// variance in fp32, type-indexed affine, optional multiplicative gate.
// HBM-bound: each row is read once and written once.

#include "gln.h"

namespace {

template <typename T, int VPL>
__global__ __launch_bounds__(256) void gln_kernel(GlnArgs a) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= a.rows) return;
  const T* x = (const T*)a.x + (int64_t)row * a.ldx + lane * VPL;
  float v[VPL];
#pragma unroll
  for (int j = 0; j < VPL; ++j) v[j] = to_f32(x[j]);
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < VPL; ++j) s += v[j];
  const float mean = wave_sum(s) / (float)a.D;
  float q = 0.f;
#pragma unroll
  for (int j = 0; j < VPL; ++j) { v[j] -= mean; q += v[j] * v[j]; }
  const float rstd = rsqrtf(wave_sum(q) / (float)a.D + a.eps);
  const int t = a.type ? a.type[row] : a.type_const;
  const float* gm = a.gamma + t * a.D + lane * VPL;
  const float* bt = a.beta + t * a.D + lane * VPL;
  T* y = (T*)a.y + (int64_t)row * a.ldy + lane * VPL;
  const T* gate = a.gate ? (const T*)a.gate + (int64_t)row * a.ldg + lane * VPL : nullptr;
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    float o = v[j] * rstd * gm[j] + bt[j];
    if (gate) o *= to_f32(gate[j]);
    y[j] = from_f32<T>(o);
  }
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
