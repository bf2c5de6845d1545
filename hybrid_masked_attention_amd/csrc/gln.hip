// Group LayerNorm kernels: one wave per few rows, each row held in registers
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
// whole vectors, element by element otherwise.  Stores are non-temporal: the
// rows stream out and are read back by another kernel, not from this one's
// cache lines.
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

template <typename T, int VPL, bool NT>
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
      if constexpr (NT) __builtin_nontemporal_store(w, &q[c]);
      else q[c] = w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < VPL; ++j) p[j] = from_f32<T>(v[j]);
  }
}

// One wave per RPW consecutive rows: every row's loads are issued before any
// reduction, so a wave keeps RPW x 64 x 16 bytes in flight (the kernel streams
// HBM; one row per wave left it latency-bound).
template <typename T, int VPL, int NOUT, int RPW, bool GATE, bool PARTS = false, bool NT = true>
__global__ __launch_bounds__(256) void gln_kernel(GlnArgs a) {
  const int row0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * RPW;
  const int lane = threadIdx.x & 63;
  if (row0 >= a.rows) return;
  int64_t xrow[RPW];
  bool ok[RPW];
  float v[RPW][VPL], g[GATE ? RPW : 1][VPL];
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const int row = row0 + r;
    ok[r] = row < a.rows;
    const int rr = ok[r] ? row : row0;   // a row past the end re-reads the first (never stored)
    xrow[r] = a.xlist ? (int64_t)a.xlist[rr / a.xdiv] + rr % a.xdiv : rr;
    if constexpr (PARTS) load_row<float, VPL>(a.x_parts + xrow[r] * a.ldx + lane * VPL, v[r]);
    else load_row<T, VPL>((const T*)a.x + xrow[r] * a.ldx + lane * VPL, v[r]);
    if constexpr (GATE) load_row<T, VPL>((const T*)a.gate + (int64_t)rr * a.ldg + lane * VPL, g[r]);
  }
  if constexpr (PARTS) {
    // the other partials, added in order; two parts of every row in flight at once
    for (int k = 1; k < a.n_parts; k += 2) {
      const bool two = k + 1 < a.n_parts;
      float w[2][RPW][VPL];
#pragma unroll
      for (int r = 0; r < RPW; ++r) {
        const float* base = a.x_parts + xrow[r] * a.ldx + lane * VPL;
        load_row<float, VPL>(base + k * a.part_stride, w[0][r]);
        load_row<float, VPL>(base + (two ? k + 1 : k) * a.part_stride, w[1][r]);
      }
#pragma unroll
      for (int r = 0; r < RPW; ++r)
#pragma unroll
        for (int j = 0; j < VPL; ++j) {
          v[r][j] += w[0][r][j];
          if (two) v[r][j] += w[1][r][j];
        }
    }
  }
  float mean[RPW], rstd[RPW];
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < VPL; ++j) s += v[r][j];
    mean[r] = s;
  }
#pragma unroll
  for (int r = 0; r < RPW; ++r) mean[r] = wave_sum(mean[r]) / (float)a.D;
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    float q = 0.f;
#pragma unroll
    for (int j = 0; j < VPL; ++j) { v[r][j] -= mean[r]; q += v[r][j] * v[r][j]; }
    rstd[r] = q;
  }
#pragma unroll
  for (int r = 0; r < RPW; ++r) rstd[r] = rsqrtf(wave_sum(rstd[r]) / (float)a.D + a.eps);
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    if (!ok[r]) continue;
    const int t = a.type ? a.type[xrow[r]] : a.type_const;
#pragma unroll
    for (int o = 0; o < NOUT; ++o) {
      const bool zero = ((a.zero_t >> o) & 1) && t == TT_T;
      const float* gamma = o ? a.gamma_more[o - 1] : a.gamma;
      const float* beta = o ? a.beta_more[o - 1] : a.beta;
      T* y = (T*)(o ? a.y_more[o - 1] : a.y);
      float gm[VPL], bt[VPL], w[VPL];
      load_row<float, VPL>(gamma + t * a.D + lane * VPL, gm);
      load_row<float, VPL>(beta + t * a.D + lane * VPL, bt);
#pragma unroll
      for (int j = 0; j < VPL; ++j) {
        w[j] = zero ? 0.f : v[r][j] * rstd[r] * gm[j] + bt[j];
        if constexpr (GATE) w[j] *= g[r][j];
      }
      store_row<T, VPL, NT>(y + (int64_t)(row0 + r) * a.ldy + lane * VPL, w);
    }
  }
}

template <typename T, int NOUT, bool GATE, bool PARTS, bool NT>
mtfm_status launch_nt(const GlnArgs& a, hipStream_t s) {
  constexpr int RPW = 4;
  const unsigned blocks = (unsigned)((a.rows + 4 * RPW - 1) / (4 * RPW));
  switch (a.D / 64) {
    case 1: gln_kernel<T, 1, NOUT, RPW, GATE, PARTS, NT><<<blocks, 256, 0, s>>>(a); break;
    case 2: gln_kernel<T, 2, NOUT, RPW, GATE, PARTS, NT><<<blocks, 256, 0, s>>>(a); break;
    case 4: gln_kernel<T, 4, NOUT, RPW, GATE, PARTS, NT><<<blocks, 256, 0, s>>>(a); break;
    case 8: gln_kernel<T, 8, NOUT, RPW, GATE, PARTS, NT><<<blocks, 256, 0, s>>>(a); break;
    case 16: gln_kernel<T, 16, NOUT, RPW, GATE, PARTS, NT><<<blocks, 256, 0, s>>>(a); break;
    default: return MTFM_E_UNSUPPORTED;
  }
  MTFM_LAUNCH_CHECK("gln");
  return MTFM_OK;
}

// Cached stores only for single-output forms asked for them (small T-row
// outputs read at once); every other form stores non-temporally.
template <typename T, int NOUT, bool GATE, bool PARTS = false>
mtfm_status launch_n(const GlnArgs& a, hipStream_t s) {
  if constexpr (NOUT == 1) {
    if (a.temporal) return launch_nt<T, NOUT, GATE, PARTS, false>(a, s);
  }
  return launch_nt<T, NOUT, GATE, PARTS, true>(a, s);
}

// The gate goes with a single output (the gated LayerNorm after attention);
// several outputs only for the ungated context normalisation.
template <typename T>
mtfm_status launch_t(const GlnArgs& a, hipStream_t s) {
  if (a.gate) {
    if (a.n_more != 0) return MTFM_E_UNSUPPORTED;
    return a.x_parts ? launch_n<T, 1, true, true>(a, s) : launch_n<T, 1, true>(a, s);
  }
  switch (a.n_more) {
    case 0: return launch_n<T, 1, false>(a, s);
    case 1: return launch_n<T, 2, false>(a, s);
    case 2: return launch_n<T, 3, false>(a, s);
    case 3: return launch_n<T, 4, false>(a, s);
    default: return MTFM_E_UNSUPPORTED;
  }
}

}  // namespace

mtfm_status launch_gln(const GlnArgs& a, int dtype, hipStream_t s) {
  if (a.rows <= 0) return MTFM_OK;
  if (a.D % 64 != 0 || a.n_more < 0 || a.n_more > 3 || (a.xlist && a.xdiv < 1)) return MTFM_E_UNSUPPORTED;
  for (int o = 0; o < a.n_more; ++o)
    if (!a.y_more[o] || !a.gamma_more[o] || !a.beta_more[o]) return MTFM_E_NULL;
  if (a.x_parts && (!a.gate || a.n_parts < 1 || ((uintptr_t)a.x_parts & 15) || a.ldx % 4 != 0 ||
                    a.part_stride % 4 != 0))
    return MTFM_E_UNSUPPORTED;
  return dtype == MTFM_BF16 ? launch_t<bf16>(a, s) : launch_t<float>(a, s);
}
