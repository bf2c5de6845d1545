// Projection GEMMs: bf16 MFMA (gfx950 v_mfma_f32_32x32x16_bf16, fp32
// accumulation) with fused epilogues, and an fp32 FMA kernel for the fp32
// correctness path.
//
// bf16 kernel: 256 threads = 4 waves in a 2 x 2 grid, block tile 128 x 128,
// each wave 64 x 64 = 2 x 2 MFMA tiles of 32 x 32; K steps of 32 staged in LDS,
// double buffered with register prefetch of the next step.  Block ids are
// remapped so that consecutive logical tiles (which share A rows) land on the
// same XCD and hit its L2.

#include "gemm.h"

namespace {

constexpr int BM = 128, BN = 128, BK = 32, LDS_STRIDE = BK + 8;  // +16 B per row against bank conflicts

MTFM_DEV int64_t map_row(const RowMap& r, int m) {
  return (int64_t)(r.list ? r.list[m] : m * r.mul) + r.add;
}

// Logical block index such that blocks sharing an XCD (hardware dispatches
// consecutive workgroup ids round-robin over 8 XCDs) get consecutive ids.
MTFM_DEV int xcd_remap(int bid, int nblocks) {
  const int q = nblocks >> 3, r = nblocks & 7;
  const int x = bid & 7, k = bid >> 3;
  return x * q + min(x, r) + k;
}

template <typename T>
MTFM_DEV const T* b_row_ptr(const GemmArgs& g, int z, int n) {
  if (n < g.bn[0]) return (const T*)g.B[0] + (int64_t)z * g.bz[0] + (int64_t)n * g.ldb;
  n -= g.bn[0];
  if (n < g.bn[1]) return (const T*)g.B[1] + (int64_t)z * g.bz[1] + (int64_t)n * g.ldb;
  n -= g.bn[1];
  return (const T*)g.B[2] + (int64_t)z * g.bz[2] + (int64_t)n * g.ldb;
}

template <typename T>
MTFM_DEV void epilogue_store(const GemmArgs& g, const RowMap& cmap, int m, int n, float acc) {
  const int64_t crow = map_row(cmap, m);
  if (g.epi == EPI_SILU_SPLIT) {
    const float v = acc / (1.0f + __expf(-acc));
    int r = 0;
    while (r < 3 && n >= g.cend[r]) ++r;
    const int c0 = r ? g.cend[r - 1] : 0;
    ((T*)g.dst[r])[crow * g.ld[r] + (n - c0)] = from_f32<T>(v * g.scale[r]);
  } else if (g.epi == EPI_RESID) {
    const float res = to_f32(((const T*)g.resid)[crow * g.ldr + n]);
    ((T*)g.out)[crow * g.ldo + n] = from_f32<T>(acc + res);
  } else if (g.epi == EPI_STORE_F32) {
    float* o = (float*)g.out + crow * g.ldo + n;
    *o = g.accumulate ? *o + acc : acc;
  } else {
    ((T*)g.out)[crow * g.ldo + n] = from_f32<T>(acc);
  }
}

__global__ __launch_bounds__(256) void gemm_bf16_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) bf16 As[2][BM * LDS_STRIDE];
  __shared__ __attribute__((aligned(16))) bf16 Bs[2][BN * LDS_STRIDE];

  const int z = blockIdx.z;
  const int n_mt = (g.M + BM - 1) / BM, n_nt = (g.N + BN - 1) / BN;
  const int lb = xcd_remap(blockIdx.x, n_mt * n_nt);
  const int mt = lb / n_nt, nt = lb % n_nt;
  const int m0 = mt * BM, n0 = nt * BN;
  RowMap amap = g.amap; amap.add += z * g.amap_zadd;
  RowMap cmap = g.cmap; cmap.add += z * g.cmap_zadd;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // each thread moves 2 x 16 B of A and 2 x 16 B of B per K step
  const bf16* a_src[2];
  const bf16* b_src[2];
  int lds_off[2];
  for (int i = 0; i < 2; ++i) {
    const int c = tid + 256 * i;
    const int row = c >> 2, kc = c & 3;
    lds_off[i] = row * LDS_STRIDE + kc * 8;
    const int m = m0 + row, n = n0 + row;
    a_src[i] = (m < g.M) ? (const bf16*)g.A + map_row(amap, m) * g.lda + kc * 8 : nullptr;
    b_src[i] = (n < g.N) ? b_row_ptr<bf16>(g, z, n) + kc * 8 : nullptr;
  }
  const bf16x8 zero8 = {};
  bf16x8 ra[2], rb[2];
  auto load_step = [&](int k0) {
    for (int i = 0; i < 2; ++i) {
      ra[i] = a_src[i] ? *(const bf16x8*)(a_src[i] + k0) : zero8;
      rb[i] = b_src[i] ? *(const bf16x8*)(b_src[i] + k0) : zero8;
    }
  };
  auto store_step = [&](int buf) {
    for (int i = 0; i < 2; ++i) {
      *(bf16x8*)(&As[buf][lds_off[i]]) = ra[i];
      *(bf16x8*)(&Bs[buf][lds_off[i]]) = rb[i];
    }
  };

  f32x16 acc[2][2];
  for (int a = 0; a < 2; ++a)
    for (int b = 0; b < 2; ++b) acc[a][b] = f32x16{};

  const int nk = g.K / BK;
  load_step(0);
  store_step(0);
  __syncthreads();
  const int fr = lane & 31, fk = (lane >> 5) * 8;
  for (int ks = 0; ks < nk; ++ks) {
    const int buf = ks & 1;
    if (ks + 1 < nk) load_step((ks + 1) * BK);
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      bf16x8 af[2], bfr[2];
      for (int mb = 0; mb < 2; ++mb)
        af[mb] = *(const bf16x8*)(&As[buf][(wm * 64 + mb * 32 + fr) * LDS_STRIDE + kk * 16 + fk]);
      for (int nb = 0; nb < 2; ++nb)
        bfr[nb] = *(const bf16x8*)(&Bs[buf][(wn * 64 + nb * 32 + fr) * LDS_STRIDE + kk * 16 + fk]);
      for (int mb = 0; mb < 2; ++mb)
        for (int nb = 0; nb < 2; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mb], bfr[nb], acc[mb][nb], 0, 0, 0);
    }
    if (ks + 1 < nk) store_step(buf ^ 1);
    __syncthreads();
  }

  // C layout of a 32x32 MFMA tile: lane l holds column l%32, rows 8(i/4) + 4(l/32) + i%4
  for (int mb = 0; mb < 2; ++mb)
    for (int nb = 0; nb < 2; ++nb)
      for (int i = 0; i < 16; ++i) {
        const int m = m0 + wm * 64 + mb * 32 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
        const int n = n0 + wn * 64 + nb * 32 + (lane & 31);
        if (m < g.M && n < g.N) epilogue_store<bf16>(g, cmap, m, n, acc[mb][nb][i]);
      }
}

// fp32 path: one thread per output element (tiny correctness configs).
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs g) {
  const int z = blockIdx.z;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)g.M * g.N) return;
  const int m = (int)(idx / g.N), n = (int)(idx % g.N);
  RowMap amap = g.amap; amap.add += z * g.amap_zadd;
  RowMap cmap = g.cmap; cmap.add += z * g.cmap_zadd;
  const float* a = (const float*)g.A + map_row(amap, m) * g.lda;
  const float* b = b_row_ptr<float>(g, z, n);
  float acc = 0.f;
  for (int k = 0; k < g.K; ++k) acc = fmaf(a[k], b[k], acc);
  epilogue_store<float>(g, cmap, m, n, acc);
}

}  // namespace

mtfm_status launch_gemm(const GemmArgs& g, int dtype, hipStream_t s) {
  if (g.M <= 0 || g.N <= 0 || g.groups <= 0) return MTFM_OK;
  if (dtype == MTFM_BF16) {
    if (g.K % BK != 0) return MTFM_E_UNSUPPORTED;
    const int blocks = ((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN);
    gemm_bf16_kernel<<<dim3(blocks, 1, g.groups), 256, 0, s>>>(g);
  } else {
    const int64_t total = (int64_t)g.M * g.N;
    gemm_f32_kernel<<<dim3((unsigned)((total + 255) / 256), 1, g.groups), 256, 0, s>>>(g);
  }
  MTFM_LAUNCH_CHECK("gemm");
  return MTFM_OK;
}
