// Projection GEMMs: bf16 MFMA (gfx950 v_mfma_f32_32x32x16_bf16, fp32
// accumulation) with fused epilogues, and an fp32 FMA kernel for the fp32
// correctness path.
//
// bf16 kernel: 256 threads = 4 waves in a 2 x 2 grid, block tile 128 x 128,
// each wave 64 x 64 = 2 x 2 MFMA tiles of 32 x 32; K steps of 64 staged in LDS,
// double buffered with register prefetch of the next step, two workgroups per
// CU.  The MFMA computes C^T (weights as the A operand) so that each lane ends
// up holding four consecutive output columns of one row: epilogue stores are
// 8 bytes wide and the column segment (U / Q / K|V) is uniform per 32-column
// block.  Block ids are remapped so that consecutive logical tiles (which share
// A rows) land on the same XCD and hit its L2.

#include <algorithm>

#include "gemm.h"

namespace {

constexpr int BM = 128, BN = 128, BK = 64, LDS_STRIDE = BK + 8;  // +16 B per row against bank conflicts
constexpr float kLog2eF = 1.44269504088896340736f;

MTFM_DEV int64_t map_row(const RowMap& r, int m) {
  if (r.list) {
    if (r.div > 1) return (int64_t)r.list[m / r.div] + m % r.div + r.add;
    return (int64_t)r.list[m] + r.add;
  }
  return (int64_t)m * r.mul + r.add;
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

MTFM_DEV float silu_fast(float x) {
  return x * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-x * kLog2eF));
}

// Scalar epilogue (fp32 path).
template <typename T>
MTFM_DEV void epilogue_one(const GemmArgs& g, const RowMap& cmap, int m, int n, float acc) {
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

template <int EPI>
MTFM_DEV void gemm_epilogue(const GemmArgs& g, const RowMap& cmap, const f32x16 (&acc)[2][2], int m0, int n0, int wm,
                            int wn, int l32, int hi) {
  // C^T layout of a 32x32 tile: lane holds row m = l32 and columns
  // 8(i/4) + 4hi + (i%4): registers 4j..4j+3 are four consecutive columns.
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    const int m = m0 + wm * 64 + mb * 32 + l32;
    if (m >= g.M) continue;
    const int64_t crow = map_row(cmap, m);
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int nblk = n0 + wn * 64 + nb * 32;
      if (nblk >= g.N) continue;
      if constexpr (EPI == EPI_SILU_SPLIT) {
        int r = 0;
        while (r < 3 && nblk >= g.cend[r]) ++r;
        const int c0 = r ? g.cend[r - 1] : 0;
        const float sc = g.scale[r];
        bf16* dst = (bf16*)g.dst[r] + crow * g.ld[r] + (nblk - c0) + 4 * hi;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          bf16x4 v;
#pragma unroll
          for (int t = 0; t < 4; ++t) v[t] = (bf16)(silu_fast(acc[nb][mb][4 * j + t]) * sc);
          *(bf16x4*)(dst + 8 * j) = v;
        }
        if (g.pre) {
          bf16* pd = (bf16*)g.pre + crow * g.ldpre + nblk + 4 * hi;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            bf16x4 v;
#pragma unroll
            for (int t = 0; t < 4; ++t) v[t] = (bf16)acc[nb][mb][4 * j + t];
            *(bf16x4*)(pd + 8 * j) = v;
          }
        }
      } else if constexpr (EPI == EPI_RESID) {
        const bf16* res = (const bf16*)g.resid + crow * g.ldr + nblk + 4 * hi;
        bf16* dst = (bf16*)g.out + crow * g.ldo + nblk + 4 * hi;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const bf16x4 rr = *(const bf16x4*)(res + 8 * j);
          bf16x4 v;
#pragma unroll
          for (int t = 0; t < 4; ++t) v[t] = (bf16)(acc[nb][mb][4 * j + t] + (float)rr[t]);
          *(bf16x4*)(dst + 8 * j) = v;
        }
      } else if constexpr (EPI == EPI_STORE_F32) {
        float* dst = (float*)g.out + crow * g.ldo + nblk + 4 * hi;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          f32x4 v;
          if (g.accumulate) v = *(const f32x4*)(dst + 8 * j);
          else v = f32x4{};
#pragma unroll
          for (int t = 0; t < 4; ++t) v[t] += acc[nb][mb][4 * j + t];
          *(f32x4*)(dst + 8 * j) = v;
        }
      } else {
        bf16* dst = (bf16*)g.out + crow * g.ldo + nblk + 4 * hi;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          bf16x4 v;
#pragma unroll
          for (int t = 0; t < 4; ++t) v[t] = (bf16)acc[nb][mb][4 * j + t];
          *(bf16x4*)(dst + 8 * j) = v;
        }
      }
    }
  }
}

// Persistent: gridDim.x workgroups (two per CU) walk the tiles of all groups;
// the (tile, K step) sequence of a workgroup is one software pipeline, so the
// next tile's first operands are being fetched while the current tile's
// epilogue runs.
template <int EPI>
__global__ __launch_bounds__(256, 2) void gemm_bf16_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) bf16 As[2][BM * LDS_STRIDE];
  __shared__ __attribute__((aligned(16))) bf16 Bs[2][BN * LDS_STRIDE];

  const int n_mt = (g.M + BM - 1) / BM, n_nt = (g.N + BN - 1) / BN;
  const int tiles_per_group = n_mt * n_nt;
  const int n_tiles = tiles_per_group * g.groups;
  const int nk = g.K / BK;
  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int my_tiles = wg < n_tiles ? (n_tiles - 1 - wg) / gridDim.x + 1 : 0;
  const int total = my_tiles * nk;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, hi = lane >> 5;

  // per-thread staging slots: 4 x 16 B of A and of B per K step
  int lds_off[4];
  const int kc = tid & 7;
#pragma unroll
  for (int i = 0; i < 4; ++i) lds_off[i] = ((tid + 256 * i) >> 3) * LDS_STRIDE + kc * 8;

  const bf16* a_src[4];
  const bf16* b_src[4];
  int cur_tile = -1;
  auto tile_setup = [&](int t) {   // operand row pointers of tile t (k = 0)
    if (t == cur_tile) return;
    cur_tile = t;
    const int z = t / tiles_per_group, tt = t % tiles_per_group;
    const int m0 = (tt / n_nt) * BM, n0 = (tt % n_nt) * BN;
    RowMap amap = g.amap; amap.add += z * g.amap_zadd;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = (tid + 256 * i) >> 3;
      const int m = m0 + row, n = n0 + row;
      a_src[i] = (m < g.M) ? (const bf16*)g.A + map_row(amap, m) * g.lda + kc * 8 : nullptr;
      b_src[i] = (n < g.N) ? b_row_ptr<bf16>(g, z, n) + kc * 8 : nullptr;
    }
  };
  bf16x8 ra[4], rb[4];
  auto load_step = [&](int s) {
    const int t = wg + (s / nk) * gridDim.x, k0 = (s % nk) * BK;
    tile_setup(t);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ra[i] = a_src[i] ? *(const bf16x8*)(a_src[i] + k0) : bf16x8{};
      rb[i] = b_src[i] ? *(const bf16x8*)(b_src[i] + k0) : bf16x8{};
    }
  };
  auto store_step = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *(bf16x8*)(&As[buf][lds_off[i]]) = ra[i];
      *(bf16x8*)(&Bs[buf][lds_off[i]]) = rb[i];
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = f32x16{};

  if (total > 0) {
    load_step(0);
    store_step(0);
  }
  __syncthreads();
  for (int s = 0; s < total; ++s) {
    const int buf = s & 1;
    if (s + 1 < total) load_step(s + 1);
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      bf16x8 xf[2], wf[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
        xf[mb] = *(const bf16x8*)(&As[buf][(wm * 64 + mb * 32 + l32) * LDS_STRIDE + kk * 16 + 8 * hi]);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
        wf[nb] = *(const bf16x8*)(&Bs[buf][(wn * 64 + nb * 32 + l32) * LDS_STRIDE + kk * 16 + 8 * hi]);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
          acc[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[nb], xf[mb], acc[nb][mb], 0, 0, 0);
    }
    if (s % nk == nk - 1) {   // tile finished: write it, reset the accumulators
      const int t = wg + (s / nk) * gridDim.x;
      const int z = t / tiles_per_group, tt = t % tiles_per_group;
      RowMap cmap = g.cmap; cmap.add += z * g.cmap_zadd;
      gemm_epilogue<EPI>(g, cmap, acc, (tt / n_nt) * BM, (tt % n_nt) * BN, wm, wn, l32, hi);
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[a][b] = f32x16{};
    }
    if (s + 1 < total) store_step(buf ^ 1);
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Weight-gradient GEMM.  Block tile 128 (m) x 128 (n), 32 rows of r per step:
// each thread loads a pair of rows r, r+1 at 8 consecutive m (or n) and
// writes them transposed into LDS as [m][r] so the MFMA operands (8
// consecutive r per lane) are 16-byte reads.  Grid: tiles x splits of r; a
// split writes its partial tile, the reduction adds splits in order.
constexpr int TBK = 32, T_STRIDE = TBK + 8;
constexpr int TN_ROWS_PER_SPLIT = 2048;

__global__ __launch_bounds__(256, 2) void gemm_tn_kernel(GemmTNArgs g, int n_split) {
  __shared__ __attribute__((aligned(16))) bf16 As[BM * T_STRIDE];
  __shared__ __attribute__((aligned(16))) bf16 Bs[BN * T_STRIDE];
  const int z = blockIdx.z;
  const int n_mt = (g.M + BM - 1) / BM, n_nt = (g.N + BN - 1) / BN;
  const int tiles = n_mt * n_nt;
  const int split = blockIdx.x / tiles, t = blockIdx.x % tiles;
  const int mt = t / n_nt, nt = t % n_nt;
  const int m0 = mt * BM, n0 = nt * BN;
  RowMap amap = g.amap; amap.add += z * g.amap_zadd;
  RowMap bmap = g.bmap; bmap.add += z * g.bmap_zadd;
  const bf16* A = (const bf16*)g.A + (int64_t)z * g.a_zoff;
  const bf16* B = (const bf16*)g.B;
  const int r_begin = split * TN_ROWS_PER_SPLIT, r_end = min(g.R, r_begin + TN_ROWS_PER_SPLIT);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, hi = lane >> 5;
  // staging item: row pair rp (16 pairs per step), 8-column chunk cc (16 chunks of 128)
  const int rp = tid >> 4, cc = tid & 15;

  f32x16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = f32x16{};

  for (int r0 = r_begin; r0 < r_end; r0 += TBK) {
    bf16x8 av[2], bv[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int r = r0 + 2 * rp + e;
      const bool ok = r < r_end;
      const int m = m0 + cc * 8, n = n0 + cc * 8;
      av[e] = (ok && m < g.M) ? *(const bf16x8*)(A + map_row(amap, r) * g.lda + m) : bf16x8{};
      bv[e] = (ok && n < g.N) ? *(const bf16x8*)(B + map_row(bmap, r) * g.ldb + n) : bf16x8{};
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      bf16x2 pa, pb;
      pa[0] = av[0][s]; pa[1] = av[1][s];
      pb[0] = bv[0][s]; pb[1] = bv[1][s];
      *(bf16x2*)(&As[(cc * 8 + s) * T_STRIDE + 2 * rp]) = pa;
      *(bf16x2*)(&Bs[(cc * 8 + s) * T_STRIDE + 2 * rp]) = pb;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < TBK / 16; ++kk) {
      bf16x8 af[2], bfr[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
        af[mb] = *(const bf16x8*)(&As[(wm * 64 + mb * 32 + l32) * T_STRIDE + kk * 16 + 8 * hi]);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
        bfr[nb] = *(const bf16x8*)(&Bs[(wn * 64 + nb * 32 + l32) * T_STRIDE + kk * 16 + 8 * hi]);
      // C^T tiles: lane = m, registers = four consecutive n
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
          acc[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[nb], af[mb], acc[nb][mb], 0, 0, 0);
    }
  }
  float* P = g.partial + ((int64_t)z * n_split + split) * (int64_t)g.M * g.N;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    const int m = m0 + wm * 64 + mb * 32 + l32;
    if (m >= g.M) continue;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int nblk = n0 + wn * 64 + nb * 32;
      if (nblk >= g.N) continue;
      float* dst = P + (int64_t)m * g.N + nblk + 4 * hi;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f32x4 v;
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = acc[nb][mb][4 * j + q];
        *(f32x4*)(dst + 8 * j) = v;
      }
    }
  }
}

// C (+)= sum over splits of the partials, in split order.
__global__ __launch_bounds__(256) void gemm_tn_reduce_kernel(GemmTNArgs g, int n_split) {
  const int z = blockIdx.y;
  const int64_t mn = (int64_t)g.M * g.N;
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= mn) return;
  const float* P = g.partial + (int64_t)z * n_split * mn + i;
  f32x4 s = *(const f32x4*)P;
  for (int k = 1; k < n_split; ++k) {
    const f32x4 v = *(const f32x4*)(P + k * mn);
#pragma unroll
    for (int q = 0; q < 4; ++q) s[q] += v[q];
  }
  const int m = (int)(i / g.N), n = (int)(i % g.N);
  float* dst = g.C + (int64_t)z * g.c_zoff + (int64_t)m * g.ldc + n;
  if (g.accumulate) {
    const f32x4 o = *(const f32x4*)dst;
#pragma unroll
    for (int q = 0; q < 4; ++q) s[q] += o[q];
  }
  *(f32x4*)dst = s;
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
  epilogue_one<float>(g, cmap, m, n, acc);
}

}  // namespace

// Compute units of the current device (cached per device id).
int device_cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cached[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

int64_t gemm_tn_partial_elems(int32_t M, int32_t N, int32_t R, int32_t groups) {
  const int64_t n_split = std::max<int64_t>(1, (R + TN_ROWS_PER_SPLIT - 1) / TN_ROWS_PER_SPLIT);
  return n_split * (int64_t)M * N * groups;
}

mtfm_status launch_gemm_tn(const GemmTNArgs& g, hipStream_t s) {
  if (g.M <= 0 || g.N <= 0 || g.groups <= 0) return MTFM_OK;
  if (g.M % 8 != 0 || g.N % 32 != 0 || g.lda % 8 != 0 || g.ldb % 8 != 0 || g.ldc % 4 != 0)
    return MTFM_E_UNSUPPORTED;
  const int n_split = std::max(1, (g.R + TN_ROWS_PER_SPLIT - 1) / TN_ROWS_PER_SPLIT);
  if (gemm_tn_partial_elems(g.M, g.N, g.R, g.groups) > g.partial_elems) return MTFM_E_WORKSPACE;
  const int tiles = ((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN);
  gemm_tn_kernel<<<dim3(tiles * n_split, 1, g.groups), 256, 0, s>>>(g, n_split);
  MTFM_LAUNCH_CHECK("gemm_tn");
  const int64_t mn4 = ((int64_t)g.M * g.N) / 4;
  gemm_tn_reduce_kernel<<<dim3((unsigned)((mn4 + 255) / 256), g.groups), 256, 0, s>>>(g, n_split);
  MTFM_LAUNCH_CHECK("gemm_tn_reduce");
  return MTFM_OK;
}

mtfm_status launch_gemm(const GemmArgs& g, int dtype, hipStream_t s) {
  if (g.M <= 0 || g.N <= 0 || g.groups <= 0) return MTFM_OK;
  if (dtype == MTFM_BF16) {
    // 32-column blocks must not straddle an output segment; K a multiple of the K step
    if (g.K % BK != 0 || g.N % 32 != 0) return MTFM_E_UNSUPPORTED;
    if (g.epi == EPI_SILU_SPLIT)
      for (int r = 0; r < 4; ++r)
        if (g.cend[r] % 32 != 0) return MTFM_E_UNSUPPORTED;
    const int64_t tiles = (int64_t)((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN) * g.groups;
    const dim3 grid((unsigned)std::min<int64_t>(tiles, 2 * (int64_t)device_cu_count()), 1, 1);
    switch (g.epi) {
      case EPI_SILU_SPLIT: gemm_bf16_kernel<EPI_SILU_SPLIT><<<grid, 256, 0, s>>>(g); break;
      case EPI_RESID: gemm_bf16_kernel<EPI_RESID><<<grid, 256, 0, s>>>(g); break;
      case EPI_STORE_F32: gemm_bf16_kernel<EPI_STORE_F32><<<grid, 256, 0, s>>>(g); break;
      default: gemm_bf16_kernel<EPI_STORE><<<grid, 256, 0, s>>>(g); break;
    }
  } else {
    const int64_t total = (int64_t)g.M * g.N;
    gemm_f32_kernel<<<dim3((unsigned)((total + 255) / 256), 1, g.groups), 256, 0, s>>>(g);
  }
  MTFM_LAUNCH_CHECK("gemm");
  return MTFM_OK;
}
