// Masked pointwise-SiLU attention kernels for gfx950.
//
// bf16 kernel: one workgroup per (query tile slice, KV group g) with one wave
// per query head of the group (r waves).  The group's K and V tiles (64 keys
// x 64 dims) are staged once in LDS and shared by the r heads ([explainer]
// §4.1 GQA: r query heads share a KV head).  Per key tile each wave computes
// S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (fp32 accumulate), applies SiLU
// pointwise in registers, rounds P to bf16 and accumulates O += P V on MFMA.
// The S^T accumulator layout (lane = query, registers = keys) is used
// directly as the A operand of P V once V's key order is permuted to match,
// so P never leaves registers.  V is transposed while being staged in LDS.
//
// Only key tiles the metadata marks visible are visited ([blog] §6.2: compute
// only key blocks holding a valid key); the mask compare runs only on mixed
// tiles and on a short last tile (separate straight-line tile bodies, so the
// unmasked body carries no compare).  T columns are never tiled ([blog] §6.2:
// the user-to-item direction is skipped): a T row's self term is one extra
// "diagonal" tile built from the query tile's own K/V rows.
//
// Throughput: every visible pair costs one exp and one reciprocal on the
// VALU (about as many cycles as its share of MFMA work), so the kernel keeps
// two waves per SIMD and issues the next key block's QK MFMAs next to the
// current block's SiLU.  QB = 2 gives each wave 64 queries (full layer);
// QB = 1 gives 32 (target layer: twice the workgroups for its few T rows).
//
// fp32 kernel: one thread per (query row, head), plain loops; the fp32
// correctness path.

#include "attn.h"

namespace {

constexpr int DH = 64;
constexpr int KS = DH + 8;  // K tile row stride in LDS (144 B)
constexpr int VS = 64 + 4;  // V^T tile row stride in LDS (136 B)

MTFM_DEV int xcd_remap(int bid, int nblocks) {
  const int q = nblocks >> 3, r = nblocks & 7;
  const int x = bid & 7, k = bid >> 3;
  return x * q + min(x, r) + k;
}

typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;

// 16-byte buffer load; offsets at or past the resource's record count read as zero.
MTFM_DEV bf16x8 buf_ld8(__amdgpu_buffer_rsrc_t r, int off) {
  const i32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return __builtin_bit_cast(bf16x8, v);
}

MTFM_DEV float silu_scaled(float s) {
  // s = x log2(e); returns SiLU(x) / ln2 = s / (1 + 2^-s)
  return s * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-s));
}

template <int R, int QB, bool PIPE>
__global__ __launch_bounds__(64 * R, 2) void attn_bf16_kernel(AttnArgs g) {
  constexpr int NT = 64 * R;
  constexpr int KPT = (512 + NT - 1) / NT;  // 16-B K chunks per thread per tile
  constexpr int VPT = (256 + NT - 1) / NT;  // V (key pair, 8 dims) items per thread per tile
  constexpr int SLICES = 2 / QB;            // workgroups per 64-row query tile
  __shared__ __attribute__((aligned(16))) bf16 Ks[2][64 * KS];
  __shared__ __attribute__((aligned(16))) bf16 Vs[2][DH * VS];
  __shared__ float rinv[32 * QB];

  const int nblocks = g.ntiles * g.G * SLICES;
  const int lb = xcd_remap(blockIdx.x, nblocks);
  const int slice = lb % SLICES;
  const int tile = (lb / SLICES) / g.G, grp = (lb / SLICES) % g.G;
  const int32_t* td = g.tiles + 8 * tile;
  const int u = td[TD_USER], row0 = td[TD_ROW0], tile_rows = td[TD_NROWS];
  const int full_end = td[TD_FULL_END], key_end = td[TD_END];
  const int qoff = slice * 32 * QB;
  const int nrows = min(32 * QB, tile_rows - qoff);
  if (nrows <= 0) return;                      // empty half of a short tile (whole workgroup)
  const int grow0 = td[TD_GROW0] + qoff, qrow0 = td[TD_QROW0] + qoff, urow0 = td[TD_UROW0];
  const int lctx = g.lens[3 * u] + g.lens[3 * u + 1];
  const bool has_diag = row0 + qoff + nrows > lctx;
  const int ntl = key_end + (has_diag ? 1 : 0);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = grp * R + wave;
  const int l32 = lane & 31, hi = lane >> 5;

  if (tid < 32 * QB) rinv[tid] = (tid < nrows) ? g.out_scale / (float)g.n[grow0 + tid] : 0.f;

  // Q fragments (B operand of S^T = K Q^T): query row qb*32 + l32, dims kk*16 + 8*hi + [0, 8)
  bf16x8 qf[QB][4];
  int plim[QB], selfq[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int qi = qb * 32 + l32;
    const bool ok = qi < nrows;
    const bf16* src = (const bf16*)g.q + (int64_t)(qrow0 + (ok ? qi : 0)) * g.ldq + h * DH + 8 * hi;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) qf[qb][kk] = ok ? *(const bf16x8*)(src + kk * 16) : bf16x8{};
    const int pp = ok ? g.p[grow0 + qi] : 0;
    plim[qb] = pp;
    selfq[qb] = ok ? (g.n[grow0 + qi] - pp) : 0;
  }

  // tile staging through buffer loads: the tile's first row and its number of
  // valid rows go into the (scalar) resource, the per-thread byte offsets are
  // loop-invariant, and rows past the valid count read as zero.
  // it < key_end -> context keys of the user; it == key_end -> the slice's own rows
  int koff[2][KPT], voff[2][VPT][2];
#pragma unroll
  for (int d = 0; d < 2; ++d) {
    const int64_t ldk = d ? g.ldkd : g.ldk, ldv = d ? g.ldvd : g.ldv;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int c = tid + NT * i;
      koff[d][i] = c < 512 ? (int)(((c >> 3) * ldk + grp * DH + (c & 7) * 8) * 2) : 0x7ffffff0;
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int c = tid + NT * i;
      const int j = 2 * (c & 31), vc = c >> 5;
      voff[d][i][0] = c < 256 ? (int)((j * ldv + grp * DH + vc * 8) * 2) : 0x7ffffff0;
      voff[d][i][1] = c < 256 ? (int)(((j + 1) * ldv + grp * DH + vc * 8) * 2) : 0x7ffffff0;
    }
  }
  bf16x8 rk[KPT], rv[VPT][2];
  auto load_tile = [&](int it) {
    const bool diag = it >= key_end;
    const int d = diag ? 1 : 0;
    const int64_t ldk = diag ? g.ldkd : g.ldk, ldv = diag ? g.ldvd : g.ldv;
    const int base = diag ? qrow0 : urow0 + it * 64;
    const int lim = diag ? nrows : min(64, lctx - it * 64);
    const bf16* kb = (diag ? (const bf16*)g.kd : (const bf16*)g.k) + (int64_t)base * ldk;
    const bf16* vb = (diag ? (const bf16*)g.vd : (const bf16*)g.v) + (int64_t)base * ldv;
    const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc((void*)kb, (short)0, (int)(lim * ldk * 2), 0x00020000);
    const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc((void*)vb, (short)0, (int)(lim * ldv * 2), 0x00020000);
#pragma unroll
    for (int i = 0; i < KPT; ++i) rk[i] = buf_ld8(kr, koff[d][i]);
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      rv[i][0] = buf_ld8(vr, voff[d][i][0]);
      rv[i][1] = buf_ld8(vr, voff[d][i][1]);
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int c = tid + NT * i;
      if (c < 512) *(bf16x8*)(&Ks[buf][(c >> 3) * KS + (c & 7) * 8]) = rk[i];
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int c = tid + NT * i;
      if (c >= 256) continue;
      const int jp = c & 31, vc = c >> 5;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        bf16x2 pr;
        pr[0] = rv[i][0][s];
        pr[1] = rv[i][1][s];
        *(bf16x2*)(&Vs[buf][(vc * 8 + s) * VS + 2 * jp]) = pr;
      }
    }
  };

  f32x16 o[QB][2];
#pragma unroll
  for (int a = 0; a < QB; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) o[a][b] = f32x16{};

  // One key tile of two 32-key blocks.  With PIPE the QK MFMAs of both blocks
  // are issued first (independent chains the scheduler can overlap with the
  // SiLU of the first block); without it each block runs QK -> SiLU -> PV,
  // which keeps fewer accumulators live.
  auto silu_pv = [&](const bf16* V, int kb, const f32x16* stb, auto masked_tag, const int* lim, const int* dsel) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    // P chunk c covers keys kb*32 + 16c + {4hi + t, 8 + 4hi + t : t < 4} in slot order
    bf16x8 pf[QB][2];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const int i = 8 * c + s;
          float pv = silu_scaled(stb[qb][i]);
          if constexpr (MASKED) {
            const int key = kb * 32 + 8 * (i >> 2) + 4 * hi + (i & 3);
            const bool vis = key < lim[qb] || key == dsel[qb];
            pv = vis ? pv : 0.f;
          }
          pf[qb][c][s] = (bf16)pv;
        }
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const bf16* vrow = &V[(nb * 32 + l32) * VS + kb * 32 + 16 * c + 4 * hi];
        const bf16x4 lo4 = *(const bf16x4*)(vrow);
        const bf16x4 hi4 = *(const bf16x4*)(vrow + 8);
        const bf16x8 vf = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          o[qb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pf[qb][c], vf, o[qb][nb], 0, 0, 0);
      }
  };
  auto qk = [&](const bf16* K, int kb, f32x16* stb) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) stb[qb] = f32x16{};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const bf16x8 af = *(const bf16x8*)(&K[(kb * 32 + l32) * KS + kk * 16 + 8 * hi]);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
        stb[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, qf[qb][kk], stb[qb], 0, 0, 0);
    }
  };
  auto tile_body = [&](const bf16* K, const bf16* V, auto masked_tag, const int* lim, const int* dsel) {
    if constexpr (PIPE) {
      f32x16 st[2][QB];
      qk(K, 0, st[0]);
      qk(K, 1, st[1]);
      silu_pv(V, 0, st[0], masked_tag, lim, dsel);
      silu_pv(V, 1, st[1], masked_tag, lim, dsel);
    } else {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        f32x16 st[QB];
        qk(K, kb, st);
        silu_pv(V, kb, st, masked_tag, lim, dsel);
      }
    }
  };

  if (ntl > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  for (int it = 0; it < ntl; ++it) {
    const int buf = it & 1;
    if (it + 1 < ntl) load_tile(it + 1);
    const bool diag = it >= key_end;
    const bool masked = diag || it >= full_end || (it + 1) * 64 > lctx;
    if (!masked) {
      tile_body(Ks[buf], Vs[buf], std::false_type{}, nullptr, nullptr);
    } else {
      int lim[QB], dsel[QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        lim[qb] = diag ? 0 : plim[qb] - it * 64;
        dsel[qb] = (diag && selfq[qb]) ? qb * 32 + l32 : -1;
      }
      tile_body(Ks[buf], Vs[buf], std::true_type{}, lim, dsel);
    }
    if (it + 1 < ntl) store_tile(buf ^ 1);
    __syncthreads();
  }

  // O layout: lane holds dim nb*32 + l32 of rows qb*32 + 8(i/4) + 4hi + i%4
  bf16* out = (bf16*)g.a;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int qi = qb * 32 + 8 * (i >> 2) + 4 * hi + (i & 3);
        if (qi < nrows)
          out[(int64_t)(qrow0 + qi) * g.lda + h * DH + nb * 32 + l32] = (bf16)(o[qb][nb][i] * rinv[qi]);
      }
}

// fp32 path: thread = (query row of the tile, head).
template <int D>
__global__ __launch_bounds__(64) void attn_f32_kernel(AttnArgs g) {
  const int tile = blockIdx.x, h = blockIdx.y;
  const int32_t* td = g.tiles + 8 * tile;
  const int nrows = td[TD_NROWS];
  const int grow0 = td[TD_GROW0], qrow0 = td[TD_QROW0], urow0 = td[TD_UROW0];
  const int qi = threadIdx.x;
  if (qi >= nrows) return;
  const int grp = h / (g.H / g.G);
  const float* q = (const float*)g.q + (int64_t)(qrow0 + qi) * g.ldq + h * D;
  float qv[D], acc[D];
  for (int c = 0; c < D; ++c) { qv[c] = q[c]; acc[c] = 0.f; }
  const int p = g.p[grow0 + qi];
  const int self = g.n[grow0 + qi] - p;
  auto visit = [&](const float* kr, const float* vr) {
    float s = 0.f;
    for (int c = 0; c < D; ++c) s = fmaf(qv[c], kr[c], s);
    const float w = s / (1.0f + exp2f(-s));
    for (int c = 0; c < D; ++c) acc[c] = fmaf(w, vr[c], acc[c]);
  };
  for (int j = 0; j < p; ++j)
    visit((const float*)g.k + (int64_t)(urow0 + j) * g.ldk + grp * D,
          (const float*)g.v + (int64_t)(urow0 + j) * g.ldv + grp * D);
  if (self)
    visit((const float*)g.kd + (int64_t)(qrow0 + qi) * g.ldkd + grp * D,
          (const float*)g.vd + (int64_t)(qrow0 + qi) * g.ldvd + grp * D);
  const float sc = g.out_scale / (float)g.n[grow0 + qi];
  float* out = (float*)g.a + (int64_t)(qrow0 + qi) * g.lda + h * D;
  for (int c = 0; c < D; ++c) out[c] = acc[c] * sc;
}

template <int QB>
mtfm_status launch_bf16(const AttnArgs& a, int r, hipStream_t s) {
  constexpr bool PIPE = QB == 1;
  const unsigned blocks = (unsigned)(a.ntiles * a.G * (2 / QB));
  switch (r) {
    case 1: attn_bf16_kernel<1, QB, PIPE><<<blocks, 64, 0, s>>>(a); break;
    case 2: attn_bf16_kernel<2, QB, PIPE><<<blocks, 128, 0, s>>>(a); break;
    case 4: attn_bf16_kernel<4, QB, PIPE><<<blocks, 256, 0, s>>>(a); break;
    case 8: attn_bf16_kernel<8, QB, PIPE><<<blocks, 512, 0, s>>>(a); break;
    default: return MTFM_E_UNSUPPORTED;
  }
  return MTFM_OK;
}

}  // namespace

mtfm_status launch_attention(const AttnArgs& a, int dtype, hipStream_t s) {
  if (a.ntiles <= 0) return MTFM_OK;
  const int r = a.H / a.G;
  if (dtype == MTFM_BF16) {
    if (a.dh != 64) return MTFM_E_UNSUPPORTED;
    mtfm_status st = a.half_tiles ? launch_bf16<1>(a, r, s) : launch_bf16<2>(a, r, s);
    if (st != MTFM_OK) return st;
  } else {
    dim3 grid((unsigned)a.ntiles, (unsigned)a.H);
    if (a.dh == 32) attn_f32_kernel<32><<<grid, 64, 0, s>>>(a);
    else if (a.dh == 64) attn_f32_kernel<64><<<grid, 64, 0, s>>>(a);
    else return MTFM_E_UNSUPPORTED;
  }
  MTFM_LAUNCH_CHECK("attention");
  return MTFM_OK;
}
