// Masked pointwise-SiLU attention kernels for gfx950.
//
// bf16 kernel: one workgroup per (query tile slice, KV group g) with one wave
// per query head of the group (r waves).  The group's K and V tiles (64 keys
// x 64 dims) are shared by the r heads in LDS ([explainer] §4.1 GQA: r query
// heads share a KV head).  They arrive through a ring of LDS stages filled by
// buffer loads straight into LDS: K from its row-major rows, V from a
// transposed copy (V^T, written by the projection GEMM) whose keys are
// permuted within groups of 16.  Per 32-key block each wave computes
// S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (fp32 accumulate; lane = query,
// registers = keys), applies SiLU pointwise, rounds P to bf16 and accumulates
// O^T += V^T P^T on MFMA: the S^T registers are already the B operand in the
// permuted key order, so P never leaves registers and every fragment is one
// 16-byte LDS read.
//
// Key tiles are aligned to 64 packed rows (aligned DMA); a tile is visited
// only when it holds a key visible to some query of the slice ([blog] §6.2:
// compute only key blocks holding a valid key), and the mask compare runs only
// on tiles not entirely inside every query's visible prefix (separate
// straight-line bodies).  T columns are never tiled ([blog] §6.2: the
// user-to-item direction is skipped): a T row's self term is one extra
// "diagonal" tile built from the query slice's own K/V rows.
//
// Every visible pair costs one exp and one reciprocal on the VALU, so the
// kernel keeps two workgroups per CU to overlap one wave's SiLU with another's
// MFMAs.  QB = 1 gives each wave 32 queries, QB = 2 gives 64.
//
// fp32 kernel: one thread per (query row, head), plain loops; the fp32
// correctness path.

#include "attn.h"

namespace {

constexpr int DH = 64;

MTFM_DEV float silu_scaled(float s) {
  // s = x log2(e); returns SiLU(x) / ln2 = s / (1 + 2^-s)
  return s * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-s));
}

// K / V^T ring: stage = K tile (64 key rows x 128 B) + V^T tile (64 dim rows
// x 128 B); the 16-byte chunk c of LDS row r sits at slot c ^ ((r >> 1) & 7).
constexpr int A_TILE = 64 * 128;
constexpr int A_STAGE = 2 * A_TILE;

typedef __attribute__((address_space(3))) void lds_void;

MTFM_DEV int a_swz(int r) { return (r >> 1) & 7; }

MTFM_DEV void lds_dma16(__amdgpu_buffer_rsrc_t r, lds_void* dst, uint32_t voff) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, voff, 0, 0, 0);
#endif
}

// Buffer resource over a wave-uniform base and size.
MTFM_DEV __amdgpu_buffer_rsrc_t a_rsrc(const void* base, uint32_t bytes) {
  const uint64_t b = (uint64_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  return __builtin_amdgcn_make_buffer_rsrc((void*)(((uint64_t)hi << 32) | lo), (short)0,
                                           (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

template <int N> MTFM_DEV void a_wait_vm_lgkm() { __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0070); }
MTFM_DEV void a_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Slot of packed row r inside its aligned group of 16 (the P V key order).
MTFM_DEV int perm16(int r) { return (r & ~15) | (r & 3) | (((r >> 3) & 1) << 2) | (((r >> 2) & 1) << 3); }

// Ring depth and workgroups per CU: 32 queries per wave fit three workgroups
// (two-stage ring + diagonal tile, 48 KB), 64 queries per wave two (three
// stages, 64 KB).
template <int QB> struct AttnShape { static constexpr int AS = QB == 1 ? 2 : 3, WG_PER_CU = QB == 1 ? 3 : 2; };

template <int R, int QB>
// (the second bound is waves per SIMD: with one wave per head, fewer than four
// heads per group leave the SIMDs a wave per workgroup or less)
__global__ __launch_bounds__(64 * R, R >= 4 ? AttnShape<QB>::WG_PER_CU : 1) void attn_bf16_kernel(AttnArgs g) {
  constexpr int AS = AttnShape<QB>::AS;
  constexpr int NT = 64 * R;
  constexpr int CPW = 8 / R;                // 1 KB DMA chunks per wave per 8 KB tile
  constexpr int DMA_PER_TILE = 2 * CPW;     // K + V^T instructions per wave per tile
  constexpr int SLICES = 2 / QB;            // workgroups per 64-row query tile
  __shared__ __attribute__((aligned(1024))) char lds[AS * A_STAGE + A_STAGE];   // ring + diagonal tile
  char* const dlds = lds + AS * A_STAGE;

  const int nblocks = g.ntiles * g.G * SLICES;
  const int lb = xcd_remap(blockIdx.x, nblocks);
  const int slice = lb % SLICES;
  const int tile = (lb / SLICES) / g.G, grp = (lb / SLICES) % g.G;
  const int32_t* td = g.tiles + 8 * tile;
  const int u = td[TD_USER], row0 = td[TD_ROW0], tile_rows = td[TD_NROWS];
  const int qoff = slice * 32 * QB;
  const int nrows = min(32 * QB, tile_rows - qoff);
  if (nrows <= 0) return;                      // empty half of a short tile (whole workgroup)
  const int grow0 = td[TD_GROW0] + qoff, qrow0 = td[TD_QROW0] + qoff, urow0 = td[TD_UROW0];
  const int lctx = g.lens[3 * u] + g.lens[3 * u + 1];
  const bool has_diag = row0 + qoff + nrows > lctx;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = grp * R + wave;
  const int l32 = lane & 31, hi = lane >> 5;

  // Key tiles are aligned to 64 packed rows: tile it covers rows ts = T0 + 64 it
  // .. ts + 63.  The descriptor bounds the user's visible keys: rows below
  // urow0 + 64 full_end (capped at the context) are visible to every query of
  // the tile, none at or past urow0 + 64 end.
  const int T0 = urow0 & ~63;
  const int key_end = td[TD_END];
  const int kend = urow0 + min(64 * key_end, lctx);
  const int n_main = key_end > 0 ? (kend - T0 + 63) >> 6 : 0;
  const int kfull = urow0 + min(64 * td[TD_FULL_END], lctx);

  // DMA lanes: chunk c = 8 rows of 128 B; lane -> row 8c + lane/8, slot lane%8
  const int rin = lane >> 3, slot = lane & 7;
  uint32_t koff[CPW], voff[CPW];
#pragma unroll
  for (int i = 0; i < CPW; ++i) {
    const int r = (i * R + wave) * 8 + rin;
    const int c = slot ^ a_swz(r);
    koff[i] = (uint32_t)(r * g.ldk * 2 + grp * DH * 2 + c * 16);
    voff[i] = (uint32_t)((grp * DH + r) * g.ldvt * 2 + c * 16);
  }
  const bf16* kbase = (const bf16*)g.k;
  const bf16* vtbase = (const bf16*)g.vt;
  const int64_t vt_elems = (int64_t)g.G * DH * g.ldvt;
  // Tiles past the last one are issued as empty loads (zero-size resources), so
  // that the number of DMA instructions in flight is a constant at every wait.
  auto issue = [&](int it, int stage) {
    const bool real = it < n_main;
    const int ts = real ? T0 + it * 64 : T0;
    const int valid = real ? min(64, g.n_key_rows - ts) : 0;
    const __amdgpu_buffer_rsrc_t kr = a_rsrc(kbase + (int64_t)ts * g.ldk, (uint32_t)(max(valid, 0) * g.ldk * 2));
    const __amdgpu_buffer_rsrc_t vr = a_rsrc(vtbase + ts, real ? (uint32_t)((vt_elems - ts) * 2) : 0u);
    char* st = lds + stage * A_STAGE;
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      lds_dma16(kr, (lds_void*)(st + (i * R + wave) * 1024), koff[i]);
      lds_dma16(vr, (lds_void*)(st + A_TILE + (i * R + wave) * 1024), voff[i]);
    }
  };
#pragma unroll
  for (int s = 0; s < AS; ++s) issue(s, s);

  // Q fragments (B operand of S^T = K Q^T): query qb*32 + l32, dims kk*16 + 8*hi + [0, 8)
  // (all loads first, uses after: the counters drain in issue order)
  bf16x8 qf[QB][4];
  int pl[QB], nl[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int qi = qb * 32 + l32;
    const bool ok = qi < nrows;
    const int qr = ok ? qi : 0;
    const bf16* src = (const bf16*)g.q + (int64_t)(qrow0 + qr) * g.ldq + h * DH + 8 * hi;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) qf[qb][kk] = *(const bf16x8*)(src + kk * 16);
    pl[qb] = g.p[grow0 + qr];
    nl[qb] = g.n[grow0 + qr];
  }
  // diagonal tile (T rows' own keys): registers -> LDS in the ring's layout
  constexpr int DPT = (512 + NT - 1) / NT;
  bf16x8 dk[DPT], dv[DPT];
  if (has_diag) {
#pragma unroll
    for (int i = 0; i < DPT; ++i) {
      const int c = tid + NT * i, r = c >> 3, cc = c & 7;
      const int rr = (c < 512 && r < nrows) ? r : 0;
      dk[i] = *(const bf16x8*)((const bf16*)g.kd + (int64_t)(qrow0 + rr) * g.ldkd + grp * DH + cc * 8);
      dv[i] = *(const bf16x8*)((const bf16*)g.vd + (int64_t)(qrow0 + rr) * g.ldvd + grp * DH + cc * 8);
    }
  }
  int plim[QB], selfq[QB];
  float rq[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const bool ok = qb * 32 + l32 < nrows;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) qf[qb][kk] = ok ? qf[qb][kk] : bf16x8{};
    plim[qb] = ok ? pl[qb] : 0;
    selfq[qb] = ok ? nl[qb] - pl[qb] : 0;
    rq[qb] = ok ? g.out_scale / (float)nl[qb] : 0.f;
  }
  if (has_diag) {
#pragma unroll
    for (int i = 0; i < DPT; ++i) {
      const int c = tid + NT * i, r = c >> 3, cc = c & 7;
      if (c >= 512) continue;
      if (r >= nrows) { dk[i] = bf16x8{}; dv[i] = bf16x8{}; }
      *(bf16x8*)(dlds + r * 128 + ((cc ^ a_swz(r)) << 4)) = dk[i];
      const int ps = perm16(r);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int d = cc * 8 + e;
        *(bf16*)(dlds + A_TILE + d * 128 + (((ps >> 3) ^ a_swz(d)) << 4) + (ps & 7) * 2) = dv[i][e];
      }
    }
  }
  // the ring's first tiles, the query rows and the diagonal tile are in place
  a_wait_vm_lgkm<0>();
  a_barrier();

  f32x16 o[2][QB];   // O^T: lane = query, registers = dims mb*32 + 8(i/4) + 4hi + i%4
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < QB; ++b) o[a][b] = f32x16{};

  const int xk = hi ^ a_swz(l32);   // fragment slot = (even chunk) ^ xk for K and V^T rows
  auto qk = [&](const char* st, int kb, f32x16* sc) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) sc[qb] = f32x16{};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const bf16x8 af = *(const bf16x8*)(st + (kb * 32 + l32) * 128 + (((2 * kk) ^ xk) << 4));
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) sc[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, qf[qb][kk], sc[qb], 0, 0, 0);
    }
  };
  // P chunk c of key block kb: keys kb*32 + 16c + {4hi + t, 8 + 4hi + t : t < 4}, the
  // order in which V^T holds them, so P^T is the B operand of O^T += V^T P^T as is.
  // Masks (template MK): 0 none; 1 keys below lim visible; 2 keys in [lo, lim);
  // 3 only key dsel (the diagonal tile).  The invisible scores are set to 0
  // before SiLU (SiLU(0) = 0 exactly), so each mask costs one compare and one
  // select per element and P still converts to bf16 in pairs.  Register i of
  // this lane holds key kb*32 + kc(i) + 4*hi with the compile-time
  // kc(i) = 8*(i/4) + i%4: the bounds are shifted by the lane part once.
  auto silu_pv = [&](const char* st, int kb, const f32x16* sc, auto mask_tag, int lo, const int* lim,
                     const int* dsel) {
    constexpr int MK = decltype(mask_tag)::value;
    bf16x8 pf[QB][2];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int shift = kb * 32 + 4 * hi;
      const int lo_l = lo - shift;
      const int lim_l = (MK == 1 || MK == 2) ? lim[qb] - shift : 0;
      const int d_l = MK == 3 ? dsel[qb] - shift : 0;
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int i = 8 * c + e;
          const int kc = 8 * (i >> 2) + (i & 3);
          float sv = sc[qb][i];
          if constexpr (MK == 1) sv = kc < lim_l ? sv : 0.f;
          if constexpr (MK == 2) sv = (kc >= lo_l && kc < lim_l) ? sv : 0.f;
          if constexpr (MK == 3) sv = kc == d_l ? sv : 0.f;
          pf[qb][c][e] = (bf16)silu_scaled(sv);
        }
    }
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const bf16x8 vf = *(const bf16x8*)(st + A_TILE + (mb * 32 + l32) * 128 + (((4 * kb + 2 * c) ^ xk) << 4));
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          o[mb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[qb][c], o[mb][qb], 0, 0, 0);
      }
  };
  // QB = 1 issues both key blocks' QK MFMAs before the first block's SiLU (more
  // independent MFMA work per wave); QB = 2 has enough of it per block already
  // and keeps fewer accumulators live.
  auto tile_body = [&](const char* st, auto mask_tag, int lo, const int* lim, const int* dsel) {
    if constexpr (QB == 1) {
      f32x16 sc[2][QB];
      qk(st, 0, sc[0]);
      qk(st, 1, sc[1]);
      silu_pv(st, 0, sc[0], mask_tag, lo, lim, dsel);
      silu_pv(st, 1, sc[1], mask_tag, lo, lim, dsel);
    } else {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        f32x16 sc[QB];
        qk(st, kb, sc);
        silu_pv(st, kb, sc, mask_tag, lo, lim, dsel);
      }
    }
  };
  using MaskNone = std::integral_constant<int, 0>;
  using MaskUpper = std::integral_constant<int, 1>;
  using MaskRange = std::integral_constant<int, 2>;
  using MaskSelf = std::integral_constant<int, 3>;

  int stage = 0;
  for (int it = 0; it < n_main; ++it) {
    const char* st = lds + stage * A_STAGE;
    const int ts = T0 + it * 64;
    if (ts >= urow0 && ts + 64 <= kfull) {
      tile_body(st, MaskNone{}, 0, nullptr, nullptr);
    } else {
      int lim[QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) lim[qb] = urow0 + plim[qb] - ts;
      if (ts >= urow0) tile_body(st, MaskUpper{}, 0, lim, nullptr);   // only the prefix end cuts this tile
      else tile_body(st, MaskRange{}, urow0 - ts, lim, nullptr);      // the user's first tile
    }
    if (it + 1 < n_main) {
      // tile it + 1 has landed once at most AS - 2 newer tiles' DMA are in flight;
      // after the barrier every wave is done with this stage and it is refilled
      a_wait_vm_lgkm<(AS - 2) * DMA_PER_TILE>();
      a_barrier();
      issue(it + AS, stage);
      stage = stage + 1 == AS ? 0 : stage + 1;
    }
  }
  if (has_diag) {
    int dsel[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) dsel[qb] = selfq[qb] ? qb * 32 + l32 : -1;
    tile_body(dlds, MaskSelf{}, 0, nullptr, dsel);
  }

  // output: lane = query, four consecutive dims per register group
  bf16* out = (bf16*)g.a;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int qi = qb * 32 + l32;
    if (qi >= nrows) continue;
    bf16* orow = out + (int64_t)(qrow0 + qi) * g.lda + h * DH + 4 * hi;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf16x4 v;
#pragma unroll
        for (int t = 0; t < 4; ++t) v[t] = (bf16)(o[mb][qb][4 * j + t] * rq[qb]);
        *(bf16x4*)(orow + mb * 32 + 8 * j) = v;
      }
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
  const unsigned blocks = (unsigned)(a.ntiles * a.G * (2 / QB));
  switch (r) {
    case 1: attn_bf16_kernel<1, QB><<<blocks, 64, 0, s>>>(a); break;
    case 2: attn_bf16_kernel<2, QB><<<blocks, 128, 0, s>>>(a); break;
    case 4: attn_bf16_kernel<4, QB><<<blocks, 256, 0, s>>>(a); break;
    case 8: attn_bf16_kernel<8, QB><<<blocks, 512, 0, s>>>(a); break;
    default: return MTFM_E_UNSUPPORTED;
  }
  return MTFM_OK;
}

}  // namespace

mtfm_status launch_attention(const AttnArgs& a, int dtype, hipStream_t s) {
  if (a.ntiles <= 0) return MTFM_OK;
  const int r = a.H / a.G;
  if (dtype == MTFM_BF16) {
    if (a.dh != 64 || !a.vt || a.ldvt % 64 != 0 || a.ldvt < a.n_key_rows) return MTFM_E_UNSUPPORTED;
    if (((uintptr_t)a.k | (uintptr_t)a.vt | (uintptr_t)a.kd | (uintptr_t)a.vd) & 15) return MTFM_E_UNSUPPORTED;
    if (a.ldk % 8 != 0 || a.ldkd % 8 != 0 || a.ldvd % 8 != 0 || a.ldq % 8 != 0 || a.lda % 4 != 0 || ((uintptr_t)a.a & 7))
      return MTFM_E_UNSUPPORTED;
    // 32-bit buffer offsets: the whole V^T and one 64-row K tile
    if ((int64_t)a.G * 64 * a.ldvt * 2 >= (int64_t)1 << 32 || 64 * a.ldk * 2 >= (int64_t)1 << 31) return MTFM_E_UNSUPPORTED;
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
