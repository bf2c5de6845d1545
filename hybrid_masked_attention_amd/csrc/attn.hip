// Masked pointwise-SiLU attention kernels for gfx950.
//
// bf16 kernel: one workgroup per 32 query rows of a query tile and all H
// heads, one wave per head of the KV groups in flight.  The K and V tiles
// (64 keys x 64 dims) of a group are shared by its r heads in LDS
// ([explainer] §4.1 GQA: r query heads share a KV head).  They arrive through
// a ring of LDS stages filled by buffer loads straight into LDS: K from its
// row-major rows, V from a transposed copy (V^T, written by the projection
// GEMM) whose keys are permuted within groups of 16.  Per 32-key block each
// wave computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (fp32 accumulate;
// lane = query, registers = keys), applies SiLU pointwise, rounds P to bf16
// and accumulates O^T += V^T P^T on MFMA: the S^T registers are already the B
// operand in the permuted key order, so P never leaves registers and every
// fragment is one 16-byte LDS read.
//
// Key tiles are aligned to 64 packed rows (aligned DMA); a tile is visited
// only when it holds a key visible to some query of the slice ([blog] §6.2:
// compute only key blocks holding a valid key), and the mask compare runs only
// on tiles not entirely inside every query's visible prefix (separate
// straight-line bodies).  T columns are never tiled ([blog] §6.2: the
// user-to-item direction is skipped): a T row's self term is one dot product
// and one value update in registers.
//
// With every head of its rows in one workgroup, the kernel finishes the layer's
// attention branch itself: A = O ln2 / n, then the gated group LayerNorm
// Y = GLN2(A) (.) U over the row ([blog] §6.1, GLN fused with the gating), so
// neither A nor Y makes a round trip through HBM before the output projection.
//
// Every visible pair costs one exp and one reciprocal on the VALU; MFMA and
// VALU work overlap across the waves resident on a SIMD (four per SIMD here),
// not within one wave.
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

// Workgroup shape.  One workgroup takes 32 query rows and every head of them,
// one wave per head of GPP KV groups at a time; the heads of further groups
// are further passes over the key tiles (P = G / GPP passes, each wave then
// holding P heads).  A ring stage holds GPP x (K + V^T) of 64 keys; two
// stages: 64 KB at GPP = 2 (two workgroups per CU, four waves per SIMD at
// r = 4), 128 KB at GPP = 4 (one workgroup of 16 waves per CU).
template <int R, int GPP> struct FusedShape {
  static constexpr int W = R * GPP;                  // waves per workgroup
  static constexpr int STAGE = GPP * A_STAGE;
  static constexpr int AS = 2;                       // ring stages
  static constexpr int CPW = 16 * GPP / W;           // 1 KB DMA chunks per wave per stage
  static constexpr int WG_LDS = (160 * 1024) / (AS * STAGE) > 8 ? 8 : (160 * 1024) / (AS * STAGE);
  // waves per SIMD the register budget is sized for: what LDS allows, at most
  // 4 with one or two passes (128 registers: at two passes the accumulators of
  // both heads stay live, and a few registers spill across the second pass
  // only), 2 beyond
  template <int P>
  static constexpr int occupancy() {
    constexpr int lds = W * WG_LDS / 4 < 1 ? 1 : W * WG_LDS / 4;
    constexpr int regs = P >= 4 ? 2 : 4;
    return lds < regs ? lds : regs;
  }
};

template <int R, int GPP, int P>
__global__ __launch_bounds__(64 * R * GPP, (FusedShape<R, GPP>::template occupancy<P>())) void attn_bf16_kernel(AttnArgs g) {
  using SH = FusedShape<R, GPP>;
  constexpr int W = SH::W, AS = SH::AS, STAGE = SH::STAGE, CPW = SH::CPW;
  __shared__ __attribute__((aligned(1024))) char lds[AS * STAGE];

  // logical block: (query tile, 32-row half[, KV group]); with per_group the
  // workgroup takes one group's heads (the grid has G times the blocks).  With
  // a work order, workgroup b runs on XCD b % 8 and takes the (b / 8)-th item
  // of that XCD's list (the G groups of a slice one after another).
  // (with key splits, the ksplit runs of a (slice, group) are further
  // consecutive logical blocks, the group varying fastest; splits come with
  // per_group, whose instances make one pass)
  const int ng = g.per_group ? g.G : 1;
  const int nks = P == 1 && g.ksplit > 1 ? g.ksplit : 1;
  const int ngrp = ng * nks;
  int gsel, sid;
  if (g.order) {
    const int x = blockIdx.x & 7, k = blockIdx.x >> 3;
    sid = g.order[8 * (k / ngrp) + x];
    if (sid < 0) return;                       // past the end of this XCD's list (whole workgroup)
    gsel = k % ngrp;
  } else {
    const int lb = xcd_remap(blockIdx.x, g.ntiles * 2 * ngrp);
    gsel = lb % ngrp;
    sid = lb / ngrp;
  }
  const int ks = gsel / ng;
  gsel %= ng;
  const int slice = sid & 1, tile = sid >> 1;
  MTFM_DCHECK_UNIFORM(tile < g.ntiles, "attention work-order entry");
  const int32_t* td = g.tiles + 8 * tile;
  const int u = td[TD_USER], row0 = td[TD_ROW0], tile_rows = td[TD_NROWS];
  const int qoff = slice * 32;
  const int nrows = min(32, tile_rows - qoff);
  if (nrows <= 0) return;                      // empty half of a short tile (whole workgroup)
  const int grow0 = td[TD_GROW0] + qoff, qrow0 = td[TD_QROW0] + qoff, urow0 = td[TD_UROW0];
  const int lctx = g.lens[3 * u] + g.lens[3 * u + 1];
  const bool any_self = row0 + qoff + nrows > lctx;   // some row of the slice is a T row (sees itself)
  MTFM_DCHECK_UNIFORM(tile_rows <= 64 && row0 % 64 == 0 && u >= 0 && urow0 >= 0, "attention tile descriptor");
  MTFM_DCHECK_UNIFORM(urow0 + lctx <= g.n_key_rows, "attention keys within the key rows");
  MTFM_DCHECK_UNIFORM(td[TD_FULL_END] <= td[TD_END] && 64 * (td[TD_END] - 1) < max(lctx, 1),
                      "attention key-tile bounds within the user's context");

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int gl = wave / R;                     // group within the pass
  const int l32 = lane & 31, hi = lane >> 5;
  const int hd = g.H * DH;

  // per query row: its query-space row qi and packed row gi (through the
  // permutation if there is one), visible context prefix, self flag, output scale
  const bool ok = l32 < nrows;
  const int qr = ok ? l32 : 0;
  const int qi = g.qperm ? g.qperm[qrow0 + qr] : qrow0 + qr;
  const int gi = g.gperm ? g.gperm[qrow0 + qr] : grow0 + qr;
  const int plim = ok ? g.p[gi] : 0;
  const int nl = ok ? g.n[gi] : 1;
  const int selfq = ok ? nl - plim : 0;
  const float rq = ok ? g.out_scale / (float)nl : 0.f;
  // smallest and largest visible prefix over the slice's rows (the same rows in
  // every wave, so workgroup-uniform)
  const int pmax_s = __builtin_amdgcn_readfirstlane(wave_max(plim));
  const int pmin_s = __builtin_amdgcn_readfirstlane(wave_min(ok ? plim : 0x7fffffff));

  // Key tiles are aligned to 64 packed rows: tile it covers rows ts = T0 + 64 it
  // .. ts + 63.  A row sees the user's keys [urow0, urow0 + p).  K rows below
  // urow0 (an earlier user's) and at or past kz_end (no row of the slice sees
  // them) reach LDS as zeros: their scores are 0 and SiLU(0) = 0, so they add
  // exactly nothing.  Keys below kfull are seen by every row of the slice, so a
  // tile needs per-row masks only where some row's prefix ends strictly inside
  // the keys it loads (never in a slice whose rows share one prefix).
  const int T0 = urow0 & ~63;
  const int kz_end = urow0 + pmax_s;
  const int kfull = urow0 + pmin_s;
  const int n_main = pmax_s > 0 ? (kz_end - T0 + 63) >> 6 : 0;
  // this workgroup's run of key tiles [it0, it1) (all of them without splits)
  const int it0 = (int)((int64_t)n_main * ks / nks), it1 = (int)((int64_t)n_main * (ks + 1) / nks);

  // DMA: the stage's 16 GPP chunks of 1 KB (per group: 8 of K rows, 8 of V^T
  // rows, 8 rows of 128 B each); wave w issues chunks w + W i.  Lane -> row
  // 8 rb + lane / 8, 16-byte slot lane % 8 (read from the swizzled chunk).
  const int rin = lane >> 3, slot = lane & 7;
  uint32_t doff[CPW];
  int dlds[CPW];
#pragma unroll
  for (int i = 0; i < CPW; ++i) {
    const int c = wave + W * i;
    const int cg = c >> 4, kind = (c >> 3) & 1, rb = c & 7;
    const int r = rb * 8 + rin;
    const int sw = slot ^ a_swz(r);
    doff[i] = kind == 0 ? (uint32_t)(r * g.ldk * 2 + cg * DH * 2 + sw * 16)
                        : (uint32_t)((cg * DH + r) * g.ldvt * 2 + sw * 16);
    dlds[i] = cg * A_STAGE + kind * A_TILE + rb * 1024;
  }
  const bf16* kbase = (const bf16*)g.k;
  const bf16* vtbase = (const bf16*)g.vt;
  const int64_t vt_elems = (int64_t)g.G * DH * g.ldvt;
  // Tiles past the last one are issued as empty loads (zero-size resources), so
  // that the number of DMA instructions in flight is a constant at every wait.
  auto issue = [&](int gbase, int it, int stage) {
    const bool real = it < it1;
    const int ts = real ? T0 + it * 64 : T0;
    // K through one resource over the user's visible keys [urow0, kz_end): a row
    // of the tile outside it has an offset (negative ones wrap) past the
    // resource and reads as zero
    const __amdgpu_buffer_rsrc_t kr =
        a_rsrc(kbase + (int64_t)urow0 * g.ldk + gbase * DH, real ? (uint32_t)(pmax_s * g.ldk * 2) : 0u);
    const uint32_t kshift = (uint32_t)((ts - urow0) * g.ldk * 2);
    const int64_t vt0 = (int64_t)gbase * DH * g.ldvt + ts;
    const __amdgpu_buffer_rsrc_t vr = a_rsrc(vtbase + vt0, real ? (uint32_t)((vt_elems - vt0) * 2) : 0u);
    char* st = lds + stage * STAGE;
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      const int c = wave + W * i;
      const bool is_v = (c >> 3) & 1;
      lds_dma16(is_v ? vr : kr, (lds_void*)(st + dlds[i]), doff[i] + (is_v ? 0u : kshift));
    }
  };


  f32x16 o[P][2];   // O^T per pass: lane = query, registers = dims mb*32 + 8(i/4) + 4hi + i%4
#pragma unroll
  for (int pp = 0; pp < P; ++pp) { o[pp][0] = f32x16{}; o[pp][1] = f32x16{}; }

  const int xk = hi ^ a_swz(l32);   // fragment slot = (even chunk) ^ xk for K and V^T rows
  using MaskNone = std::integral_constant<int, 0>;
  using MaskUpper = std::integral_constant<int, 1>;

#pragma unroll
  for (int pp = 0; pp < P; ++pp) {
    const int gbase = (gsel + pp) * GPP;
    const int grp = gbase + gl;
    const int h = grp * R + wave % R;
    if (pp > 0) {
      a_wait_vm_lgkm<0>();
      a_barrier();                             // every wave is done with the previous pass's ring
    }
#pragma unroll
    for (int s = 0; s < AS; ++s) issue(gbase, it0 + s, s);
    // Q fragments (B operand of S^T = K Q^T): query l32, dims kk*16 + 8*hi + [0, 8)
    bf16x8 qf[4];
    {
      const bf16* src = (const bf16*)g.q + (int64_t)qi * g.ldq + h * DH + 8 * hi;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) qf[kk] = ok ? *(const bf16x8*)(src + kk * 16) : bf16x8{};
    }
    const char* gl_lds = lds + gl * A_STAGE;   // this wave's group inside a stage
    a_wait_vm_lgkm<0>();
    a_barrier();                               // the ring's first tiles are in place

    auto qk = [&](const char* st, int kb, f32x16& sc) {
      sc = f32x16{};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const bf16x8 af = *(const bf16x8*)(st + (kb * 32 + l32) * 128 + (((2 * kk) ^ xk) << 4));
        sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, qf[kk], sc, 0, 0, 0);
      }
    };
    // P chunk c of key block kb: keys kb*32 + 16c + {4hi + t, 8 + 4hi + t : t < 4}, the
    // order in which V^T holds them, so P^T is the B operand of O^T += V^T P^T as is.
    // Masks (template MK): 0 none; 1 keys below lim visible.
    // The invisible scores are set to 0 before SiLU (SiLU(0) = 0 exactly), so a
    // mask costs one compare and one select per element and P still converts to
    // bf16 in pairs.  Register i of this lane holds key kb*32 + kc(i) + 4*hi with
    // the compile-time kc(i) = 8*(i/4) + i%4: the bounds are shifted once.
    auto silu_pv = [&](const char* st, int kb, const f32x16& sc, auto mask_tag, int lim) {
      constexpr int MK = decltype(mask_tag)::value;
      bf16x8 pf[2];
      const int shift = kb * 32 + 4 * hi;
      const int lim_l = lim - shift;
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int i = 8 * c + e;
          const int kc = 8 * (i >> 2) + (i & 3);
          float sv = sc[i];
          if constexpr (MK == 1) sv = kc < lim_l ? sv : 0.f;
          pf[c][e] = (bf16)silu_scaled(sv);
        }
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          const bf16x8 vf = *(const bf16x8*)(st + A_TILE + (mb * 32 + l32) * 128 + (((4 * kb + 2 * c) ^ xk) << 4));
          o[pp][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[c], o[pp][mb], 0, 0, 0);
        }
    };
    // one 32-key block at a time (a wave gets no MFMA / VALU overlap within
    // itself, only with the other waves of its SIMD, so holding one block's
    // scores keeps four waves per SIMD within their registers).  On a cut tile
    // the keys below lim of a row are visible (those below lo, an earlier
    // user's, are zeros); lim_hi is the largest lim over the slice: a block
    // entirely below lo or from lim_hi on is skipped (its products would all be
    // zero).
    auto tile_body = [&](const char* st, auto mask_tag, int lo, int lim, int lim_hi) {
      constexpr int MK = decltype(mask_tag)::value;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        f32x16 sc;
        if constexpr (MK == 0) {
          qk(st, kb, sc);
          silu_pv(st, kb, sc, mask_tag, lim);
        } else {
          const int b0 = 32 * kb, b1 = b0 + 32;
          if (lo >= b1 || lim_hi <= b0) continue;             // no row sees a key of the block
          qk(st, kb, sc);
          silu_pv(st, kb, sc, mask_tag, lim);
        }
      }
    };

    int stage = 0;
    auto next_tile = [&](int it) {
      if (it + 1 < it1) {
        // tile it + 1 has landed once at most AS - 2 newer tiles' DMA are in flight;
        // after the barrier every wave is done with this stage and it is refilled
        a_wait_vm_lgkm<(AS - 2) * CPW>();
        a_barrier();
        issue(gbase, it + AS, stage);
        stage = stage + 1 == AS ? 0 : stage + 1;
      }
    };
    // The leading tiles, whose nonzero keys every row sees (all of them when the
    // slice's rows share one prefix), run without masks in a loop of their own
    // (straight-line, so the compiler overlaps one block's SiLU with the next
    // block's products); the few tiles in which some row's prefix ends follow.
    const int n_unmasked = kfull >= kz_end ? n_main : min(n_main, max(kfull - T0, 0) >> 6);
    int it = it0;
    for (; it < min(n_unmasked, it1); ++it) {
      tile_body(gl_lds + stage * STAGE, MaskNone{}, 0, 0, 0);
      next_tile(it);
    }
    for (; it < it1; ++it) {
      const int ts = T0 + it * 64;
      tile_body(gl_lds + stage * STAGE, MaskUpper{}, max(urow0 - ts, 0), urow0 + plim - ts, kz_end - ts);
      next_tile(it);
    }

    // A T row's only T key is itself ([explainer] §8.2 matrix; the user-to-item
    // direction is never tiled): its score and value term in registers.  The
    // lane holds half of the query's dims (kk*16 + 8hi + [0, 8)); the other half
    // is in lane ^ 32.
    if (any_self && ks == 0) {
      // (the row index passes through an empty asm so that the row addresses
      // are formed here in each pass rather than kept live across the passes)
      int qs = qi;
      asm volatile("" : "+v"(qs));
      const bf16* krow = (const bf16*)g.kd + (int64_t)qs * g.ldkd + grp * DH + 8 * hi;
      float part = 0.f;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const bf16x8 kv = *(const bf16x8*)(krow + kk * 16);
#pragma unroll
        for (int e = 0; e < 8; ++e) part = fmaf((float)qf[kk][e], (float)kv[e], part);
      }
      part += __shfl_xor(part, 32, 64);
      const float ps = selfq ? (float)(bf16)silu_scaled(part) : 0.f;
      // only a T row's own value is read (and may be stored): other rows' slots
      // of the row-major V need not hold finite values
      const bf16* vrow = (const bf16*)g.vd + (int64_t)qs * g.ldvd + grp * DH + 4 * hi;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const bf16x4 vv = selfq ? *(const bf16x4*)(vrow + mb * 32 + 8 * j) : bf16x4{};
#pragma unroll
          for (int t = 0; t < 4; ++t) o[pp][mb][4 * j + t] = fmaf(ps, (float)vv[t], o[pp][mb][4 * j + t]);
        }
    }
  }

  // A = O ln2 / n_i; wave w holds heads w + W pp
#pragma unroll
  for (int pp = 0; pp < P; ++pp)
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[pp][mb][i] *= rq;
  if (nks > 1) {
    // key splits: this run's fp32 partial (per_group: one pass, one head per wave)
    if (ok) {
      float* prow = g.a_part + ks * g.part_stride + (int64_t)qi * g.lda + (gsel * W + wave) * DH + 4 * hi;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          f32x4 v;
#pragma unroll
          for (int t = 0; t < 4; ++t) v[t] = o[0][mb][4 * j + t];
          *(f32x4*)(prow + mb * 32 + 8 * j) = v;
        }
    }
    return;
  }
  if (g.a && ok) {
#pragma unroll
    for (int pp = 0; pp < P; ++pp) {
      bf16* orow = (bf16*)g.a + (int64_t)qi * g.lda + ((gsel + pp) * W + wave) * DH + 4 * hi;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          bf16x4 v;
#pragma unroll
          for (int t = 0; t < 4; ++t) v[t] = (bf16)o[pp][mb][4 * j + t];
          *(bf16x4*)(orow + mb * 32 + 8 * j) = v;
        }
    }
  }
  if (!g.y) return;

  // Fused epilogue ([blog] §6.1, the gated group LayerNorm after attention):
  //   Y = (LayerNorm(A) * gamma[type] + beta[type]) (.) U
  // over the row's H*dh values, fp32 two-pass statistics: per lane over its
  // 32 P values, with lane ^ 32 (the other half of each head), then across the
  // W waves through LDS (the ring is free once every wave is past its loop).
  float* red = (float*)lds;
  float s1 = 0.f;
#pragma unroll
  for (int pp = 0; pp < P; ++pp)
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int i = 0; i < 16; ++i) s1 += o[pp][mb][i];
  s1 += __shfl_xor(s1, 32, 64);
  a_wait_vm_lgkm<0>();
  a_barrier();
  if (hi == 0) red[wave * 32 + l32] = s1;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int w = 0; w < W; ++w) tot += red[w * 32 + l32];
  const float mean = tot / (float)hd;
  float s2 = 0.f;
#pragma unroll
  for (int pp = 0; pp < P; ++pp)
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float dv = o[pp][mb][i] - mean;
        o[pp][mb][i] = dv;
        s2 += dv * dv;
      }
  s2 += __shfl_xor(s2, 32, 64);
  if (hi == 0) red[(W + wave) * 32 + l32] = s2;
  __syncthreads();
  float var = 0.f;
#pragma unroll
  for (int w = 0; w < W; ++w) var += red[(W + w) * 32 + l32];
  const float rstd = rsqrtf(var / (float)hd + g.eps);
  if (!ok) return;
  const int t = g.type[gi];
  const float* gam = g.ln_g + (int64_t)t * hd;
  const float* bet = g.ln_b + (int64_t)t * hd;
  const bool gb_vec = (((uintptr_t)g.ln_g | (uintptr_t)g.ln_b) & 15) == 0;   // 16-byte loads where aligned
  const bf16* urow = (const bf16*)g.u + (int64_t)qi * g.ldu;
  bf16* yrow = (bf16*)g.y + (int64_t)qi * g.ldy;
#pragma unroll
  for (int pp = 0; pp < P; ++pp)
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d0 = (pp * W + wave) * DH + mb * 32 + 8 * j + 4 * hi;
        float gm[4], bt[4];
        if (gb_vec) {
          const f32x4 g4 = *(const f32x4*)(gam + d0), b4 = *(const f32x4*)(bet + d0);
#pragma unroll
          for (int q = 0; q < 4; ++q) { gm[q] = g4[q]; bt[q] = b4[q]; }
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) { gm[q] = gam[d0 + q]; bt[q] = bet[d0 + q]; }
        }
        const bf16x4 uu = *(const bf16x4*)(urow + d0);
        bf16x4 v;
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = (bf16)((o[pp][mb][4 * j + q] * rstd * gm[q] + bt[q]) * (float)uu[q]);
        *(bf16x4*)(yrow + d0) = v;
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

template <int R, int GPP, int P>
void launch_fused(const AttnArgs& a, hipStream_t s) {
  const unsigned blocks = (unsigned)((a.order ? (int64_t)a.n_order : 2 * (int64_t)a.ntiles) * (a.per_group ? a.G : 1) *
                                     (a.ksplit > 1 ? a.ksplit : 1));
  attn_bf16_kernel<R, GPP, P><<<blocks, 64 * R * GPP, 0, s>>>(a);
}

// Groups per ring stage GPP = min(G, 4, 16 / r) (at most 16 waves and a 64 KB
// stage) and passes G / GPP, for H = r G query heads (H <= 16).
mtfm_status launch_bf16(const AttnArgs& a, int r, hipStream_t s) {
  const int G = a.G;
  if (a.per_group) {   // one group per workgroup: r waves, a single pass
    switch (r) {
      case 1: launch_fused<1, 1, 1>(a, s); break;
      case 2: launch_fused<2, 1, 1>(a, s); break;
      case 4: launch_fused<4, 1, 1>(a, s); break;
      case 8: launch_fused<8, 1, 1>(a, s); break;
      default: return MTFM_E_UNSUPPORTED;
    }
    return MTFM_OK;
  }
  switch (r) {
    case 1:
      if (G == 1) launch_fused<1, 1, 1>(a, s);
      else if (G == 2) launch_fused<1, 2, 1>(a, s);
      else if (G == 4) launch_fused<1, 4, 1>(a, s);
      else if (G == 8) launch_fused<1, 4, 2>(a, s);
      else if (G == 16) launch_fused<1, 4, 4>(a, s);
      else return MTFM_E_UNSUPPORTED;
      break;
    case 2:
      if (G == 1) launch_fused<2, 1, 1>(a, s);
      else if (G == 2) launch_fused<2, 2, 1>(a, s);
      else if (G == 4) launch_fused<2, 4, 1>(a, s);
      else if (G == 8) launch_fused<2, 4, 2>(a, s);
      else return MTFM_E_UNSUPPORTED;
      break;
    case 4:
      if (G == 1) launch_fused<4, 1, 1>(a, s);
      else if (G == 2) launch_fused<4, 1, 2>(a, s);
      else if (G == 4) launch_fused<4, 1, 4>(a, s);
      else return MTFM_E_UNSUPPORTED;
      break;
    case 8:
      if (G == 1) launch_fused<8, 1, 1>(a, s);
      else if (G == 2) launch_fused<8, 2, 1>(a, s);
      else return MTFM_E_UNSUPPORTED;
      break;
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
    // 32-bit buffer offsets: the whole V^T and one user's K rows (with a tile's
    // reach below the user's first row)
    if ((int64_t)a.G * 64 * a.ldvt * 2 >= (int64_t)1 << 32 ||
        ((int64_t)max(a.max_user_rows, 0) + 64) * a.ldk * 2 >= (int64_t)1 << 31)
      return MTFM_E_UNSUPPORTED;
    if (a.max_user_rows <= 0) return MTFM_E_UNSUPPORTED;
    if (a.per_group && a.y) return MTFM_E_UNSUPPORTED;   // the gated epilogue needs every head of a row
    if (a.ksplit > 1 && (!a.per_group || !a.a_part || ((uintptr_t)a.a_part & 15) || a.part_stride % 4 != 0 ||
                         a.ksplit > 64))
      return MTFM_E_UNSUPPORTED;
    if (a.order && (a.n_order <= 0 || a.n_order % 8 != 0)) return MTFM_E_UNSUPPORTED;
    if (!a.qperm != !a.gperm) return MTFM_E_UNSUPPORTED;
    if (a.y && (!a.u || !a.ln_g || !a.ln_b || !a.type || a.ldy % 4 != 0 || a.ldu % 4 != 0 ||
                ((uintptr_t)a.y & 7) || ((uintptr_t)a.u & 7)))
      return MTFM_E_UNSUPPORTED;
    mtfm_status st = launch_bf16(a, r, s);
    if (st != MTFM_OK) return st;
  } else {
    if (a.qperm) return MTFM_E_UNSUPPORTED;
    dim3 grid((unsigned)a.ntiles, (unsigned)a.H);
    if (a.dh == 32) attn_f32_kernel<32><<<grid, 64, 0, s>>>(a);
    else if (a.dh == 64) attn_f32_kernel<64><<<grid, 64, 0, s>>>(a);
    else return MTFM_E_UNSUPPORTED;
  }
  MTFM_LAUNCH_CHECK("attention");
  return MTFM_OK;
}
