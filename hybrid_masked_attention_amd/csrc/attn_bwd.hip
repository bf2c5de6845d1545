// Backward of the masked pointwise-SiLU attention (bf16 MFMA, fp32 accumulate).
//
// With s' = Q' K^T (Q' = Q log2(e)/sqrt(dh), so x = s' ln2 is the scaled
// score), P = SiLU(x) on visible pairs, A = P V / n and dAn = dA / n:
//   dP  = dAn V^T,   dS = dP (.) SiLU'(x) on visible pairs,
//   dQ  = dS K / sqrt(dh),   dK = dS^T Q / sqrt(dh) = ln2 dS^T Q',   dV = P^T dAn,
// with dK, dV of a KV group summed over its r query heads ([explainer] §4.1
// GQA).  Three kernels, none with atomics:
//   * dq:  one workgroup per (32-row query slice, group), one wave per head;
//          the visible context key tiles stream through an LDS ring of K and
//          V tiles filled by buffer DMA; S^T and dP^T accumulate with lane =
//          query so dS feeds dQ from registers, K^T through the transposing
//          LDS read.
//   * dkv: one workgroup per (64-key context tile, group), two waves per
//          head (one per 32-key half); walks the user's query tiles that see
//          the keys in 32-query stages brought in by buffer DMA, S and dP with
//          lane = key so P and dS feed the dV / dK MFMAs from registers, Q' and
//          dA/n through the transposing LDS read; the r heads' dK, dV are
//          summed through LDS in a fixed order.
//   * self: one wave per (T row, group): the T row's only T key is itself
//          ([blog] §3.2), so its term is a few dot products.

#include "bwd_kernels.h"

namespace {

constexpr int DH = 64;
constexpr float kLn2 = 0.69314718055994530942f;

MTFM_DEV int64_t map_b(const RowMapB& r, int m) {
  if (r.list) return (int64_t)r.list[m / r.div] + m % r.div;
  return m;
}

MTFM_DEV float dsilu_f(float h) {
  const float s = 1.0f / (1.0f + __expf(-h));
  return s * (1.0f + h * (1.0f - s));
}

// s' -> (SiLU(x), SiLU'(x)) with x = s' ln2
MTFM_DEV void silu_and_grad(float sp, float* p, float* dp) {
  const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-sp));
  const float x = sp * kLn2;
  *p = x * sg;
  *dp = sg * (1.0f + x * (1.0f - sg));
}

// The same pair with SiLU scaled by 1/ln2 (callers fold ln2 in later), in
// fewer operations: SiLU(x)/ln2 = s' sg and SiLU'(x) = sg + (s' sg) ln2 (1 - sg).
// A masked pair is given the score kMaskedScore: 2^512 overflows to +inf, the
// sigmoid is then exactly 0 and both results are 0.
constexpr float kMaskedScore = -512.0f;
MTFM_DEV void silu_grad_scaled(float sp, float* p_ln2, float* dp) {
  const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-sp));
  const float q = sp * sg;
  *p_ln2 = q;
  *dp = __builtin_fmaf(q, __builtin_fmaf(-kLn2, sg, kLn2), sg);
}

MTFM_DEV bf16x8 ld8(const bf16* p) { return *(const bf16x8*)p; }

// --------------------------------------------------------------------------
// LDS ring helpers shared by the dQ and dK/dV kernels.

// 16-byte unit u of stage row r sits at slot u ^ kv_swz(r): conflict-free for
// both the row reads (16 consecutive rows, one unit) and the transposing reads
// (4 consecutive rows, 4 units).
MTFM_DEV int kv_swz(int r) { return (((r >> 1) & 1) << 2) | ((r >> 2) & 3); }

typedef __attribute__((address_space(3))) void lds_void_t;
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

MTFM_DEV void kv_dma(__amdgpu_buffer_rsrc_t r, lds_void_t* dst, uint32_t voff, int bytes) {
#if defined(__HIP_DEVICE_COMPILE__)
  if (bytes == 16) __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, voff, 0, 0, 0);
  else __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 4, voff, 0, 0, 0);
#endif
}

MTFM_DEV __amdgpu_buffer_rsrc_t kv_rsrc(const void* base, uint32_t bytes) {
  const uint64_t b = (uint64_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  return __builtin_amdgcn_make_buffer_rsrc((void*)(((uint64_t)hi << 32) | lo), (short)0,
                                           (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

template <int N> MTFM_DEV void kv_wait_vm() { __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0070); }
MTFM_DEV void kv_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Transposing read ds_read_b64_tr_b16: lanes 4m + c of each 16-lane group
// point at row m, 4 columns; lane j receives column j of the 4 rows.  The 16
// reads of a stage (Q' and dA/n hi, 2 x 2 x 2 fragments) are issued together
// and waited for inside the same block, so their results are complete when it
// ends.  They are written as one block rather than as separate builtins because
// the compiler cannot tell that they do not touch the stages still being filled
// by DMA and would otherwise wait for the whole ring before each of them.
// a[nb][h2] = LDS address of fragment (c = 0, nb, h2) of Q'; +2048 for c = 1,
// +4096 for dA/n.
MTFM_DEV void kv_tr16(const uint32_t (&a)[2][2], i16x4 (&q)[2][2][2], i16x4 (&d)[2][2][2]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %16\n\t"
      "ds_read_b64_tr_b16 %1, %17\n\t"
      "ds_read_b64_tr_b16 %2, %18\n\t"
      "ds_read_b64_tr_b16 %3, %19\n\t"
      "ds_read_b64_tr_b16 %4, %16 offset:2048\n\t"
      "ds_read_b64_tr_b16 %5, %17 offset:2048\n\t"
      "ds_read_b64_tr_b16 %6, %18 offset:2048\n\t"
      "ds_read_b64_tr_b16 %7, %19 offset:2048\n\t"
      "ds_read_b64_tr_b16 %8, %16 offset:4096\n\t"
      "ds_read_b64_tr_b16 %9, %17 offset:4096\n\t"
      "ds_read_b64_tr_b16 %10, %18 offset:4096\n\t"
      "ds_read_b64_tr_b16 %11, %19 offset:4096\n\t"
      "ds_read_b64_tr_b16 %12, %16 offset:6144\n\t"
      "ds_read_b64_tr_b16 %13, %17 offset:6144\n\t"
      "ds_read_b64_tr_b16 %14, %18 offset:6144\n\t"
      "ds_read_b64_tr_b16 %15, %19 offset:6144\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(q[0][0][0]), "=&v"(q[0][0][1]), "=&v"(q[0][1][0]), "=&v"(q[0][1][1]),
        "=&v"(q[1][0][0]), "=&v"(q[1][0][1]), "=&v"(q[1][1][0]), "=&v"(q[1][1][1]),
        "=&v"(d[0][0][0]), "=&v"(d[0][0][1]), "=&v"(d[0][1][0]), "=&v"(d[0][1][1]),
        "=&v"(d[1][0][0]), "=&v"(d[1][0][1]), "=&v"(d[1][1][0]), "=&v"(d[1][1][1])
      : "v"(a[0][0]), "v"(a[0][1]), "v"(a[1][0]), "v"(a[1][1])
      : "memory");
}

// The 32 prefix limits of a stage's queries, in this lane's register order:
// p[4j + t] = limit of query 8j + 4hi + t (a = LDS address of query 4hi).
MTFM_DEV void kv_plim(uint32_t a, int4 (&p)[4]) {
  asm volatile(
      "ds_read_b128 %0, %4\n\t"
      "ds_read_b128 %1, %4 offset:32\n\t"
      "ds_read_b128 %2, %4 offset:64\n\t"
      "ds_read_b128 %3, %4 offset:96\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(p[0]), "=&v"(p[1]), "=&v"(p[2]), "=&v"(p[3])
      : "v"(a)
      : "memory");
}

MTFM_DEV uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)(p);
}

// --------------------------------------------------------------------------
// dQ kernel.  One workgroup per (32-row query slice, KV group), one wave per
// head of the group (32 queries, lane = query).  The user's visible context
// key tiles (64 keys, aligned to the user's first row) stream through a
// three-stage LDS ring of K and V tiles (8 KB each, rows swizzled as kv_swz),
// filled by buffer DMA two tiles ahead and shared by the r heads.  S^T = K Q'^T
// and dP^T = V (dA/n)^T accumulate with lane = query, so dS feeds dQ += dS K
// straight from registers; the K^T operand (8 consecutive keys of one head
// dimension per lane) comes from the row-major K tile through the
// transposing LDS read.
constexpr int DQ_NS = 3;
constexpr int DQ_TILE = 64 * 128;       // 64 key rows x 128 B
constexpr int DQ_STAGE = 2 * DQ_TILE;   // K, then V

// The 8 transposing reads of one 32-key block: fragment (c, nb, h2) at LDS
// address a[nb][h2] (+2048 B for c = 1, the next 16 keys); one block with its
// own wait, for the reason given at kv_tr16.
MTFM_DEV void dq_tr8(const uint32_t (&a)[2][2], i16x4 (&o)[2][2][2]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8\n\t"
      "ds_read_b64_tr_b16 %1, %9\n\t"
      "ds_read_b64_tr_b16 %2, %10\n\t"
      "ds_read_b64_tr_b16 %3, %11\n\t"
      "ds_read_b64_tr_b16 %4, %8 offset:2048\n\t"
      "ds_read_b64_tr_b16 %5, %9 offset:2048\n\t"
      "ds_read_b64_tr_b16 %6, %10 offset:2048\n\t"
      "ds_read_b64_tr_b16 %7, %11 offset:2048\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o[0][0][0]), "=&v"(o[0][0][1]), "=&v"(o[0][1][0]), "=&v"(o[0][1][1]),
        "=&v"(o[1][0][0]), "=&v"(o[1][0][1]), "=&v"(o[1][1][0]), "=&v"(o[1][1][1])
      : "v"(a[0][0]), "v"(a[0][1]), "v"(a[1][0]), "v"(a[1][1])
      : "memory");
}

template <int R>
__global__ __launch_bounds__(64 * R, R >= 4 ? 3 : 1) void attn_bwd_dq_kernel(AttnBwdArgs g) {
  constexpr int CPW = 16 / R;             // 1 KB DMA chunks per wave per stage
  static_assert(CPW * R == 16, "chunks per stage");
  __shared__ __attribute__((aligned(1024))) char lds[DQ_NS * DQ_STAGE];
  auto uni = [](int v) { return __builtin_amdgcn_readfirstlane(v); };
  typedef __attribute__((address_space(4))) const int32_t cint;

  const int nblocks = g.nqtiles * g.G * 2;
  const int lb = xcd_remap(blockIdx.x, nblocks);
  const int slice = lb & 1;
  const int tile = (lb >> 1) / g.G, grp = (lb >> 1) % g.G;
  const cint* td = (const cint*)g.qtiles + 8 * tile;
  const int u = uni(td[TD_USER]), tile_rows = uni(td[TD_NROWS]);
  const int full_end = uni(td[TD_FULL_END]), ntl = uni(td[TD_END]);
  const int qoff = slice * 32;
  const int nrows = min(32, tile_rows - qoff);
  if (nrows <= 0) return;
  const int grow0 = uni(td[TD_GROW0]) + qoff, qrow0 = uni(td[TD_QROW0]) + qoff, urow0 = uni(td[TD_UROW0]);
  const cint* lens = (const cint*)g.lens;
  const int lctx = uni(lens[3 * u] + lens[3 * u + 1]);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = grp * R + wave;
  const int l32 = lane & 31, hi = lane >> 5;
  const bool qok = l32 < nrows;

  // this wave's queries (B operands, lane = query, dims kk*16 + 8hi): loaded
  // before the first DMA so that waiting for them never waits for the ring
  bf16x8 qf[4], df[4], dl[4];
  {
    const int64_t qrow = qrow0 + (qok ? l32 : 0);
    const bf16* qs = g.q + qrow * g.ldq + h * DH + 8 * hi;
    const bf16* ds = g.dan + qrow * g.lddan + h * DH + 8 * hi;
    const bf16* dls = g.dan_lo + qrow * g.lddan + h * DH + 8 * hi;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      qf[kk] = ld8(qs + kk * 16);
      df[kk] = ld8(ds + kk * 16);
      dl[kk] = ld8(dls + kk * 16);
    }
  }
  const int plim_raw = g.p[grow0 + (qok ? l32 : 0)];

  // DMA: chunk c (16 per stage) = tensor c / 8 (K, V), rows 8 (c % 8) + lane / 8,
  // slot lane % 8 holding the 16-byte unit slot ^ kv_swz(row).  Tiles past the
  // last one are issued as empty loads so that every wait sees the same count.
  const int rin = lane >> 3, slot = lane & 7;
  auto issue = [&](int it, int buf) {
    const bool real = it < ntl;
    const int valid = real ? min(64, lctx - it * 64) : 0;
    const int64_t row0 = urow0 + (real ? it * 64 : 0);
    const __amdgpu_buffer_rsrc_t rk = kv_rsrc(g.k + row0 * g.ldk + grp * DH, (uint32_t)(valid * g.ldk * 2));
    const __amdgpu_buffer_rsrc_t rv = kv_rsrc(g.v + row0 * g.ldv + grp * DH, (uint32_t)(valid * g.ldv * 2));
    char* st = lds + buf * DQ_STAGE;
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      const int c = i * R + wave;
      const int t = c >> 3, r = (c & 7) * 8 + rin;
      const int64_t ld = t ? g.ldv : g.ldk;
      const uint32_t voff = (uint32_t)(r * ld * 2 + ((slot ^ kv_swz(r)) << 4));
      kv_dma(t ? rv : rk, (lds_void_t*)(st + t * DQ_TILE + (c & 7) * 1024), voff, 16);
    }
  };
#pragma unroll
  for (int s = 0; s < DQ_NS - 1; ++s) issue(s, s);

#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    qf[kk] = qok ? qf[kk] : bf16x8{};
    df[kk] = qok ? df[kk] : bf16x8{};
    dl[kk] = qok ? dl[kk] : bf16x8{};
  }
  const int plim = qok ? plim_raw : 0;
  // row reads: key kb*32 + l32, unit 2kk + hi; transposing reads of fragment
  // (c, nb, h2): keys kb*32 + 16c + 8h2 + 4hi + (lane/4)%4, dims nb*32 +
  // 16((lane/16)%2) + 4(lane%4) .. + 3 (kb and c only move the row by 32 / 16)
  const int sw32 = kv_swz(l32);
  uint32_t tro[2][2];
  {
    const int tm = (lane >> 2) & 3, tcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int r = 8 * h2 + 4 * hi + tm;
        const int col = nb * 32 + tcol;
        tro[nb][h2] = (uint32_t)(r * 128 + (((col >> 3) ^ kv_swz(r)) << 4) + (col & 7) * 2);
      }
  }
  const uint32_t lds0 = lds_addr(lds);

  f32x16 dq[2] = {f32x16{}, f32x16{}};
  for (int it = 0; it < ntl; ++it) {
    kv_wait_vm<(DQ_NS - 2) * CPW>();
    kv_barrier();
    issue(it + DQ_NS - 1, (it + DQ_NS - 1) % DQ_NS);
    const int buf = it % DQ_NS;
    const char* st = lds + buf * DQ_STAGE;
    const bool masked = it >= full_end || (it + 1) * 64 > lctx;
    const int lim = plim - it * 64;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      // S^T, dP^T: lane = query, registers = keys kb*32 + 8(i/4) + 4hi + i%4
      f32x16 sc = {}, dpt = {};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int off = (kb * 32 + l32) * 128 + (((2 * kk + hi) ^ sw32) << 4);
        const bf16x8 kf = *(const bf16x8*)(st + off);
        const bf16x8 vf = *(const bf16x8*)(st + DQ_TILE + off);
        sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[kk], sc, 0, 0, 0);
        dpt = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, df[kk], dpt, 0, 0, 0);
        dpt = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, dl[kk], dpt, 0, 0, 0);
      }
      if (masked) {
        const int lim_l = lim - kb * 32 - 4 * hi;
#pragma unroll
        for (int i = 0; i < 16; ++i) sc[i] = 8 * (i >> 2) + (i & 3) < lim_l ? sc[i] : kMaskedScore;
      }
      bf16x8 dsf[2];
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int i = 8 * c + e;
          float pv, dsg;
          silu_grad_scaled(sc[i], &pv, &dsg);
          dsf[c][e] = (bf16)(dpt[i] * dsg);
        }
      i16x4 kt4[2][2][2];
      {
        uint32_t ta[2][2];
        const uint32_t base = lds0 + (uint32_t)(buf * DQ_STAGE + kb * 4096);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) ta[nb][h2] = base + tro[nb][h2];
        dq_tr8(ta, kt4);
      }
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          const bf16x8 kt8 = __builtin_bit_cast(bf16x8, __builtin_shufflevector(kt4[c][nb][0], kt4[c][nb][1], 0, 1, 2, 3, 4, 5, 6, 7));
          dq[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dsf[c], kt8, dq[nb], 0, 0, 0);
        }
    }
  }
  kv_wait_vm<0>();   // the ring's trailing (empty) loads land before the workgroup ends
  // dq layout: lane = dim nb*32 + l32, registers = queries 8(i/4) + 4hi + i%4.  A row
  // with a self key (a T row) adds the self kernel's term, written before this kernel.
  const int hd = g.H * DH;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int qi = 8 * (i >> 2) + 4 * hi + (i & 3);
    if (qi >= nrows) continue;
    const int64_t qr = qrow0 + qi;
    const bool self = g.n[grow0 + qi] - g.p[grow0 + qi] > 0;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int col = h * DH + nb * 32 + l32;
      float v = dq[nb][i];
      if (self) v += g.dq[qr * hd + col];
      const float hqv = (float)g.hq[qr * g.ldhq + col];
      g.dhq[qr * g.lddhq + col] = (bf16)(v * g.dq_scale * dsilu_f(hqv));
    }
  }
}


// --------------------------------------------------------------------------
// dK / dV kernel.  One workgroup per (64-key context tile, group) with 2 HC
// waves: wave w takes key half w % 2 (32 keys, lane = key) and head w / 2 of
// the current chunk of HC heads (R / HC passes over the query stages); every
// wave sums its heads into one dK, dV accumulator.  The user's
// query tiles that see the keys are walked in stages of 32 queries: per head
// Q', dA/n hi and lo (32 rows x 128 B each), plus the 32 prefix limits, are
// brought into an LDS ring by buffer DMA one stage ahead.  S and dP come out
// with lane = key, so P and dS feed the dV / dK MFMAs straight from registers;
// the other operand (Q', dA/n with lane = head dimension, 8 queries per lane)
// is read from the row-major stage with the transposing LDS read.
constexpr int KV_NS = 2;                   // ring depth (stages)
constexpr int KV_TENSOR = 32 * 128;        // one 32-row tensor of a head
constexpr int KV_HEAD = 3 * KV_TENSOR;     // Q', dA/n hi, dA/n lo
constexpr int KV_CPW = 6;                  // 1 KB DMA chunks per wave per stage

// Two heads per pass and a two-stage ring (49.7 KB of LDS, at most 170 VGPRs)
// let three workgroups share a CU, so one workgroup's barrier waits, DMA waits
// and prologue / epilogue overlap the others' work: measured faster than four
// heads per pass (one workgroup per CU), one head per pass, and two heads with
// a three-stage ring (two workgroups per CU).
template <int R> struct DkvShape {
  static constexpr int HC = R < 2 ? R : 2;          // heads per pass
  static constexpr int NW = 2 * HC;                 // waves
  static constexpr int STAGE = HC * KV_HEAD + 256;  // + prefix limits (64 lanes x 4 B)
};

template <int R>
__global__ __launch_bounds__(128 * DkvShape<R>::HC, 3) void attn_bwd_dkv_kernel(AttnBwdArgs g) {
  using SH = DkvShape<R>;
  constexpr int HC = SH::HC, NW = SH::NW, STAGE = SH::STAGE;
  constexpr int NPASS = R / HC;
  static_assert(12 * HC == KV_CPW * NW, "chunks per stage");
  __shared__ __attribute__((aligned(1024))) char lds[KV_NS * STAGE];

  // every index below is wave-uniform: readfirstlane keeps the descriptor reads
  // on the scalar unit, away from the vector-memory counter that paces the ring
  auto uni = [](int v) { return __builtin_amdgcn_readfirstlane(v); };
  typedef __attribute__((address_space(4))) const int32_t cint;   // read-only for the whole launch
  const cint* qtl = (const cint*)g.qtiles;
  const int ntg = uni(g.user[UT_KTILE * (g.n_users + 1) + g.n_users]);
  const int lb = xcd_remap(blockIdx.x, ntg * g.G);
  const int ktg = lb / g.G, grp = lb % g.G;
  const int stride = g.n_users + 1;
  const int u = uni(upper_index(g.user + UT_KTILE * stride, g.n_users, ktg));
  const int kt = uni(ktg - g.user[UT_KTILE * stride + u]);
  const int lctx = uni(g.lens[3 * u] + g.lens[3 * u + 1]);
  const int urow0 = uni(g.user[UT_ROW * stride + u]);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kh = wave & 1, hw = wave >> 1;
  const int l32 = lane & 31, hi = lane >> 5;
  const int key0 = kt * 64 + kh * 32;
  const int key = key0 + l32;                    // this lane's key (context index)
  const bool kok = key < lctx;

  bf16x8 kf[4], vf[4];
  {
    const int64_t row = urow0 + (kok ? key : 0);
    const bf16* ks = g.k + row * g.ldk + grp * DH + 8 * hi;
    const bf16* vs = g.v + row * g.ldv + grp * DH + 8 * hi;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      kf[kk] = ld8(ks + kk * 16);
      vf[kk] = ld8(vs + kk * 16);
    }
  }

  // Stage cursor: pass (head chunk), query tile, 32-row half.  Tiles whose
  // queries see none of the keys are skipped.
  const int qt0 = uni(g.user[g.query_tiles_row * stride + u]);
  const int qt1 = uni(g.user[g.query_tiles_row * stride + u + 1]);
  auto next_tile = [&](int qt) {
    while (qt < qt1 && uni(qtl[8 * qt + TD_END]) <= kt) qt = uni(qt + 1);
    return qt;
  };
  struct Cur { int pass, qt, sub; };
  auto advance = [&](Cur& c) {
    if (c.sub == 0 && uni(qtl[8 * c.qt + TD_NROWS]) > 32) { c.sub = 1; return; }
    c.sub = 0;
    c.qt = next_tile(c.qt + 1);
    if (c.qt >= qt1) { ++c.pass; c.qt = next_tile(qt0); }
  };
  const int first = next_tile(qt0);
  Cur ci{first < qt1 ? 0 : NPASS, first, 0};   // issue cursor
  Cur cc = ci;                                  // compute cursor

  // DMA lane roles: chunk = 8 rows x 128 B; lane -> row 8 (chunk % 4) + lane / 8, slot lane % 8
  const int rin = lane >> 3, slot = lane & 7;
  auto issue = [&](int buf) {
    // stages past the last one are issued as empty loads (zero-size resources),
    // so that every wait sees the same number of DMA instructions in flight
    const bool real = ci.pass < NPASS;
    int rows = 0, grow = 0;
    int64_t qrow = 0;
    if (real) {
      const cint* td = qtl + 8 * ci.qt;
      rows = uni(min(32, td[TD_NROWS] - 32 * ci.sub));
      qrow = uni(td[TD_QROW0] + 32 * ci.sub);
      grow = uni(td[TD_GROW0] + 32 * ci.sub);
    }
    const int hbase = grp * R + (real ? ci.pass : 0) * HC;
    char* st = lds + buf * STAGE;
#pragma unroll
    for (int i = 0; i < KV_CPW; ++i) {
      const int c = i * NW + wave;            // chunk of the stage
      const int hh = c / 12, t = (c % 12) >> 2, rb = c & 3;
      const bf16* src = t == 0 ? g.q : (t == 1 ? g.dan : g.dan_lo);
      const int64_t ld = t == 0 ? g.ldq : g.lddan;
      const __amdgpu_buffer_rsrc_t rs =
          kv_rsrc(src + qrow * ld + (hbase + hh) * DH, (uint32_t)(rows * ld * 2));
      const int r = rb * 8 + rin;
      const uint32_t voff = (uint32_t)(r * ld * 2 + ((slot ^ kv_swz(r)) << 4));
      kv_dma(rs, (lds_void_t*)(st + hh * KV_HEAD + t * KV_TENSOR + rb * 1024), voff, 16);
    }
    if (wave == 0) {
      const __amdgpu_buffer_rsrc_t rs = kv_rsrc(g.p + grow, (uint32_t)(rows * 4));
      kv_dma(rs, (lds_void_t*)(st + HC * KV_HEAD), (uint32_t)(lane * 4), 4);
    }
    if (real) advance(ci);
  };
#pragma unroll
  for (int s = 0; s < KV_NS - 1; ++s) issue(s);

  f32x16 dk[2] = {f32x16{}, f32x16{}}, dv[2] = {f32x16{}, f32x16{}};
  // row-read offset (A operands: query l32, dims kk*16 + 8hi) and transposing-read offsets
  const int sw32 = kv_swz(l32);
  // transposing reads of fragment (c, nb, h2): row 16c + 8h2 + 4hi + m, columns
  // nb*32 + 16((lane/16)%2) + 4(lane%4) .. + 3, m = (lane/4)%4; c moves the row by 16
  // (2048 B) without changing the swizzle
  uint32_t tr_off[2][2];
  {
    const int tm = (lane >> 2) & 3, tcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int r = 8 * h2 + 4 * hi + tm;
        const int col = nb * 32 + tcol;
        tr_off[nb][h2] = (uint32_t)(r * 128 + (((col >> 3) ^ kv_swz(r)) << 4) + (col & 7) * 2);
      }
  }
  int it = 0;
  while (cc.pass < NPASS) {
    const int buf = it % KV_NS;
    if (wave == 0) kv_wait_vm<(KV_NS - 2) * (KV_CPW + 1)>();
    else kv_wait_vm<(KV_NS - 2) * KV_CPW>();
    kv_barrier();
    issue((it + KV_NS - 1) % KV_NS);
    const char* st = lds + buf * STAGE;
    const char* hb = st + hw * KV_HEAD;
    const uint32_t hb_addr = lds_addr(hb);
    const cint* td = qtl + 8 * cc.qt;
    const bool masked = !(kt < uni(td[TD_FULL_END]) && (kt + 1) * 64 <= lctx);

    f32x16 sc = {}, dp = {};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int off = l32 * 128 + (((2 * kk + hi) ^ sw32) << 4);
      const bf16x8 qa = *(const bf16x8*)(hb + off);
      const bf16x8 da = *(const bf16x8*)(hb + KV_TENSOR + off);
      const bf16x8 dl = *(const bf16x8*)(hb + 2 * KV_TENSOR + off);
      sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kf[kk], sc, 0, 0, 0);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da, vf[kk], dp, 0, 0, 0);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dl, vf[kk], dp, 0, 0, 0);
    }
    // layout: lane = key, registers = queries 8(i/4) + 4hi + i%4
    int plim[16] = {};
    if (masked) {
      int4 pv4[4];
      kv_plim(lds_addr(st + HC * KV_HEAD + 16 * hi), pv4);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        plim[4 * j] = pv4[j].x; plim[4 * j + 1] = pv4[j].y; plim[4 * j + 2] = pv4[j].z; plim[4 * j + 3] = pv4[j].w;
      }
    }
    if (masked) {
#pragma unroll
      for (int i = 0; i < 16; ++i) sc[i] = key < plim[i] ? sc[i] : kMaskedScore;
    }
    // P is kept as P / ln2 (ln2 applied to dV at the end)
    bf16x8 pf[2], dsf[2];
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int i = 8 * c + e;
        float pv, dsg;
        silu_grad_scaled(sc[i], &pv, &dsg);
        pf[c][e] = (bf16)pv;
        dsf[c][e] = (bf16)(dp[i] * dsg);
      }
    // dV += P^T dA/n, dK += dS^T Q' over this stage's 32 queries: k slot (hi, e) of
    // pf[c] is query 16c + 8(e/4) + 4hi + e%4, the transposing reads match it
    i16x4 q4[2][2][2], d4[2][2][2];
    {
      uint32_t ta[2][2];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) ta[nb][h2] = hb_addr + tr_off[nb][h2];
      kv_tr16(ta, q4, d4);
    }
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const bf16x8 qt8 = __builtin_bit_cast(bf16x8, __builtin_shufflevector(q4[c][nb][0], q4[c][nb][1], 0, 1, 2, 3, 4, 5, 6, 7));
        const bf16x8 dt8 = __builtin_bit_cast(bf16x8, __builtin_shufflevector(d4[c][nb][0], d4[c][nb][1], 0, 1, 2, 3, 4, 5, 6, 7));
        dv[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pf[c], dt8, dv[nb], 0, 0, 0);
        dk[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dsf[c], qt8, dk[nb], 0, 0, 0);
      }
    advance(cc);
    ++it;
  }
  // drain the ring (the last issued stages are empty), then sum the heads of
  // each key half in a fixed order and apply SiLU' of the K / V pre-activations:
  // dK first, then dV, each through a [NW][32 keys][64 dims] fp32 buffer in the
  // (then idle) ring
  static_assert(NW * 32 * DH * 4 <= KV_NS * STAGE, "reduction buffer fits in the ring");
  kv_wait_vm<0>();
  kv_barrier();
  float* red = reinterpret_cast<float*>(lds);
#pragma unroll
  for (int part = 0; part < 2; ++part) {
    const f32x16* acc = part ? dv : dk;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int kr = 8 * (i >> 2) + 4 * hi + (i & 3);
        red[(wave * 32 + kr) * DH + nb * 32 + l32] = acc[nb][i];
      }
    __syncthreads();
    const bf16* hsrc = part ? g.hv : g.hk;
    const int64_t ldh = part ? g.ldhv : g.ldhk;
    bf16* dst = part ? g.dhv : g.dhk;
    const int64_t ldd = part ? g.lddhv : g.lddhk;
    for (int e = tid; e < 64 * DH; e += 64 * NW) {
      const int kr64 = e / DH, c = e % DH;
      const int half = kr64 >> 5, kr = kr64 & 31;
      if (kt * 64 + kr64 >= lctx) continue;
      float sum = 0.f;
      for (int w = 0; w < HC; ++w) sum += red[((2 * w + half) * 32 + kr) * DH + c];
      const int64_t row = urow0 + kt * 64 + kr64;
      const float h = (float)hsrc[row * ldh + grp * DH + c];
      dst[row * ldd + grp * DH + c] = (bf16)(sum * kLn2 * dsilu_f(h));
    }
    __syncthreads();
  }
}

// --------------------------------------------------------------------------
// T-row self term: one wave per (T row, group), lane = head dimension.
__global__ __launch_bounds__(256) void attn_bwd_self_kernel(AttnBwdArgs g) {
  const int w = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (w >= g.n_self_rows * g.G) return;
  const int i = w / g.G, grp = w % g.G;
  const int c = threadIdx.x & 63;
  const int64_t qs = map_b(g.self_rows, i), gs = map_b(g.self_packed, i);
  const int r = g.H / g.G;
  const float k = (float)g.ks[qs * g.ldks + grp * DH + c];
  const float v = (float)g.vs[qs * g.ldvs + grp * DH + c];
  const bool self = g.n[gs] - g.p[gs] > 0;
  float dk = 0.f, dv = 0.f;
  const int hd = g.H * DH;
  for (int hh = 0; hh < r && self; ++hh) {
    const int h = grp * r + hh;
    const float q = (float)g.q[qs * g.ldq + h * DH + c];
    const float da = (float)g.dan[qs * g.lddan + h * DH + c] + (float)g.dan_lo[qs * g.lddan + h * DH + c];
    const float sp = wave_sum(q * k), dpv = wave_sum(da * v);
    float pv, dsg;
    silu_and_grad(sp, &pv, &dsg);
    const float ds = dpv * dsg;
    g.dq[qs * hd + h * DH + c] = ds * k;   // added by the dQ kernel, which runs next
    dk += ds * q * kLn2;
    dv += pv * da;
  }
  const float hk = (float)g.hks[qs * g.ldhks + grp * DH + c];
  const float hv = (float)g.hvs[qs * g.ldhvs + grp * DH + c];
  g.dhks[qs * g.lddhks + grp * DH + c] = (bf16)(dk * dsilu_f(hk));
  g.dhvs[qs * g.lddhvs + grp * DH + c] = (bf16)(dv * dsilu_f(hv));
}

template <int R>
mtfm_status launch_r(const AttnBwdArgs& a, int64_t n_key_tiles, hipStream_t s) {
  // the self term first: the dQ kernel adds it to the T rows' dQ
  if (a.n_self_rows > 0) {
    attn_bwd_self_kernel<<<(unsigned)((a.n_self_rows * a.G + 3) / 4), 256, 0, s>>>(a);
    MTFM_LAUNCH_CHECK("attn_bwd_self");
  }
  if (a.nqtiles > 0) {
    attn_bwd_dq_kernel<R><<<(unsigned)(a.nqtiles * a.G * 2), 64 * R, 0, s>>>(a);
    MTFM_LAUNCH_CHECK("attn_bwd_dq");
  }
  if (n_key_tiles > 0 && a.nqtiles > 0) {
    attn_bwd_dkv_kernel<R><<<(unsigned)(n_key_tiles * a.G), 128 * DkvShape<R>::HC, 0, s>>>(a);
    MTFM_LAUNCH_CHECK("attn_bwd_dkv");
  }
  return MTFM_OK;
}

}  // namespace

mtfm_status launch_attn_bwd(const AttnBwdArgs& a, int64_t n_key_tiles, hipStream_t s) {
  switch (a.H / a.G) {
    case 1: return launch_r<1>(a, n_key_tiles, s);
    case 2: return launch_r<2>(a, n_key_tiles, s);
    case 4: return launch_r<4>(a, n_key_tiles, s);
    case 8: return launch_r<8>(a, n_key_tiles, s);
    default: return MTFM_E_UNSUPPORTED;
  }
}
