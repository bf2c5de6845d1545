// Backward of the masked pointwise-SiLU attention (bf16 MFMA, fp32 accumulate).
//
// With s' = Q' K^T (Q' = Q log2(e)/sqrt(dh), so x = s' ln2 is the scaled
// score), P = SiLU(x) on visible pairs, A = P V / n and dAn = dA / n:
//   dP  = dAn V^T,   dS = dP (.) SiLU'(x) on visible pairs,
//   dQ  = dS K / sqrt(dh),   dK = dS^T Q / sqrt(dh) = ln2 dS^T Q',   dV = P^T dAn,
// with dK, dV of a KV group summed over its r query heads ([explainer] §4.1
// GQA).  Three kernels, none with atomics:
//   * dq:  one workgroup per (32-row query slice, group), one wave per head;
//          loops over the visible context key tiles like the forward (K, K^T
//          and V tiles staged in LDS), S^T and dP^T accumulate with lane =
//          query so dS feeds the dQ MFMA straight from registers.
//   * dkv: one workgroup per (32-key context slice, group), one wave per head;
//          loops over the user's query tiles that see the keys, S and dP with
//          lane = key so P and dS feed the dV / dK MFMAs from registers; the r
//          heads' dK, dV are summed through LDS in a fixed order.
//   * self: one wave per (T row, group): the T row's only T key is itself
//          ([blog] §3.2), so its term is a few dot products.

#include "bwd_kernels.h"

namespace {

constexpr int DH = 64;
constexpr int KS = DH + 8;  // row-major tile stride (144 B)
constexpr int VS = 64 + 4;  // transposed tile stride (136 B)
constexpr float kLn2 = 0.69314718055994530942f;

MTFM_DEV int xcd_remap(int bid, int nblocks) {
  const int q = nblocks >> 3, r = nblocks & 7;
  const int x = bid & 7, k = bid >> 3;
  return x * q + min(x, r) + k;
}

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

MTFM_DEV bf16x8 ld8(const bf16* p) { return *(const bf16x8*)p; }

MTFM_DEV bf16x8 tr_frag(const bf16* base, int row, int col) {
  // slots s < 4: columns col + s;  s >= 4: columns col + 8 + (s - 4)
  const bf16x4 lo4 = *(const bf16x4*)(base + row * VS + col);
  const bf16x4 hi4 = *(const bf16x4*)(base + row * VS + col + 8);
  return __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
}

// --------------------------------------------------------------------------
template <int R>
__global__ __launch_bounds__(64 * R, 2) void attn_bwd_dq_kernel(AttnBwdArgs g) {
  constexpr int NT = 64 * R;
  constexpr int PPT = (256 + NT - 1) / NT;  // K (key pair, 8 dims) items per thread
  constexpr int VPT = (512 + NT - 1) / NT;  // V 16-B chunks per thread
  __shared__ __attribute__((aligned(16))) bf16 Ks[2][64 * KS];
  __shared__ __attribute__((aligned(16))) bf16 Kt[2][DH * VS];
  __shared__ __attribute__((aligned(16))) bf16 Vs[2][64 * KS];

  const int nblocks = g.nqtiles * g.G * 2;
  const int lb = xcd_remap(blockIdx.x, nblocks);
  const int slice = lb & 1;
  const int tile = (lb >> 1) / g.G, grp = (lb >> 1) % g.G;
  const int32_t* td = g.qtiles + 8 * tile;
  const int u = td[TD_USER], tile_rows = td[TD_NROWS];
  const int full_end = td[TD_FULL_END], key_end = td[TD_END];
  const int qoff = slice * 32;
  const int nrows = min(32, tile_rows - qoff);
  if (nrows <= 0) return;
  const int grow0 = td[TD_GROW0] + qoff, qrow0 = td[TD_QROW0] + qoff, urow0 = td[TD_UROW0];
  const int lctx = g.lens[3 * u] + g.lens[3 * u + 1];
  const int ntl = key_end;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = grp * R + wave;
  const int l32 = lane & 31, hi = lane >> 5;
  const bool qok = l32 < nrows;

  bf16x8 qf[4], df[4], dl[4];
  {
    const int64_t qrow = qrow0 + (qok ? l32 : 0);
    const bf16* qs = g.q + qrow * g.ldq + h * DH + 8 * hi;
    const bf16* ds = g.dan + qrow * g.lddan + h * DH + 8 * hi;
    const bf16* dls = g.dan_lo + qrow * g.lddan + h * DH + 8 * hi;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      qf[kk] = qok ? ld8(qs + kk * 16) : bf16x8{};
      df[kk] = qok ? ld8(ds + kk * 16) : bf16x8{};
      dl[kk] = qok ? ld8(dls + kk * 16) : bf16x8{};
    }
  }
  const int plim = qok ? g.p[grow0 + l32] : 0;

  bf16x8 rk[PPT][2], rv[VPT];
  auto load_tile = [&](int it) {
    const int base = urow0 + it * 64;
    const int lim = min(64, lctx - it * 64);
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const int c = tid + NT * i;
      const int jp = c & 31, kc = c >> 5, j = 2 * jp;
      const bool in = c < 256;
      rk[i][0] = (in && j < lim) ? ld8(g.k + (int64_t)(base + j) * g.ldk + grp * DH + kc * 8) : bf16x8{};
      rk[i][1] = (in && j + 1 < lim) ? ld8(g.k + (int64_t)(base + j + 1) * g.ldk + grp * DH + kc * 8) : bf16x8{};
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int c = tid + NT * i;
      const int j = c >> 3, kc = c & 7;
      rv[i] = (c < 512 && j < lim) ? ld8(g.v + (int64_t)(base + j) * g.ldv + grp * DH + kc * 8) : bf16x8{};
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const int c = tid + NT * i;
      if (c >= 256) continue;
      const int jp = c & 31, kc = c >> 5, j = 2 * jp;
      *(bf16x8*)(&Ks[buf][j * KS + kc * 8]) = rk[i][0];
      *(bf16x8*)(&Ks[buf][(j + 1) * KS + kc * 8]) = rk[i][1];
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        bf16x2 pr;
        pr[0] = rk[i][0][s];
        pr[1] = rk[i][1][s];
        *(bf16x2*)(&Kt[buf][(kc * 8 + s) * VS + j]) = pr;
      }
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int c = tid + NT * i;
      if (c < 512) *(bf16x8*)(&Vs[buf][(c >> 3) * KS + (c & 7) * 8]) = rv[i];
    }
  };

  f32x16 dq[2] = {f32x16{}, f32x16{}};
  if (ntl > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();
  for (int it = 0; it < ntl; ++it) {
    const int buf = it & 1;
    if (it + 1 < ntl) load_tile(it + 1);
    const bool masked = it >= full_end || (it + 1) * 64 > lctx;
    const int lim = plim - it * 64;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 st = {}, dpt = {};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const bf16x8 kf = ld8(&Ks[buf][(kb * 32 + l32) * KS + kk * 16 + 8 * hi]);
        const bf16x8 vf = ld8(&Vs[buf][(kb * 32 + l32) * KS + kk * 16 + 8 * hi]);
        st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[kk], st, 0, 0, 0);
        dpt = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, df[kk], dpt, 0, 0, 0);
        dpt = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, dl[kk], dpt, 0, 0, 0);
      }
      bf16x8 dsf[2];
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const int i = 8 * c + s;
          float pv, dsg;
          silu_and_grad(st[i], &pv, &dsg);
          float d = dpt[i] * dsg;
          if (masked) {
            const int key = kb * 32 + 8 * (i >> 2) + 4 * hi + (i & 3);
            d = key < lim ? d : 0.f;
          }
          dsf[c][s] = (bf16)d;
        }
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          const bf16x8 kt = tr_frag(Kt[buf], nb * 32 + l32, kb * 32 + 16 * c + 4 * hi);
          dq[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dsf[c], kt, dq[nb], 0, 0, 0);
        }
    }
    if (it + 1 < ntl) store_tile(buf ^ 1);
    __syncthreads();
  }
  // dq layout: lane = dim nb*32 + l32, registers = queries 8(i/4) + 4hi + i%4
  const int hd = g.H * DH;
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int qi = 8 * (i >> 2) + 4 * hi + (i & 3);
      if (qi < nrows) g.dq[(int64_t)(qrow0 + qi) * hd + h * DH + nb * 32 + l32] = dq[nb][i];
    }
}

// --------------------------------------------------------------------------
template <int R>
__global__ __launch_bounds__(64 * R, 2) void attn_bwd_dkv_kernel(AttnBwdArgs g) {
  __shared__ __attribute__((aligned(16))) bf16 stage[R][2][DH * VS];  // per wave: Q'^T, dAn^T

  const int n_key_tiles_total = g.user[UT_KTILE * (g.n_users + 1) + g.n_users];
  const int nblocks = n_key_tiles_total * g.G * 2;
  const int lb = xcd_remap(blockIdx.x, nblocks);
  const int half = lb & 1;
  const int ktg = (lb >> 1) / g.G, grp = (lb >> 1) % g.G;
  const int stride = g.n_users + 1;
  const int u = upper_index(g.user + UT_KTILE * stride, g.n_users, ktg);
  const int kt = ktg - g.user[UT_KTILE * stride + u];
  const int lctx = g.lens[3 * u] + g.lens[3 * u + 1];
  const int key0 = kt * 64 + half * 32;
  const int nkeys = min(32, lctx - key0);
  if (nkeys <= 0) return;
  const int urow0 = g.user[UT_ROW * stride + u];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = grp * R + wave;
  const int l32 = lane & 31, hi = lane >> 5;
  const bool kok = l32 < nkeys;

  bf16x8 kf[4], vf[4];
  {
    const bf16* ks = g.k + (int64_t)(urow0 + key0 + (kok ? l32 : 0)) * g.ldk + grp * DH + 8 * hi;
    const bf16* vs = g.v + (int64_t)(urow0 + key0 + (kok ? l32 : 0)) * g.ldv + grp * DH + 8 * hi;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      kf[kk] = kok ? ld8(ks + kk * 16) : bf16x8{};
      vf[kk] = kok ? ld8(vs + kk * 16) : bf16x8{};
    }
  }
  f32x16 dk[2] = {f32x16{}, f32x16{}}, dv[2] = {f32x16{}, f32x16{}};
  bf16* Qt = stage[wave][0];
  bf16* Dt = stage[wave][1];
  const int key = key0 + l32;  // this lane's key (context index)

  const int qt0 = g.user[g.query_tiles_row * stride + u], qt1 = g.user[g.query_tiles_row * stride + u + 1];
  for (int qt = qt0; qt < qt1; ++qt) {
    const int32_t* td = g.qtiles + 8 * qt;
    if (td[TD_END] <= kt) continue;  // no query of this tile sees the key tile
    const int nrows = td[TD_NROWS], grow0 = td[TD_GROW0], qrow0 = td[TD_QROW0];
    const bool masked = !(kt < td[TD_FULL_END] && (kt + 1) * 64 <= lctx);
    // stage this head's Q'^T and dAn^T (64 queries x 64 dims) transposed
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = lane + 64 * i;            // (query pair, dim chunk)
      const int qp = c & 31, kc = c >> 5, q = 2 * qp;
      bf16x8 a0 = q < nrows ? ld8(g.q + (int64_t)(qrow0 + q) * g.ldq + h * DH + kc * 8) : bf16x8{};
      bf16x8 a1 = q + 1 < nrows ? ld8(g.q + (int64_t)(qrow0 + q + 1) * g.ldq + h * DH + kc * 8) : bf16x8{};
      bf16x8 b0 = q < nrows ? ld8(g.dan + (int64_t)(qrow0 + q) * g.lddan + h * DH + kc * 8) : bf16x8{};
      bf16x8 b1 = q + 1 < nrows ? ld8(g.dan + (int64_t)(qrow0 + q + 1) * g.lddan + h * DH + kc * 8) : bf16x8{};
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        bf16x2 pa, pb;
        pa[0] = a0[s]; pa[1] = a1[s];
        pb[0] = b0[s]; pb[1] = b1[s];
        *(bf16x2*)(&Qt[(kc * 8 + s) * VS + q]) = pa;
        *(bf16x2*)(&Dt[(kc * 8 + s) * VS + q]) = pb;
      }
    }
    __syncthreads();
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int qi = qb * 32 + l32;
      const bool qok = qi < nrows;
      f32x16 s = {}, dp = {};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const bf16x8 qa = qok ? ld8(g.q + (int64_t)(qrow0 + qi) * g.ldq + h * DH + kk * 16 + 8 * hi) : bf16x8{};
        const int64_t doff = (int64_t)(qrow0 + qi) * g.lddan + h * DH + kk * 16 + 8 * hi;
        const bf16x8 da = qok ? ld8(g.dan + doff) : bf16x8{};
        const bf16x8 dl = qok ? ld8(g.dan_lo + doff) : bf16x8{};
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kf[kk], s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da, vf[kk], dp, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dl, vf[kk], dp, 0, 0, 0);
      }
      // layout: lane = key (l32), registers = queries qb*32 + 8(i/4) + 4hi + i%4
      bf16x8 pf[2], dsf[2];
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int i = 8 * c + e;
          float pv, dsg;
          silu_and_grad(s[i], &pv, &dsg);
          float d = dp[i] * dsg;
          if (masked) {
            const int q = qb * 32 + 8 * (i >> 2) + 4 * hi + (i & 3);
            const bool vis = q < nrows && key < g.p[grow0 + q];
            pv = vis ? pv : 0.f;
            d = vis ? d : 0.f;
          }
          pf[c][e] = (bf16)pv;
          dsf[c][e] = (bf16)d;
        }
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          const bf16x8 dt = tr_frag(Dt, nb * 32 + l32, qb * 32 + 16 * c + 4 * hi);
          const bf16x8 qtf = tr_frag(Qt, nb * 32 + l32, qb * 32 + 16 * c + 4 * hi);
          dv[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pf[c], dt, dv[nb], 0, 0, 0);
          dk[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dsf[c], qtf, dk[nb], 0, 0, 0);
        }
    }
  }
  // sum the r heads in a fixed order through LDS, then apply SiLU' of the K / V pre-activations
  __syncthreads();
  float* red = reinterpret_cast<float*>(&stage[0][0][0]);  // [R][2][32 keys][64 dims]
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int kr = 8 * (i >> 2) + 4 * hi + (i & 3);
      red[((wave * 2 + 0) * 32 + kr) * DH + nb * 32 + l32] = dk[nb][i];
      red[((wave * 2 + 1) * 32 + kr) * DH + nb * 32 + l32] = dv[nb][i];
    }
  __syncthreads();
  for (int e = tid; e < 32 * DH; e += 64 * R) {
    const int kr = e / DH, c = e % DH;
    if (kr >= nkeys) continue;
    float sk = 0.f, sv = 0.f;
    for (int w = 0; w < R; ++w) {
      sk += red[((w * 2 + 0) * 32 + kr) * DH + c];
      sv += red[((w * 2 + 1) * 32 + kr) * DH + c];
    }
    const int64_t row = urow0 + key0 + kr;
    const float hk = (float)g.hk[row * g.ldhk + grp * DH + c];
    const float hv = (float)g.hv[row * g.ldhv + grp * DH + c];
    g.dhk[row * g.lddhk + grp * DH + c] = (bf16)(sk * kLn2 * dsilu_f(hk));
    g.dhv[row * g.lddhv + grp * DH + c] = (bf16)(sv * dsilu_f(hv));
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
    g.dq[qs * hd + h * DH + c] += ds * k;
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
  if (a.nqtiles > 0) {
    attn_bwd_dq_kernel<R><<<(unsigned)(a.nqtiles * a.G * 2), 64 * R, 0, s>>>(a);
    MTFM_LAUNCH_CHECK("attn_bwd_dq");
  }
  if (n_key_tiles > 0 && a.nqtiles > 0) {
    attn_bwd_dkv_kernel<R><<<(unsigned)(n_key_tiles * a.G * 2), 64 * R, 0, s>>>(a);
    MTFM_LAUNCH_CHECK("attn_bwd_dkv");
  }
  if (a.n_self_rows > 0) {
    attn_bwd_self_kernel<<<(unsigned)((a.n_self_rows * a.G + 3) / 4), 256, 0, s>>>(a);
    MTFM_LAUNCH_CHECK("attn_bwd_self");
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
