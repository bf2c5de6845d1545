// Backward of the full- and target-attention layers (bf16 path).
//
// Gradients of L = sum(X' (.) dY) with respect to X, the projection weights
// and the group-LayerNorm parameters, for the layer equations of
// [explainer] §4.1 (full) and §4.2 (target; V2 per-sub-token Q of [blog]
// §3.3.2).  Each call first recomputes the forward into the workspace,
// keeping the pre-SiLU projections, then runs the chain
//   dW_o = dY^T Y,  dY~ = dY W_o,
//   GLN2 backward   -> dU (.) SiLU'(h_U), dA / n,  dgamma2, dbeta2
//   attention bwd   -> dQ, dK, dV (.) SiLU'(h)
//   dW = dH^T X~,   dX~ = dH W,
//   GLN1 backward   -> dX (+ dY through the residual), dgamma1, dbeta1.
// Weight gradients accumulate in fp32 over all packed rows (split partial
// sums added in a fixed order); nothing uses atomics, so results are
// deterministic.

#include <algorithm>

#include "api_internal.h"
#include "bwd_kernels.h"

namespace {

struct BwdWs {
  int64_t xt, z, hpre, kv, kvpre, vt, ldvt, a, y, wot, w1t, wkvt, dyv, dan, dan_lo, dq, dh, dhkv, dxt, pg, part;
  int64_t part_elems, pg_blocks, total;
};

BwdWs bwd_layout(const MetaPlan& p, const mtfm_dims* d, int op) {
  const int64_t D = d->d_model;
  const int64_t hd = (int64_t)d->n_q_heads * d->head_dim, gd = (int64_t)d->n_kv_heads * d->head_dim;
  const int64_t zw = 2 * hd + 2 * gd;
  const int64_t R = p.n_rows, T = p.n_t_rows, S = p.split;
  const bool full = op == MTFM_OP_FULL_BWD;
  const int64_t Q = full ? R : T;  // rows of the query space
  BwdWs w{};
  int64_t off = 0;
  auto take = [&](int64_t bytes) { int64_t o = off; off = align_up(off + std::max<int64_t>(bytes, 0), 256); return o; };
  w.xt = take(R * D * 2);
  w.z = take(Q * zw * 2);
  w.hpre = take(Q * zw * 2);
  w.kv = full ? 0 : take(R * 2 * gd * 2);
  w.kvpre = full ? 0 : take(R * 2 * gd * 2);
  w.ldvt = vt_ld(R);
  w.vt = take(gd * w.ldvt * 2);
  w.a = take(Q * hd * 2);
  w.y = take(Q * hd * 2);
  w.wot = take(hd * D * 2);
  w.w1t = take(S * D * zw * 2);
  w.wkvt = full ? 0 : take(D * 2 * gd * 2);
  w.dyv = take(Q * hd * 4);
  w.dan = take(Q * hd * 2);
  w.dan_lo = take(Q * hd * 2);
  w.dq = take(Q * hd * 4);
  w.dh = take(Q * zw * 2);
  w.dhkv = full ? 0 : take(R * 2 * gd * 2);
  w.dxt = take(R * D * 4);
  w.pg_blocks = gln_bwd_grid((int)std::max<int64_t>(R, 1));
  w.pg = take(w.pg_blocks * 6 * std::max<int64_t>(D, hd) * 4);
  // largest weight-gradient product: [zw][D] over all rows, or [hd][D] per sub-token group
  int64_t pe = gemm_tn_partial_elems((int32_t)zw, (int32_t)D, (int32_t)std::max<int64_t>(R, 1), 1);
  pe = std::max(pe, gemm_tn_partial_elems((int32_t)D, (int32_t)hd, (int32_t)std::max<int64_t>(Q, 1), 1));
  pe = std::max(pe, gemm_tn_partial_elems((int32_t)hd, (int32_t)D, (int32_t)std::max<int64_t>(p.n_parents, 1),
                                          (int32_t)S));
  w.part_elems = pe;
  w.part = take(pe * 4);
  w.total = off;
  return w;
}

RowMap list_map(const int32_t* list, int div = 1, int add = 0) { return RowMap{list, 0, add, div}; }

// C = sum over r < R of A[am(r)]^T B[bm(r)]; a_rows, b_rows = rows of the A, B buffers
mtfm_status tn(hipStream_t s, const BwdWs& L, char* ws, int M, int N, int R, const void* A, int64_t lda, RowMap am,
               int64_t a_rows, const void* B, int64_t ldb, RowMap bm, int64_t b_rows, float* C, int accumulate,
               int groups = 1, int azadd = 0, int bzadd = 0, int64_t czoff = 0) {
  GemmTNArgs t{};
  t.M = M; t.N = N; t.R = R; t.groups = groups;
  t.A = A; t.lda = lda; t.amap = am; t.amap_zadd = azadd; t.a_rows = a_rows;
  t.B = B; t.ldb = ldb; t.bmap = bm; t.bmap_zadd = bzadd; t.b_rows = b_rows;
  t.C = C; t.ldc = N; t.c_zoff = czoff; t.accumulate = accumulate;
  t.partial = (float*)(ws + L.part); t.partial_elems = L.part_elems;
  TimedLaunch tl(MTFM_K_BWD, s);
  return launch_gemm_tn(t, s);
}

mtfm_status transpose(hipStream_t s, const void* a, int ra, const void* b, int rb, const void* c, int rc, int cols,
                      void* out, int64_t ldo) {
  TransposeArgs t{};
  t.in[0] = (const bf16*)a; t.seg_rows[0] = ra;
  t.in[1] = (const bf16*)b; t.seg_rows[1] = rb;
  t.in[2] = (const bf16*)c; t.seg_rows[2] = rc;
  t.rows = ra + rb + rc; t.cols = cols;
  t.out = (bf16*)out; t.ldo = ldo;
  return launch_transpose(t, s);
}

mtfm_status check_bwd_dims(const mtfm_dims* d) {
  if (d->dtype != MTFM_BF16) return MTFM_E_UNSUPPORTED;  // the backward runs on the bf16 path only
  const int hd = d->n_q_heads * d->head_dim;
  // row kernels: 4, 8 or 16 values per lane
  auto ok = [](int w) { return w == 256 || w == 512 || w == 1024; };
  if (!ok(d->d_model) || !ok(hd)) return MTFM_E_UNSUPPORTED;
  return MTFM_OK;
}

}  // namespace

int64_t bwd_ws_bytes(const MetaPlan& p, const mtfm_dims* d, int op) {
  if (check_bwd_dims(d) != MTFM_OK) return 0;
  return bwd_layout(p, d, op).total;
}

// ---------------------------------------------------------------------------
mtfm_status run_full_bwd(const Ctx& c, const mtfm_dims* d, const mtfm_full_w* w, const void* x_in, const void* dy,
                         void* dx, const mtfm_full_grad* gr, char* ws, const FwdKeep* keep) {
  TRY(check_bwd_dims(d));
  const MetaPlan& p = c.plan;
  const hipStream_t s = c.s;
  const int H = d->n_q_heads, G = d->n_kv_heads, dh = d->head_dim, D = d->d_model;
  const int hd = H * dh, gd = G * dh, zw = 2 * hd + 2 * gd;
  const int R = (int)p.n_rows;
  const BwdWs L = bwd_layout(p, d, MTFM_OP_FULL_BWD);
  bf16* xt = (bf16*)(keep ? keep->xt : ws + L.xt);
  bf16* z = (bf16*)(keep ? keep->z : ws + L.z);
  bf16* hpre = (bf16*)(keep ? keep->hpre : ws + L.hpre);
  bf16* a = (bf16*)(keep ? keep->a : ws + L.a);
  bf16* y = (bf16*)(ws + L.y);
  bf16* wot = (bf16*)(ws + L.wot);
  bf16* w1t = (bf16*)(ws + L.w1t);
  float* dyv = (float*)(ws + L.dyv);
  bf16* dan = (bf16*)(ws + L.dan);
  bf16* dan_lo = (bf16*)(ws + L.dan_lo);
  float* dq = (float*)(ws + L.dq);
  bf16* dh_ = (bf16*)(ws + L.dh);
  float* dxt = (float*)(ws + L.dxt);
  float* pg = (float*)(ws + L.pg);
  if (R == 0) return MTFM_OK;

  // ---- forward recompute (keeps pre-activations), unless the forward pass kept it
  if (!keep) {
    GlnArgs g1{};
    g1.rows = R; g1.D = D; g1.x = x_in; g1.ldx = D; g1.y = xt; g1.ldy = D;
    g1.gamma = w->ln1_g; g1.beta = w->ln1_b; g1.type = c.meta.type; g1.eps = d->ln_eps;
    TRY(timed_gln(g1, MTFM_BF16, s));
    GemmArgs gp{};
    gp.M = R; gp.N = zw; gp.K = D; gp.groups = 1;
    gp.A = xt; gp.lda = D; gp.amap = identity_map();
    gp.B[0] = w->w_uqkv; gp.bn[0] = zw; gp.ldb = D;
    gp.cmap = identity_map();
    gp.epi = EPI_SILU_SPLIT;
    gp.dst[0] = z; gp.ld[0] = zw; gp.cend[0] = hd; gp.scale[0] = 1.f;
    gp.dst[1] = z + hd; gp.ld[1] = zw; gp.cend[1] = 2 * hd; gp.scale[1] = q_scale(dh);
    gp.dst[2] = z + 2 * hd; gp.ld[2] = zw; gp.cend[2] = zw; gp.scale[2] = 1.f;
    gp.cend[3] = zw;
    gp.pre = hpre; gp.ldpre = zw;
    gp.vt = ws + L.vt; gp.ldvt = L.ldvt; gp.vt_col0 = 2 * hd + gd; gp.vt_cols = gd;
    TRY(timed_gemm(MTFM_K_GEMM_UQKV, gp, MTFM_BF16, s));
    {
      AttnArgs aa{};
      aa.q = z + hd; aa.ldq = zw; aa.k = z + 2 * hd; aa.ldk = zw; aa.v = z + 2 * hd + gd; aa.ldv = zw;
      aa.vt = ws + L.vt; aa.ldvt = L.ldvt; aa.n_key_rows = R; aa.max_user_rows = p.max_user_rows;
      aa.kd = aa.k; aa.ldkd = zw; aa.vd = aa.v; aa.ldvd = zw;
      aa.a = a; aa.lda = hd;
      aa.tiles = c.meta.full_tiles; aa.ntiles = (int32_t)p.n_full_tiles;
      aa.order = c.meta.full_order; aa.n_order = (int32_t)p.n_full_order;
      aa.p = c.meta.p; aa.n = c.meta.n; aa.lens = c.b->lens_d;
      aa.H = H; aa.G = G; aa.dh = dh; aa.out_scale = kLn2;
      TRY(timed_attention(MTFM_K_ATTN_FULL, aa, MTFM_BF16, s));
    }
  }
  GlnArgs g2{};
  g2.rows = R; g2.D = hd; g2.x = a; g2.ldx = hd; g2.y = y; g2.ldy = hd; g2.gate = z; g2.ldg = zw;
  g2.gamma = w->ln2_g; g2.beta = w->ln2_b; g2.type = c.meta.type; g2.eps = d->ln_eps;
  TRY(timed_gln(g2, MTFM_BF16, s));

  // ---- output projection
  TRY(tn(s, L, ws, D, hd, R, dy, D, identity_map(), R, y, hd, identity_map(), R, gr->w_o, 0));
  TRY(transpose(s, w->w_o, D, nullptr, 0, nullptr, 0, hd, wot, D));
  {
    GemmArgs gd_{};
    gd_.M = R; gd_.N = hd; gd_.K = D; gd_.groups = 1;
    gd_.A = dy; gd_.lda = D; gd_.amap = identity_map();
    gd_.B[0] = wot; gd_.bn[0] = hd; gd_.ldb = D;
    gd_.cmap = identity_map(); gd_.epi = EPI_STORE_F32; gd_.out = dyv; gd_.ldo = hd;
    TimedLaunch tl(MTFM_K_BWD, s);
    TRY(launch_gemm(gd_, MTFM_BF16, s));
  }
  // ---- GLN2 (gated) backward
  {
    Gln2BwdArgs b{};
    b.rows = R; b.D = hd; b.a = a; b.lda = hd; b.gamma = w->ln2_g; b.beta = w->ln2_b;
    b.type = c.meta.type; b.nmap = RowMapB{nullptr, 1}; b.n = c.meta.n; b.eps = d->ln_eps;
    b.u = z; b.ldu = zw; b.hu = hpre; b.ldhu = zw; b.dy = dyv; b.lddy = hd;
    b.dhu = dh_; b.lddhu = zw; b.dan = dan; b.dan_lo = dan_lo; b.lddan = hd; b.pg = pg;
    TimedLaunch tl(MTFM_K_BWD, s);
    TRY(launch_gln2_bwd(b, s));
    TRY(launch_param_reduce(pg, gln_bwd_grid(R), hd, gr->ln2_g, gr->ln2_b, s));
  }
  // ---- attention backward
  {
    AttnBwdArgs b{};
    b.q = z + hd; b.ldq = zw; b.k = z + 2 * hd; b.ldk = zw; b.v = z + 2 * hd + gd; b.ldv = zw;
    b.dan = dan; b.dan_lo = dan_lo; b.lddan = hd;
    b.qtiles = c.meta.full_tiles; b.nqtiles = (int32_t)p.n_full_tiles;
    b.user = c.meta.user; b.n_users = p.n_users; b.query_tiles_row = UT_FTILE;
    b.p = c.meta.p; b.n = c.meta.n; b.lens = c.b->lens_d; b.H = H; b.G = G;
    b.dq = dq;
    b.hk = hpre + 2 * hd; b.ldhk = zw; b.hv = hpre + 2 * hd + gd; b.ldhv = zw;
    b.dhk = dh_ + 2 * hd; b.lddhk = zw; b.dhv = dh_ + 2 * hd + gd; b.lddhv = zw;
    b.n_self_rows = (int32_t)p.n_t_rows;
    b.self_rows = RowMapB{c.meta.parent_row, p.split}; b.self_packed = RowMapB{c.meta.parent_row, p.split};
    b.ks = z + 2 * hd; b.ldks = zw; b.vs = z + 2 * hd + gd; b.ldvs = zw;
    b.hks = hpre + 2 * hd; b.ldhks = zw; b.hvs = hpre + 2 * hd + gd; b.ldhvs = zw;
    b.dhks = dh_ + 2 * hd; b.lddhks = zw; b.dhvs = dh_ + 2 * hd + gd; b.lddhvs = zw;
    b.hq = hpre + hd; b.ldhq = zw; b.dhq = dh_ + hd; b.lddhq = zw; b.dq_scale = 1.0f / std::sqrt((float)dh);
    TimedLaunch tl(MTFM_K_BWD, s);
    TRY(launch_attn_bwd(b, p.n_key_tiles, s));
  }
  // ---- input projection and GLN1
  TRY(tn(s, L, ws, zw, D, R, dh_, zw, identity_map(), R, xt, D, identity_map(), R, gr->w_uqkv, 0));
  TRY(transpose(s, w->w_uqkv, zw, nullptr, 0, nullptr, 0, D, w1t, zw));
  {
    GemmArgs gx{};
    gx.M = R; gx.N = D; gx.K = zw; gx.groups = 1;
    gx.A = dh_; gx.lda = zw; gx.amap = identity_map();
    gx.B[0] = w1t; gx.bn[0] = D; gx.ldb = zw;
    gx.cmap = identity_map(); gx.epi = EPI_STORE_F32; gx.out = dxt; gx.ldo = D;
    TimedLaunch tl(MTFM_K_BWD, s);
    TRY(launch_gemm(gx, MTFM_BF16, s));
  }
  {
    Gln1BwdArgs b{};
    b.rows = R; b.D = D; b.x = (const bf16*)x_in; b.ldx = D; b.gamma = w->ln1_g; b.type = c.meta.type;
    b.eps = d->ln_eps; b.dxt = dxt; b.lddxt = D; b.dres = (const bf16*)dy; b.lddres = D;
    b.dx = (bf16*)dx; b.lddx = D; b.pg = pg;
    TimedLaunch tl(MTFM_K_BWD, s);
    TRY(launch_gln1_bwd(b, s));
    TRY(launch_param_reduce(pg, gln_bwd_grid(R), D, gr->ln1_g, gr->ln1_b, s));
  }
  return MTFM_OK;
}

// ---------------------------------------------------------------------------
mtfm_status run_target_bwd(const Ctx& c, const mtfm_dims* d, const mtfm_target_w* w, const void* x_in,
                           const void* dy, void* dx, const mtfm_target_grad* gr, char* ws, const FwdKeep* keep) {
  TRY(check_bwd_dims(d));
  const MetaPlan& p = c.plan;
  const hipStream_t s = c.s;
  const int H = d->n_q_heads, G = d->n_kv_heads, dh = d->head_dim, D = d->d_model;
  const int hd = H * dh, gd = G * dh, zw = 2 * hd + 2 * gd;
  const int R = (int)p.n_rows, T = (int)p.n_t_rows, P = (int)p.n_parents, C = (int)p.n_ctx_rows, S = p.split;
  const BwdWs L = bwd_layout(p, d, MTFM_OP_TARGET_BWD);
  if (keep && p.n_t_rows == 0) keep = nullptr;   // the forward kept nothing for a layer without T rows
  bf16* xt = (bf16*)(keep ? keep->xt : ws + L.xt);
  bf16* zt = (bf16*)(keep ? keep->z : ws + L.z);
  bf16* ztpre = (bf16*)(keep ? keep->hpre : ws + L.hpre);
  bf16* kv = (bf16*)(keep ? keep->kv : ws + L.kv);
  bf16* kvpre = (bf16*)(keep ? keep->kvpre : ws + L.kvpre);
  bf16* a = (bf16*)(keep ? keep->a : ws + L.a);
  bf16* y = (bf16*)(ws + L.y);
  bf16* wot = (bf16*)(ws + L.wot);
  bf16* wtk = (bf16*)(ws + L.w1t);   // [S][D][zw]: transposed [W_u; W_q[k]; W_kv]
  bf16* wkvt = (bf16*)(ws + L.wkvt);
  float* dyv = (float*)(ws + L.dyv);
  bf16* dan = (bf16*)(ws + L.dan);
  bf16* dan_lo = (bf16*)(ws + L.dan_lo);
  float* dq = (float*)(ws + L.dq);
  bf16* dht = (bf16*)(ws + L.dh);
  bf16* dhkv = (bf16*)(ws + L.dhkv);
  float* dxt = (float*)(ws + L.dxt);
  float* pg = (float*)(ws + L.pg);
  const RowMap t_rows = list_map(c.meta.parent_row, S);     // T row t -> packed row
  const RowMap ctx_rows = list_map(c.meta.ctx_rows);
  if (R == 0) return MTFM_OK;

  // ---- forward recompute, unless the forward pass kept it
  if (!keep) {
    GlnArgs g1{};
    g1.rows = R; g1.D = D; g1.x = x_in; g1.ldx = D; g1.y = xt; g1.ldy = D;
    g1.gamma = w->ln1_g; g1.beta = w->ln1_b; g1.type = c.meta.type; g1.eps = d->ln_eps;
    TRY(timed_gln(g1, MTFM_BF16, s));
  }
  if (C > 0 && !keep) {
    // K, V (and their pre-activations) of every packed row, V also transposed
    GemmArgs gk{};
    gk.M = R; gk.N = 2 * gd; gk.K = D; gk.groups = 1;
    gk.A = xt; gk.lda = D; gk.amap = identity_map();
    gk.B[0] = w->w_kv; gk.bn[0] = 2 * gd; gk.ldb = D;
    gk.cmap = identity_map(); gk.epi = EPI_SILU_SPLIT;
    gk.dst[0] = kv; gk.ld[0] = 2 * gd; gk.cend[0] = 2 * gd; gk.scale[0] = 1.f;
    gk.cend[1] = gk.cend[2] = gk.cend[3] = 2 * gd;
    gk.pre = kvpre; gk.ldpre = 2 * gd;
    gk.vt = ws + L.vt; gk.ldvt = L.ldvt; gk.vt_col0 = gd; gk.vt_cols = gd;
    TRY(timed_gemm(MTFM_K_GEMM_KV, gk, MTFM_BF16, s));
  }
  if (T > 0 && !keep) {
    GemmArgs gt{};
    gt.M = P; gt.N = zw; gt.K = D; gt.groups = S;
    gt.A = xt; gt.lda = D; gt.amap = list_map(c.meta.parent_row); gt.amap_zadd = 1; gt.a_rows = c.plan.n_rows;
    gt.B[0] = w->w_u; gt.bn[0] = hd;
    gt.B[1] = w->w_q; gt.bn[1] = hd; gt.bz[1] = (int64_t)hd * D;
    gt.B[2] = w->w_kv; gt.bn[2] = 2 * gd;
    gt.ldb = D;
    gt.cmap = RowMap{nullptr, S, 0, 0}; gt.cmap_zadd = 1;
    gt.epi = EPI_SILU_SPLIT;
    gt.dst[0] = zt; gt.ld[0] = zw; gt.cend[0] = hd; gt.scale[0] = 1.f;
    gt.dst[1] = zt + hd; gt.ld[1] = zw; gt.cend[1] = 2 * hd; gt.scale[1] = q_scale(dh);
    gt.dst[2] = zt + 2 * hd; gt.ld[2] = zw; gt.cend[2] = zw; gt.scale[2] = 1.f;
    gt.cend[3] = zw;
    gt.pre = ztpre; gt.ldpre = zw;
    TRY(timed_gemm(MTFM_K_GEMM_T, gt, MTFM_BF16, s));
    {
      AttnArgs aa{};
      aa.q = zt + hd; aa.ldq = zw; aa.k = kv; aa.ldk = 2 * gd; aa.v = kv + gd; aa.ldv = 2 * gd;
      aa.vt = ws + L.vt; aa.ldvt = L.ldvt; aa.n_key_rows = R; aa.max_user_rows = p.max_user_rows;
      aa.kd = zt + 2 * hd; aa.ldkd = zw; aa.vd = zt + 2 * hd + gd; aa.ldvd = zw;
      aa.a = a; aa.lda = hd;
      aa.tiles = c.meta.target_tiles; aa.ntiles = (int32_t)p.n_target_tiles;
      aa.order = c.meta.target_order; aa.n_order = (int32_t)p.n_target_order;
      aa.p = c.meta.p; aa.n = c.meta.n; aa.lens = c.b->lens_d;
      aa.H = H; aa.G = G; aa.dh = dh; aa.out_scale = kLn2;
      TRY(timed_attention(MTFM_K_ATTN_TARGET, aa, MTFM_BF16, s));
    }
  }
  if (T > 0) {
    GlnArgs g2{};
    g2.rows = T; g2.D = hd; g2.x = a; g2.ldx = hd; g2.y = y; g2.ldy = hd; g2.gate = zt; g2.ldg = zw;
    g2.gamma = w->ln2_g; g2.beta = w->ln2_b; g2.type = nullptr; g2.type_const = TT_T; g2.eps = d->ln_eps;
    TRY(timed_gln(g2, MTFM_BF16, s));
  }

  // ---- output projection (T rows only; H/R rows pass dY through unchanged)
  if (T > 0) {
    TRY(tn(s, L, ws, D, hd, T, dy, D, t_rows, R, y, hd, identity_map(), T, gr->w_o, 0));
    TRY(transpose(s, w->w_o, D, nullptr, 0, nullptr, 0, hd, wot, D));
    GemmArgs gd_{};
    gd_.M = T; gd_.N = hd; gd_.K = D; gd_.groups = 1;
    gd_.A = dy; gd_.lda = D; gd_.amap = t_rows; gd_.a_rows = c.plan.n_rows;
    gd_.B[0] = wot; gd_.bn[0] = hd; gd_.ldb = D;
    gd_.cmap = identity_map(); gd_.epi = EPI_STORE_F32; gd_.out = dyv; gd_.ldo = hd;
    {
      TimedLaunch tl(MTFM_K_BWD, s);
      TRY(launch_gemm(gd_, MTFM_BF16, s));
    }
    Gln2BwdArgs b{};
    b.rows = T; b.D = hd; b.a = a; b.lda = hd; b.gamma = w->ln2_g; b.beta = w->ln2_b;
    b.type = nullptr; b.type_const = TT_T; b.nmap = RowMapB{c.meta.parent_row, S}; b.n = c.meta.n;
    b.eps = d->ln_eps;
    b.u = zt; b.ldu = zw; b.hu = ztpre; b.ldhu = zw; b.dy = dyv; b.lddy = hd;
    b.dhu = dht; b.lddhu = zw; b.dan = dan; b.dan_lo = dan_lo; b.lddan = hd; b.pg = pg;
    {
      TimedLaunch tl(MTFM_K_BWD, s);
      TRY(launch_gln2_bwd(b, s));
    }
    TRY(launch_param_reduce(pg, gln_bwd_grid(T), hd, gr->ln2_g, gr->ln2_b, s));
  } else {
    hipError_t e = hipMemsetAsync(gr->w_o, 0, (size_t)D * hd * 4, s);
    if (e == hipSuccess) e = hipMemsetAsync(gr->ln2_g, 0, (size_t)3 * hd * 4, s);
    if (e == hipSuccess) e = hipMemsetAsync(gr->ln2_b, 0, (size_t)3 * hd * 4, s);
    if (e != hipSuccess) return hip_fail(e, "hipMemsetAsync");
  }

  // ---- attention backward
  if (T > 0) {
    AttnBwdArgs b{};
    b.q = zt + hd; b.ldq = zw; b.k = kv; b.ldk = 2 * gd; b.v = kv + gd; b.ldv = 2 * gd;
    b.dan = dan; b.dan_lo = dan_lo; b.lddan = hd;
    b.qtiles = c.meta.target_tiles; b.nqtiles = (int32_t)p.n_target_tiles;
    b.user = c.meta.user; b.n_users = p.n_users; b.query_tiles_row = UT_TTILE;
    b.p = c.meta.p; b.n = c.meta.n; b.lens = c.b->lens_d; b.H = H; b.G = G;
    b.dq = dq;
    b.hk = kvpre; b.ldhk = 2 * gd; b.hv = kvpre + gd; b.ldhv = 2 * gd;
    b.dhk = dhkv; b.lddhk = 2 * gd; b.dhv = dhkv + gd; b.lddhv = 2 * gd;
    b.n_self_rows = T;
    b.self_rows = RowMapB{nullptr, 1}; b.self_packed = RowMapB{c.meta.parent_row, S};
    b.ks = zt + 2 * hd; b.ldks = zw; b.vs = zt + 2 * hd + gd; b.ldvs = zw;
    b.hks = ztpre + 2 * hd; b.ldhks = zw; b.hvs = ztpre + 2 * hd + gd; b.ldhvs = zw;
    b.dhks = dht + 2 * hd; b.lddhks = zw; b.dhvs = dht + 2 * hd + gd; b.lddhvs = zw;
    b.hq = ztpre + hd; b.ldhq = zw; b.dhq = dht + hd; b.lddhq = zw; b.dq_scale = 1.0f / std::sqrt((float)dh);
    {
      TimedLaunch tl(MTFM_K_BWD, s);
      TRY(launch_attn_bwd(b, p.n_key_tiles, s));
    }
  }

  // ---- weight gradients of the input projections
  if (T > 0) {
    TRY(tn(s, L, ws, hd, D, T, dht, zw, identity_map(), T, xt, D, t_rows, R, gr->w_u, 0));
    // W_q[k]: rows of sub-token k, T row S*m + k, packed row parent_row[m] + k
    TRY(tn(s, L, ws, hd, D, P, dht + hd, zw, RowMap{nullptr, S, 0, 0}, T, xt, D, list_map(c.meta.parent_row), R, gr->w_q, 0,
           S, 1, 1, (int64_t)hd * D));
  } else {
    hipError_t e = hipMemsetAsync(gr->w_u, 0, (size_t)hd * D * 4, s);
    if (e == hipSuccess) e = hipMemsetAsync(gr->w_q, 0, (size_t)S * hd * D * 4, s);
    if (e != hipSuccess) return hip_fail(e, "hipMemsetAsync");
  }
  if (C > 0) TRY(tn(s, L, ws, 2 * gd, D, C, dhkv, 2 * gd, ctx_rows, R, xt, D, ctx_rows, R, gr->w_kv, 0));
  if (T > 0) TRY(tn(s, L, ws, 2 * gd, D, T, dht + 2 * hd, zw, identity_map(), T, xt, D, t_rows, R, gr->w_kv, C > 0 ? 1 : 0));
  if (C == 0 && T == 0) {
    hipError_t e = hipMemsetAsync(gr->w_kv, 0, (size_t)2 * gd * D * 4, s);
    if (e != hipSuccess) return hip_fail(e, "hipMemsetAsync");
  }

  // ---- dX~ = dH W on every row (context rows through K|V only; every row is
  // either a context row or a T row, so the two products cover dX~)
  if (C > 0) {
    TRY(transpose(s, w->w_kv, 2 * gd, nullptr, 0, nullptr, 0, D, wkvt, 2 * gd));
    GemmArgs gx{};
    gx.M = C; gx.N = D; gx.K = 2 * gd; gx.groups = 1;
    gx.A = dhkv; gx.lda = 2 * gd; gx.amap = ctx_rows; gx.a_rows = c.plan.n_rows;
    gx.B[0] = wkvt; gx.bn[0] = D; gx.ldb = 2 * gd;
    gx.cmap = ctx_rows; gx.epi = EPI_STORE_F32; gx.out = dxt; gx.ldo = D;
    TimedLaunch tl(MTFM_K_BWD, s);
    TRY(launch_gemm(gx, MTFM_BF16, s));
  }
  if (T > 0) {
    for (int k = 0; k < S; ++k)
      TRY(transpose(s, w->w_u, hd, (const bf16*)w->w_q + (int64_t)k * hd * D, hd, w->w_kv, 2 * gd, D,
                    wtk + (int64_t)k * D * zw, zw));
    GemmArgs gx{};
    gx.M = P; gx.N = D; gx.K = zw; gx.groups = S;
    gx.A = dht; gx.lda = zw; gx.amap = RowMap{nullptr, S, 0, 0}; gx.amap_zadd = 1;
    gx.B[0] = wtk; gx.bn[0] = D; gx.bz[0] = (int64_t)D * zw; gx.ldb = zw;
    gx.cmap = list_map(c.meta.parent_row); gx.cmap_zadd = 1;
    gx.epi = EPI_STORE_F32; gx.out = dxt; gx.ldo = D;
    TimedLaunch tl(MTFM_K_BWD, s);
    TRY(launch_gemm(gx, MTFM_BF16, s));
  }
  {
    Gln1BwdArgs b{};
    b.rows = R; b.D = D; b.x = (const bf16*)x_in; b.ldx = D; b.gamma = w->ln1_g; b.type = c.meta.type;
    b.eps = d->ln_eps; b.dxt = dxt; b.lddxt = D; b.dres = (const bf16*)dy; b.lddres = D;
    b.dx = (bf16*)dx; b.lddx = D; b.pg = pg;
    TimedLaunch tl(MTFM_K_BWD, s);
    TRY(launch_gln1_bwd(b, s));
    TRY(launch_param_reduce(pg, gln_bwd_grid(R), D, gr->ln1_g, gr->ln1_b, s));
  }
  return MTFM_OK;
}
