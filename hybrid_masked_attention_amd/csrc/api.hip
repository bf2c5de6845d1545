// C ABI of libmtfm: argument validation, metadata and workspace layout, and
// the launch sequences of the full-attention layer, the target-attention
// layer and the hybrid backbone.  Host code only; kernels live in the other
// translation units.  No entry point allocates, synchronises or reads device
// memory back.

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <initializer_list>
#include <string>
#include <vector>

#include "api_internal.h"
#include "v2.h"

thread_local std::string g_last_error;

void set_last_error(const char* msg) { g_last_error = msg; }

mtfm_status hip_fail(hipError_t e, const char* where) {
  g_last_error = std::string(where) + ": " + hipGetErrorString(e);
  return MTFM_E_HIP;
}

int64_t align_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

// ---------------------------------------------------------------------------
// Metadata plan: totals from the host lengths, array offsets in the buffer.

// Entries of a layer's attention work order: 8 x the longest XCD list, from
// the same ranking and dealing the device performs (users by estimated work,
// descending, ties by index; rank r goes to XCD order_xcd(r)).  0 (no order:
// the kernels keep the XCD-contiguous one, which splits a long user over
// several XCDs) when the dealing would load some XCD with more than 1.25 x
// the mean work, as with a few users or one user far longer than the rest.
static int64_t order_entries(const int32_t* lens, int n_users, int split, int layer) {
  if (n_users <= 0 || n_users > kOrderMaxUsers) return 0;
  std::vector<int64_t> work(n_users);
  std::vector<int32_t> idx(n_users);
  for (int u = 0; u < n_users; ++u) {
    work[u] = order_user_work(lens, u, split, layer);
    idx[u] = u;
  }
  std::sort(idx.begin(), idx.end(), [&](int32_t a, int32_t b) { return work[a] != work[b] ? work[a] > work[b] : a < b; });
  int64_t count[8] = {}, load[8] = {}, total = 0;
  for (int r = 0; r < n_users; ++r) {
    count[order_xcd(r)] += order_slices(lens, idx[r], split, layer);
    load[order_xcd(r)] += work[idx[r]];
    total += work[idx[r]];
  }
  if (4 * 8 * *std::max_element(load, load + 8) > 5 * total) return 0;
  return 8 * *std::max_element(count, count + 8);
}
mtfm_status plan_meta(const mtfm_batch* b, MetaPlan* plan) {
  if (!b || !plan) return MTFM_E_NULL;
  if (b->n_users < 0) return MTFM_E_DIMS;
  if (b->split != 1 && b->split != 4) return MTFM_E_DIMS;
  if (b->n_users > 0 && !b->lens_h) return MTFM_E_NULL;
  MetaPlan p;
  p.n_users = b->n_users;
  p.split = b->split;
  for (int u = 0; u < b->n_users; ++u) {
    const int64_t lh = b->lens_h[3 * u], lr = b->lens_h[3 * u + 1], lt = b->lens_h[3 * u + 2];
    if (lh < 0 || lr < 0 || lt < 0) return MTFM_E_DIMS;
    const int64_t rows = lh + lr + b->split * lt;
    p.n_rows += rows;
    p.n_t_rows += b->split * lt;
    p.n_parents += lt;
    p.n_ctx_rows += lh + lr;
    p.n_full_tiles += (rows + kTile - 1) / kTile;
    p.n_target_tiles += (b->split * lt + kTile - 1) / kTile;
    p.n_key_tiles += (lh + lr + kTile - 1) / kTile;
    p.max_user_rows = (int32_t)std::min<int64_t>(std::max<int64_t>(p.max_user_rows, rows), INT32_MAX);
    p.max_t_rows = (int32_t)std::min<int64_t>(std::max<int64_t>(p.max_t_rows, b->split * lt), INT32_MAX);
    p.max_ctx_rows = (int32_t)std::min<int64_t>(std::max<int64_t>(p.max_ctx_rows, lh + lr), INT32_MAX);
    if (p.n_rows > INT32_MAX - 4096) return MTFM_E_DIMS;
  }
  p.n_full_order = order_entries(b->lens_h, b->n_users, b->split, OL_FULL);
  p.n_target_order = order_entries(b->lens_h, b->n_users, b->split, OL_TARGET);
  mtfm_meta_layout& l = p.lay;
  l.n_rows = p.n_rows; l.n_t_rows = p.n_t_rows; l.n_parents = p.n_parents; l.n_ctx_rows = p.n_ctx_rows;
  l.n_full_tiles = p.n_full_tiles; l.n_target_tiles = p.n_target_tiles; l.n_key_tiles = p.n_key_tiles;
  int64_t off = 0;
  auto take = [&](int64_t bytes) { int64_t o = off; off = align_up(off + bytes, 256); return o; };
  l.off_user = take((int64_t)UT_COUNT * (p.n_users + 1) * 4);
  l.off_p = take(p.n_rows * 4);
  l.off_n = take(p.n_rows * 4);
  l.off_type = take(p.n_rows);
  l.off_full_tiles = take(p.n_full_tiles * 32);
  l.off_target_tiles = take(p.n_target_tiles * 32);
  l.off_ctx_rows = take(p.n_ctx_rows * 4);
  l.off_parent_row = take(p.n_parents * 4);
  l.n_full_order = p.n_full_order; l.n_target_order = p.n_target_order;
  l.off_full_order = take(p.n_full_order * 4);
  l.off_target_order = take(p.n_target_order * 4);
  l.off_tsort_q = take(p.n_t_rows * 4);
  l.off_tsort_g = take(p.n_t_rows * 4);
  l.off_target_tiles_sorted = take(p.n_target_tiles * 32);
  l.total_bytes = off;
  *plan = p;
  return MTFM_OK;
}

MetaPtrs meta_ptrs(const MetaPlan& plan, const void* meta_d) {
  const char* base = static_cast<const char*>(meta_d);
  MetaPtrs m;
  m.user = reinterpret_cast<const int32_t*>(base + plan.lay.off_user);
  m.p = reinterpret_cast<const int32_t*>(base + plan.lay.off_p);
  m.n = reinterpret_cast<const int32_t*>(base + plan.lay.off_n);
  m.type = reinterpret_cast<const uint8_t*>(base + plan.lay.off_type);
  m.full_tiles = reinterpret_cast<const int32_t*>(base + plan.lay.off_full_tiles);
  m.target_tiles = reinterpret_cast<const int32_t*>(base + plan.lay.off_target_tiles);
  m.ctx_rows = reinterpret_cast<const int32_t*>(base + plan.lay.off_ctx_rows);
  m.parent_row = reinterpret_cast<const int32_t*>(base + plan.lay.off_parent_row);
  m.full_order = plan.n_full_order ? reinterpret_cast<const int32_t*>(base + plan.lay.off_full_order) : nullptr;
  m.target_order = plan.n_target_order ? reinterpret_cast<const int32_t*>(base + plan.lay.off_target_order) : nullptr;
  m.tsort_q = reinterpret_cast<const int32_t*>(base + plan.lay.off_tsort_q);
  m.tsort_g = reinterpret_cast<const int32_t*>(base + plan.lay.off_tsort_g);
  m.target_tiles_sorted = reinterpret_cast<const int32_t*>(base + plan.lay.off_target_tiles_sorted);
  return m;
}

mtfm_status check_dims(const mtfm_dims* d) {
  if (!d) return MTFM_E_NULL;
  if (d->d_model <= 0 || d->n_q_heads <= 0 || d->n_kv_heads <= 0 || d->head_dim <= 0) return MTFM_E_DIMS;
  if (!(d->ln_eps > 0.f) || !std::isfinite(d->ln_eps)) return MTFM_E_DIMS;
  if (d->dtype != MTFM_F32 && d->dtype != MTFM_BF16) return MTFM_E_UNSUPPORTED;
  if (d->n_q_heads % d->n_kv_heads != 0) return MTFM_E_UNSUPPORTED;
  const int hd = d->n_q_heads * d->head_dim;
  if (d->dtype == MTFM_BF16) {
    if (d->head_dim != 64) return MTFM_E_UNSUPPORTED;
    const int r = d->n_q_heads / d->n_kv_heads;
    if (r != 1 && r != 2 && r != 4 && r != 8) return MTFM_E_UNSUPPORTED;
  } else {
    if (d->head_dim != 32 && d->head_dim != 64) return MTFM_E_UNSUPPORTED;
  }
  // row kernels hold a row in one wave as 1, 2, 4, 8 or 16 values per lane
  auto row_width_ok = [](int w) { return w == 64 || w == 128 || w == 256 || w == 512 || w == 1024; };
  if (!row_width_ok(d->d_model) || !row_width_ok(hd)) return MTFM_E_UNSUPPORTED;
  return MTFM_OK;
}

// Workspace layout of one forward layer (byte offsets, 256-B aligned).
LayerWs layer_ws(const MetaPlan& p, const mtfm_dims* d, int op) {
  const int64_t es = elem_size(d->dtype);
  const int64_t hd = (int64_t)d->n_q_heads * d->head_dim, gd = (int64_t)d->n_kv_heads * d->head_dim;
  const int64_t zw = 2 * hd + 2 * gd;
  LayerWs w;
  int64_t off = 0;
  auto take = [&](int64_t bytes) { int64_t o = off; off = align_up(off + std::max<int64_t>(bytes, 0), 256); return o; };
  w.xt = take(p.n_rows * d->d_model * es);
  if (d->dtype == MTFM_BF16) {
    w.ldvt = vt_ld(p.n_rows);
    w.vt = take(gd * w.ldvt * es);
  }
  if (op == MTFM_OP_FULL) {
    w.z = take(p.n_rows * zw * es);
    w.a = take(p.n_rows * hd * es);
    w.y = take(p.n_rows * hd * es);
  } else {
    w.kv = take(p.n_rows * 2 * gd * es);
    w.z = take(p.n_t_rows * zw * es);
    w.a = take(p.n_t_rows * hd * es);
    w.y = take(p.n_t_rows * hd * es);
  }
  w.total = off;
  return w;
}

// Key splits of the per-group target attention on the inference paths.  Its
// grid is (32-row T slice, KV group): with few T rows against long contexts
// (a request of one user with a long history) it fills few of the ~1,024
// workgroup slots (256 CUs x 4) while each workgroup walks a whole context.
// A is a plain sum over keys divided by n, so a slice's key tiles can be
// split over ks workgroups whose fp32 partials the gated LayerNorm adds.  ks
// fills the slots, leaves each run at least 8 key tiles of the longest
// context, and stays at most 16 with the partials within 16 MiB (1: none).
static int target_key_splits(const MetaPlan& p, const mtfm_dims* d) {
  if (d->dtype != MTFM_BF16 || p.n_t_rows == 0) return 1;
  const int64_t wgs = std::max<int64_t>(2 * p.n_target_tiles * d->n_kv_heads, 1);
  const int64_t part = std::max<int64_t>(p.n_t_rows * (int64_t)d->n_q_heads * d->head_dim * 4, 1);
  const int64_t ks = std::min<int64_t>({1024 / wgs, ((int64_t)p.max_ctx_rows + 63) / 64 / 8, 16, ((int64_t)16 << 20) / part});
  return ks >= 2 ? (int)ks : 1;
}

// Workspace of the backbone with the target layers' context stage hoisted
// (bf16): the full layer's workspace, then per target layer of a block its
// normalised rows X~ [R][d], K [R][G*dh] and V^T [G*dh][ldvt], then the T-row
// buffers shared by the target layers (with key splits, the fp32 partials of A).
struct BackboneWs {
  int64_t full = 0;
  int64_t xt[4] = {}, k[4] = {}, vt[4] = {};
  int64_t xtt = 0, zt = 0, a = 0, y = 0, apart = 0;
  int32_t ksplit = 1;
  int64_t ldvt = 0, total = 0;
};

BackboneWs backbone_ws(const MetaPlan& p, const mtfm_dims* d, int k_target) {
  const int64_t es = elem_size(d->dtype);
  const int64_t hd = (int64_t)d->n_q_heads * d->head_dim, gd = (int64_t)d->n_kv_heads * d->head_dim;
  const int64_t zw = 2 * hd + 2 * gd;
  BackboneWs w;
  int64_t off = 0;
  auto take = [&](int64_t bytes) { int64_t o = off; off = align_up(off + std::max<int64_t>(bytes, 0), 256); return o; };
  w.full = take(layer_ws(p, d, MTFM_OP_FULL).total);
  w.ldvt = vt_ld(p.n_rows);
  // each kind for the k layers back to back (one grouped projection writes them)
  const int64_t xt0 = take(k_target * p.n_rows * d->d_model * es);
  const int64_t k0 = take(k_target * p.n_rows * gd * es);
  const int64_t vt0 = take(k_target * gd * w.ldvt * es);
  for (int l = 0; l < k_target; ++l) {
    w.xt[l] = xt0 + l * p.n_rows * d->d_model * es;
    w.k[l] = k0 + l * p.n_rows * gd * es;
    w.vt[l] = vt0 + l * gd * w.ldvt * es;
  }
  w.xtt = take(p.n_t_rows * d->d_model * es);
  w.zt = take(p.n_t_rows * zw * es);
  w.a = take(p.n_t_rows * hd * es);
  w.y = take(p.n_t_rows * hd * es);
  w.ksplit = target_key_splits(p, d);
  w.apart = take(w.ksplit > 1 ? w.ksplit * p.n_t_rows * hd * 4 : 0);
  w.total = off;
  return w;
}

namespace {

mtfm_status check_batch_device(const mtfm_batch* b, const MetaPlan& p) {
  if (p.n_users > 0 && !b->lens_d) return MTFM_E_NULL;
  int64_t n_act = 0;
  for (int u = 0; u < p.n_users; ++u) n_act += b->lens_h[3 * u + 1];
  if (n_act > 0 && !b->ts_r_d) return MTFM_E_NULL;
  if (p.n_parents > 0 && !b->ts_t_d) return MTFM_E_NULL;
  return MTFM_OK;
}

// Packed 2:4 projections are read by the bf16 forward only and must be
// 16-byte aligned; fwd_dims = nullptr (backward) skips the check, the
// backward ignores them.
mtfm_status check_packed(const mtfm_dims* fwd_dims, std::initializer_list<const void*> packed) {
  if (!fwd_dims) return MTFM_OK;
  for (const void* p : packed)
    if (p && (fwd_dims->dtype != MTFM_BF16 || ((uintptr_t)p & 15) != 0)) return MTFM_E_UNSUPPORTED;
  return MTFM_OK;
}

mtfm_status check_full_w(const mtfm_full_w* w, const mtfm_dims* fwd_dims = nullptr) {
  if (!w || !w->ln1_g || !w->ln1_b || !w->w_uqkv || !w->ln2_g || !w->ln2_b || !w->w_o) return MTFM_E_NULL;
  return check_packed(fwd_dims, {w->w_uqkv_s24, w->w_o_s24});
}

mtfm_status check_target_w(const mtfm_target_w* w, const mtfm_dims* fwd_dims = nullptr) {
  if (!w || !w->ln1_g || !w->ln1_b || !w->w_u || !w->w_q || !w->w_kv || !w->ln2_g || !w->ln2_b || !w->w_o)
    return MTFM_E_NULL;
  return check_packed(fwd_dims, {w->w_t_s24, w->w_kv_s24, w->w_o_s24});
}

}  // namespace

mtfm_status prepare(const mtfm_batch* b, const mtfm_dims* d, const void* meta_d, const void* x0, const void* x1,
                    void* ws, size_t ws_bytes, int op, Ctx* c, void* stream) {
  TRY(plan_meta(b, &c->plan));
  TRY(check_dims(d));
  if (!meta_d || !x0 || !x1) return MTFM_E_NULL;
  TRY(check_batch_device(b, c->plan));
  const size_t need = mtfm_workspace_bytes(b, d, op);
  if (need > 0 && !ws) return MTFM_E_NULL;
  if (ws_bytes < need) return MTFM_E_WORKSPACE;
  c->b = b;
  c->meta = meta_ptrs(c->plan, meta_d);
  c->s = (hipStream_t)stream;
  return MTFM_OK;
}

// Fused epilogue of the bf16 attention (the gated group LayerNorm, written as
// Y); A itself only where something reads it afterwards.
static void fuse_gated_gln(AttnArgs& aa, const Ctx& c, const mtfm_dims* d, const float* g2, const float* b2,
                           const void* u, int64_t ldu, void* y, int64_t ldy, void* a_keep) {
  aa.y = y; aa.ldy = ldy;
  aa.u = u; aa.ldu = ldu;
  aa.ln_g = g2; aa.ln_b = b2;
  aa.type = c.meta.type; aa.eps = d->ln_eps;
  aa.a = (c.write_a || a_keep) ? aa.a : nullptr;
}

// Gated group LayerNorm of the T rows after the target attention (their A,
// T-row order): the target layer's query rows are too few to fill the GPU
// with one workgroup per 32 rows and every head, so its attention runs one
// workgroup per KV group and the normalisation, which needs every head of a
// row, follows as a pass over the T rows alone.
static mtfm_status target_gated_gln(const Ctx& c, const mtfm_dims* d, const float* g2, const float* b2,
                                    const void* a, const void* u, int64_t ldu, void* y, int dt,
                                    const float* parts = nullptr, int n_parts = 0, bool temporal = false) {
  const int hd = d->n_q_heads * d->head_dim;
  GlnArgs g{};
  g.rows = (int32_t)c.plan.n_t_rows; g.D = hd; g.x = a; g.ldx = hd; g.y = y; g.ldy = hd;
  g.x_parts = parts; g.n_parts = n_parts; g.part_stride = c.plan.n_t_rows * hd;
  g.gate = u; g.ldg = ldu;
  g.gamma = g2; g.beta = b2; g.type = nullptr; g.type_const = TT_T; g.eps = d->ln_eps;
  g.temporal = temporal ? 1 : 0;
  return timed_gln(g, dt, c.s, MTFM_K_GLN_T);
}

// ---------------------------------------------------------------------------
// Full-attention layer ([explainer] §4.1):
//   X~ = GLN1(X); [U|Q|K|V] = SiLU(X~ W^T); A = masked SiLU attention / n;
//   X' = (GLN2(A) (.) U) W_o^T + X
mtfm_status run_full(const Ctx& c, const mtfm_dims* d, const mtfm_full_w* w, const void* x_in, void* x_out,
                     char* ws, const KvOut* kv, const FwdKeep* keep) {
  const MetaPlan& p = c.plan;
  const int dt = d->dtype;
  const int64_t es = elem_size(dt);
  const int H = d->n_q_heads, G = d->n_kv_heads, dh = d->head_dim, D = d->d_model;
  const int hd = H * dh, gd = G * dh, zw = 2 * hd + 2 * gd;
  const LayerWs L = layer_ws(p, d, MTFM_OP_FULL);
  char* xt = keep ? keep->xt : ws + L.xt;
  char* z = keep ? keep->z : ws + L.z;
  char* a = keep ? keep->a : ws + L.a;
  char* y = ws + L.y;
  if (p.n_rows == 0) return MTFM_OK;

  GlnArgs g1{};
  g1.rows = (int32_t)p.n_rows; g1.D = D; g1.x = x_in; g1.ldx = D; g1.y = xt; g1.ldy = D;
  g1.gamma = w->ln1_g; g1.beta = w->ln1_b; g1.type = c.meta.type; g1.eps = d->ln_eps;
  TRY(timed_gln(g1, dt, c.s));

  GemmArgs gp{};
  gp.M = (int32_t)p.n_rows; gp.N = zw; gp.K = D; gp.groups = 1;
  gp.A = xt; gp.lda = D; gp.amap = identity_map();
  gp.B[0] = w->w_uqkv; gp.bn[0] = zw; gp.ldb = D;
  gp.bs24 = w->w_uqkv_s24; gp.bs24_rows = zw;
  gp.cmap = identity_map();
  gp.epi = EPI_SILU_SPLIT;
  gp.dst[0] = z; gp.ld[0] = zw; gp.cend[0] = hd; gp.scale[0] = 1.f;
  gp.dst[1] = z + hd * es; gp.ld[1] = zw; gp.cend[1] = 2 * hd; gp.scale[1] = q_scale(dh);
  gp.dst[2] = z + 2 * hd * es; gp.ld[2] = zw; gp.cend[2] = zw; gp.scale[2] = 1.f;
  gp.cend[3] = zw;
  if (dt == MTFM_BF16) { gp.vt = ws + L.vt; gp.ldvt = L.ldvt; gp.vt_col0 = 2 * hd + gd; gp.vt_cols = gd; }
  if (keep) { gp.pre = keep->hpre; gp.ldpre = zw; }
  if (dt == MTFM_BF16 && !keep) {
    // the attention reads K row-major for every key row but V row-major only
    // for the T rows' own value (the keys' values come from V^T): the V
    // segment is stored for T rows only (the backward keeps all of it)
    gp.cend[2] = 2 * hd + gd;
    gp.dst[3] = z + (2 * hd + gd) * es; gp.ld[3] = zw; gp.cend[3] = zw; gp.scale[3] = 1.f;
    gp.seg3_type = c.meta.type;
  }
  if (kv) {
    // K straight into the cache ([rows][gd]), V only transposed (bf16 path; no T rows, so
    // no query reads its own row-major K/V)
    gp.dst[2] = kv->k; gp.ld[2] = gd; gp.cend[2] = 2 * hd + gd;
    gp.dst[3] = nullptr; gp.ld[3] = gd; gp.cend[3] = zw; gp.scale[3] = 1.f;
    gp.vt = kv->vt; gp.ldvt = kv->ldvt;
  }
  TRY(timed_gemm(MTFM_K_GEMM_UQKV, gp, dt, c.s));

  AttnArgs aa{};
  aa.q = z + hd * es; aa.ldq = zw;
  aa.k = z + 2 * hd * es; aa.ldk = zw;
  aa.v = z + (2 * hd + gd) * es; aa.ldv = zw;
  aa.vt = ws + L.vt; aa.ldvt = L.ldvt; aa.n_key_rows = (int32_t)p.n_rows; aa.max_user_rows = p.max_user_rows;
  aa.kd = aa.k; aa.ldkd = zw; aa.vd = aa.v; aa.ldvd = zw;
  if (kv) {
    aa.k = kv->k; aa.ldk = gd; aa.v = nullptr; aa.ldv = 0;
    aa.vt = kv->vt; aa.ldvt = kv->ldvt;
    aa.kd = kv->k; aa.ldkd = gd; aa.vd = kv->k; aa.ldvd = gd;
  }
  aa.a = a; aa.lda = hd;
  aa.tiles = c.meta.full_tiles; aa.ntiles = (int32_t)p.n_full_tiles;
  aa.order = c.meta.full_order; aa.n_order = (int32_t)p.n_full_order;
  aa.p = c.meta.p; aa.n = c.meta.n; aa.lens = c.b->lens_d;
  aa.H = H; aa.G = G; aa.dh = dh; aa.out_scale = kLn2;
  if (dt == MTFM_BF16) fuse_gated_gln(aa, c, d, w->ln2_g, w->ln2_b, z, zw, y, hd, keep ? keep->a : nullptr);
  TRY(timed_attention(MTFM_K_ATTN_FULL, aa, dt, c.s));

  if (dt != MTFM_BF16) {
    GlnArgs g2{};
    g2.rows = (int32_t)p.n_rows; g2.D = hd; g2.x = a; g2.ldx = hd; g2.y = y; g2.ldy = hd;
    g2.gate = z; g2.ldg = zw;
    g2.gamma = w->ln2_g; g2.beta = w->ln2_b; g2.type = c.meta.type; g2.eps = d->ln_eps;
    TRY(timed_gln(g2, dt, c.s));
  }

  GemmArgs go{};
  go.M = (int32_t)p.n_rows; go.N = D; go.K = hd; go.groups = 1;
  go.A = y; go.lda = hd; go.amap = identity_map();
  go.B[0] = w->w_o; go.bn[0] = D; go.ldb = hd;
  go.bs24 = w->w_o_s24; go.bs24_rows = D;
  go.cmap = identity_map();
  go.epi = EPI_RESID; go.resid = x_in; go.ldr = D; go.out = x_out; go.ldo = D;
  TRY(timed_gemm(MTFM_K_GEMM_OUT, go, dt, c.s));
  return MTFM_OK;
}

// ---------------------------------------------------------------------------
// Target-attention layer ([explainer] §4.2; V2 per-sub-token Q, [blog] §3.3.2):
//   X~ = GLN1(X) on all rows; [K|V] = SiLU(X~ W_kv^T) on H/R rows (a T row's
//   own K/V comes from its row GEMM below, it is the only T key it sees);
//   [U_T|Q_T|K_T|V_T] = SiLU(X~_T [W_u; W_q[k]; W_kv]^T) per sub-token k;
//   A_T = masked attention; X'_T = (GLN2(A_T) (.) U_T) W_o^T + X_T.
mtfm_status run_target(const Ctx& c, const mtfm_dims* d, const mtfm_target_w* w, const void* x_in, void* x_out,
                       char* ws, const FwdKeep* keep) {
  const MetaPlan& p = c.plan;
  const int dt = d->dtype;
  const int64_t es = elem_size(dt);
  const int H = d->n_q_heads, G = d->n_kv_heads, dh = d->head_dim, D = d->d_model;
  const int hd = H * dh, gd = G * dh, zw = 2 * hd + 2 * gd;
  const int S = p.split;
  const LayerWs L = layer_ws(p, d, MTFM_OP_TARGET);
  char* xt = keep ? keep->xt : ws + L.xt;
  char* kv = keep ? keep->kv : ws + L.kv;
  char* zt = keep ? keep->z : ws + L.z;
  char* a = keep ? keep->a : ws + L.a;
  char* y = ws + L.y;
  if (x_out != x_in && p.n_rows > 0) {
    hipError_t e = hipMemcpyAsync(x_out, x_in, (size_t)p.n_rows * D * es, hipMemcpyDeviceToDevice, c.s);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync");
  }
  if (p.n_t_rows == 0) return MTFM_OK;

  GlnArgs g1{};
  g1.rows = (int32_t)p.n_rows; g1.D = D; g1.x = x_in; g1.ldx = D; g1.y = xt; g1.ldy = D;
  g1.gamma = w->ln1_g; g1.beta = w->ln1_b; g1.type = c.meta.type; g1.eps = d->ln_eps;
  TRY(timed_gln(g1, dt, c.s, MTFM_K_GLN_T));

  if (p.n_ctx_rows > 0) {
    // K (row-major) and V of every packed row (the T rows' are unused): the
    // attention reads the context keys as whole 64-row tiles of packed rows,
    // V through its transposed copy (bf16)
    GemmArgs gk{};
    gk.M = (int32_t)p.n_rows; gk.N = 2 * gd; gk.K = D; gk.groups = 1;
    gk.A = xt; gk.lda = D; gk.amap = identity_map();
    gk.B[0] = w->w_kv; gk.bn[0] = 2 * gd; gk.ldb = D;
    gk.bs24 = w->w_kv_s24; gk.bs24_rows = 2 * gd;
    gk.cmap = identity_map();
    gk.epi = EPI_SILU_SPLIT;
    gk.dst[0] = kv; gk.ld[0] = 2 * gd; gk.cend[0] = gd; gk.scale[0] = 1.f;
    gk.dst[1] = dt == MTFM_BF16 ? nullptr : kv + gd * es; gk.ld[1] = 2 * gd; gk.cend[1] = 2 * gd; gk.scale[1] = 1.f;
    gk.cend[2] = gk.cend[3] = 2 * gd;
    if (keep) {   // the backward also needs V row-major and the pre-activations
      gk.cend[0] = 2 * gd; gk.dst[1] = nullptr;
      gk.pre = keep->kvpre; gk.ldpre = 2 * gd;
    }
    if (dt == MTFM_BF16) { gk.vt = ws + L.vt; gk.ldvt = L.ldvt; gk.vt_col0 = gd; gk.vt_cols = gd; }
    TRY(timed_gemm(MTFM_K_GEMM_KV, gk, dt, c.s));
  }

  GemmArgs gt{};
  gt.M = (int32_t)p.n_parents; gt.N = zw; gt.K = D; gt.groups = S;
  gt.A = xt; gt.lda = D; gt.amap = RowMap{c.meta.parent_row, 0, 0}; gt.amap_zadd = 1; gt.a_rows = c.plan.n_rows;
  gt.B[0] = w->w_u; gt.bn[0] = hd;
  gt.B[1] = w->w_q; gt.bn[1] = hd; gt.bz[1] = (int64_t)hd * D;
  gt.B[2] = w->w_kv; gt.bn[2] = 2 * gd;
  gt.ldb = D;
  gt.bs24 = w->w_t_s24; gt.bs24_rows = S * zw; gt.bs24_zrows = zw;
  gt.cmap = RowMap{nullptr, S, 0}; gt.cmap_zadd = 1;
  gt.epi = EPI_SILU_SPLIT;
  gt.dst[0] = zt; gt.ld[0] = zw; gt.cend[0] = hd; gt.scale[0] = 1.f;
  gt.dst[1] = zt + hd * es; gt.ld[1] = zw; gt.cend[1] = 2 * hd; gt.scale[1] = q_scale(dh);
  gt.dst[2] = zt + 2 * hd * es; gt.ld[2] = zw; gt.cend[2] = zw; gt.scale[2] = 1.f;
  gt.cend[3] = zw;
  if (keep) { gt.pre = keep->hpre; gt.ldpre = zw; }
  TRY(timed_gemm(MTFM_K_GEMM_T, gt, dt, c.s));

  AttnArgs aa{};
  aa.q = zt + hd * es; aa.ldq = zw;
  aa.k = kv; aa.ldk = 2 * gd;
  aa.v = kv + gd * es; aa.ldv = 2 * gd;
  aa.vt = ws + L.vt; aa.ldvt = L.ldvt; aa.n_key_rows = (int32_t)p.n_rows; aa.max_user_rows = p.max_user_rows;
  aa.kd = zt + 2 * hd * es; aa.ldkd = zw;
  aa.vd = zt + (2 * hd + gd) * es; aa.ldvd = zw;
  aa.a = a; aa.lda = hd;
  aa.tiles = c.meta.target_tiles; aa.ntiles = (int32_t)p.n_target_tiles;
  aa.order = c.meta.target_order; aa.n_order = (int32_t)p.n_target_order;
  if (dt == MTFM_BF16) {
    // T rows ordered by visible prefix: slices of similar rows cut fewer key tiles
    aa.tiles = c.meta.target_tiles_sorted; aa.qperm = c.meta.tsort_q; aa.gperm = c.meta.tsort_g;
  }
  aa.p = c.meta.p; aa.n = c.meta.n; aa.lens = c.b->lens_d;
  aa.H = H; aa.G = G; aa.dh = dh; aa.out_scale = kLn2;
  aa.per_group = 1;
  TRY(timed_attention(MTFM_K_ATTN_TARGET, aa, dt, c.s));

  {
    GlnArgs g2{};
    g2.rows = (int32_t)p.n_t_rows; g2.D = hd; g2.x = a; g2.ldx = hd; g2.y = y; g2.ldy = hd;
    g2.gate = zt; g2.ldg = zw;
    g2.gamma = w->ln2_g; g2.beta = w->ln2_b; g2.type = nullptr; g2.type_const = TT_T; g2.eps = d->ln_eps;
    TRY(timed_gln(g2, dt, c.s, MTFM_K_GLN_T));
  }

  GemmArgs go{};
  go.M = (int32_t)p.n_parents; go.N = D; go.K = hd; go.groups = S;
  go.A = y; go.lda = hd; go.amap = RowMap{nullptr, S, 0}; go.amap_zadd = 1;
  go.B[0] = w->w_o; go.bn[0] = D; go.ldb = hd;
  go.bs24 = w->w_o_s24; go.bs24_rows = D;
  go.cmap = RowMap{c.meta.parent_row, 0, 0}; go.cmap_zadd = 1;
  go.epi = EPI_RESID; go.resid = x_in; go.ldr = D; go.out = x_out; go.ldo = D;
  TRY(timed_gemm(MTFM_K_GEMM_OUT_T, go, dt, c.s));
  return MTFM_OK;
}

// ---------------------------------------------------------------------------
// Context stage of the target layers l = 0..k-1 of one block, right after its
// full layer: one normalisation pass over all rows writes every layer's X~
// (T rows as zeros in layers 1..k-1: their K/V are never read as keys; layer
// 0's T rows are its T-row pre-norm, which run_target_rows reads from there,
// since the T rows have not changed since the full layer), then each layer's K
// and V^T over all packed rows: when the k layers' K|V weights are all dense
// or all packed (2:4), one grouped launch (more workgroups than any one
// layer's, so a shorter tail), else one launch per layer; with a K/V cache
// (serving), one launch per layer into its cache entry.
mtfm_status run_target_context(const Ctx& c, const mtfm_dims* d, const mtfm_target_w* w, int k, const void* x,
                               char* ws, const BackboneWs& L, const KvOut* kv = nullptr) {
  const MetaPlan& p = c.plan;
  const int dt = d->dtype;
  const int64_t es = elem_size(dt);
  const int G = d->n_kv_heads, dh = d->head_dim, D = d->d_model, gd = G * dh;
  GlnArgs g1{};
  g1.rows = (int32_t)p.n_rows; g1.D = D; g1.x = x; g1.ldx = D; g1.y = ws + L.xt[0]; g1.ldy = D;
  g1.gamma = w[0].ln1_g; g1.beta = w[0].ln1_b; g1.type = c.meta.type; g1.eps = d->ln_eps;
  g1.n_more = k - 1; g1.zero_t = ((1 << k) - 1) & ~1;
  for (int l = 1; l < k; ++l) {
    g1.y_more[l - 1] = ws + L.xt[l]; g1.gamma_more[l - 1] = w[l].ln1_g; g1.beta_more[l - 1] = w[l].ln1_b;
  }
  TRY(timed_gln(g1, dt, c.s, MTFM_K_GLN_T));
  int n_packed = 0;
  for (int l = 0; l < k; ++l) n_packed += w[l].w_kv_s24 ? 1 : 0;
  if (!kv && dt == MTFM_BF16 && (n_packed == 0 || n_packed == k)) {
    // group l reads X~_l and layer l's weights and writes K_l and V^T_l (the
    // buffers of the k layers lie back to back)
    GemmArgs gk{};
    gk.M = (int32_t)p.n_rows; gk.N = 2 * gd; gk.K = D; gk.groups = k;
    gk.A = ws + L.xt[0]; gk.lda = D; gk.amap = identity_map(); gk.amap_zadd = (int32_t)p.n_rows;
    gk.B[0] = w[0].w_kv; gk.bn[0] = 2 * gd; gk.ldb = D;
    if (n_packed) { gk.bs24 = w[0].w_kv_s24; gk.bs24_rows = 2 * gd; gk.bs24_zrows = 0; }
    for (int l = 0; l < k; ++l) gk.bgroup[l] = n_packed ? w[l].w_kv_s24 : w[l].w_kv;
    gk.cmap = identity_map(); gk.cmap_zadd = (int32_t)p.n_rows;
    gk.epi = EPI_SILU_SPLIT;
    gk.dst[0] = ws + L.k[0]; gk.ld[0] = gd; gk.cend[0] = gd; gk.scale[0] = 1.f;
    gk.dst[1] = nullptr; gk.cend[1] = gk.cend[2] = gk.cend[3] = 2 * gd; gk.scale[1] = 1.f;
    gk.vt = ws + L.vt[0]; gk.ldvt = L.ldvt; gk.vt_col0 = gd; gk.vt_cols = gd;
    gk.vt_zstride = k > 1 ? (L.vt[1] - L.vt[0]) / es : 0;
    return timed_gemm(MTFM_K_GEMM_KV, gk, dt, c.s);
  }
  for (int l = 0; l < k; ++l) {
    GemmArgs gk{};
    gk.M = (int32_t)p.n_rows; gk.N = 2 * gd; gk.K = D; gk.groups = 1;
    gk.A = ws + L.xt[l]; gk.lda = D; gk.amap = identity_map();
    gk.B[0] = w[l].w_kv; gk.bn[0] = 2 * gd; gk.ldb = D;
    gk.bs24 = w[l].w_kv_s24; gk.bs24_rows = 2 * gd;
    gk.cmap = identity_map();
    gk.epi = EPI_SILU_SPLIT;
    gk.dst[0] = kv ? kv[l].k : ws + L.k[l]; gk.ld[0] = gd; gk.cend[0] = gd; gk.scale[0] = 1.f;
    gk.dst[1] = nullptr; gk.cend[1] = gk.cend[2] = gk.cend[3] = 2 * gd; gk.scale[1] = 1.f;
    gk.vt = kv ? kv[l].vt : ws + L.vt[l]; gk.ldvt = kv ? kv[l].ldvt : L.ldvt; gk.vt_col0 = gd; gk.vt_cols = gd;
    TRY(timed_gemm(MTFM_K_GEMM_KV, gk, dt, c.s));
  }
  return MTFM_OK;
}

// T-row part of target layer l after run_target_context: normalise the T rows
// of the current X, project them, attend over the precomputed K / V^T, gate,
// project out and add the residual in place.
mtfm_status run_target_rows(const Ctx& c, const mtfm_dims* d, const mtfm_target_w* w, void* x, char* ws,
                            const BackboneWs& L, int l) {
  const MetaPlan& p = c.plan;
  const int dt = d->dtype;
  const int64_t es = elem_size(dt);
  const int H = d->n_q_heads, G = d->n_kv_heads, dh = d->head_dim, D = d->d_model;
  const int hd = H * dh, gd = G * dh, zw = 2 * hd + 2 * gd;
  const int S = p.split;
  char* xtt = ws + L.xtt;
  char* zt = ws + L.zt;
  char* a = ws + L.a;
  char* y = ws + L.y;
  if (p.n_t_rows == 0) return MTFM_OK;

  // T row t = parent m * S + sub-token z sits at packed row parent_row[m] + z
  GemmArgs gt{};
  gt.M = (int32_t)p.n_parents; gt.N = zw; gt.K = D; gt.groups = S;
  // gathered GEMM rows are addressed through one 31-bit offset range
  if (l == 0 && (int64_t)p.n_rows * D * 2 + (int64_t)D * 2 < ((int64_t)1 << 31)) {
    // the context stage's normalisation of layer 0 already holds the T rows' X~
    // (same rows, same parameters): gather them from there
    gt.A = ws + L.xt[0]; gt.lda = D; gt.amap = RowMap{c.meta.parent_row, 0, 0}; gt.amap_zadd = 1;
    gt.a_rows = p.n_rows;
  } else {
    GlnArgs g1{};
    g1.rows = (int32_t)p.n_t_rows; g1.D = D; g1.x = x; g1.ldx = D; g1.y = xtt; g1.ldy = D;
    g1.xlist = c.meta.parent_row; g1.xdiv = S;
    g1.gamma = w->ln1_g; g1.beta = w->ln1_b; g1.type = nullptr; g1.type_const = TT_T; g1.eps = d->ln_eps;
    TRY(timed_gln(g1, dt, c.s, MTFM_K_GLN_T));
    gt.A = xtt; gt.lda = D; gt.amap = RowMap{nullptr, S, 0}; gt.amap_zadd = 1;
  }
  gt.B[0] = w->w_u; gt.bn[0] = hd;
  gt.B[1] = w->w_q; gt.bn[1] = hd; gt.bz[1] = (int64_t)hd * D;
  gt.B[2] = w->w_kv; gt.bn[2] = 2 * gd;
  gt.ldb = D;
  gt.bs24 = w->w_t_s24; gt.bs24_rows = S * zw; gt.bs24_zrows = zw;
  gt.cmap = RowMap{nullptr, S, 0}; gt.cmap_zadd = 1;
  gt.epi = EPI_SILU_SPLIT;
  gt.dst[0] = zt; gt.ld[0] = zw; gt.cend[0] = hd; gt.scale[0] = 1.f;
  gt.dst[1] = zt + hd * es; gt.ld[1] = zw; gt.cend[1] = 2 * hd; gt.scale[1] = q_scale(dh);
  gt.dst[2] = zt + 2 * hd * es; gt.ld[2] = zw; gt.cend[2] = zw; gt.scale[2] = 1.f;
  gt.cend[3] = zw;
  TRY(timed_gemm(MTFM_K_GEMM_T, gt, dt, c.s));

  AttnArgs aa{};
  aa.q = zt + hd * es; aa.ldq = zw;
  aa.k = ws + L.k[l]; aa.ldk = gd;
  aa.v = nullptr; aa.ldv = 0;
  aa.vt = ws + L.vt[l]; aa.ldvt = L.ldvt; aa.n_key_rows = (int32_t)p.n_rows; aa.max_user_rows = p.max_user_rows;
  aa.kd = zt + 2 * hd * es; aa.ldkd = zw;
  aa.vd = zt + (2 * hd + gd) * es; aa.ldvd = zw;
  aa.a = a; aa.lda = hd;
  aa.tiles = c.meta.target_tiles; aa.ntiles = (int32_t)p.n_target_tiles;
  aa.order = c.meta.target_order; aa.n_order = (int32_t)p.n_target_order;
  if (dt == MTFM_BF16) {
    // T rows ordered by visible prefix: slices of similar rows cut fewer key tiles
    aa.tiles = c.meta.target_tiles_sorted; aa.qperm = c.meta.tsort_q; aa.gperm = c.meta.tsort_g;
  }
  aa.p = c.meta.p; aa.n = c.meta.n; aa.lens = c.b->lens_d;
  aa.H = H; aa.G = G; aa.dh = dh; aa.out_scale = kLn2;
  aa.per_group = 1;
  float* parts = L.ksplit > 1 ? (float*)(ws + L.apart) : nullptr;
  if (parts) { aa.ksplit = L.ksplit; aa.a_part = parts; aa.part_stride = p.n_t_rows * hd; }
  TRY(timed_attention(MTFM_K_ATTN_TARGET, aa, dt, c.s));

  TRY(target_gated_gln(c, d, w->ln2_g, w->ln2_b, a, zt, zw, y, dt, parts, L.ksplit));

  GemmArgs go{};
  go.M = (int32_t)p.n_parents; go.N = D; go.K = hd; go.groups = S;
  go.A = y; go.lda = hd; go.amap = RowMap{nullptr, S, 0}; go.amap_zadd = 1;
  go.B[0] = w->w_o; go.bn[0] = D; go.ldb = hd;
  go.bs24 = w->w_o_s24; go.bs24_rows = D;
  go.cmap = RowMap{c.meta.parent_row, 0, 0}; go.cmap_zadd = 1;
  go.epi = EPI_RESID; go.resid = x; go.ldr = D; go.out = x; go.ldo = D;
  TRY(timed_gemm(MTFM_K_GEMM_OUT_T, go, dt, c.s));
  return MTFM_OK;
}

// ---------------------------------------------------------------------------

// ---------------------------------------------------------------------------
// V2 target side ([blog] §3.3.2): AutoSplit, per-sub-token SwiGLU FFN with the
// token mixing, mean pooling (readings in include/mtfm.h).
namespace {

struct FfnWs {
  int64_t wgu = 0, xtt = 0, h = 0, total = 0;
};

FfnWs ffn_ws(const MetaPlan& p, const mtfm_dims* d, int d_ff) {
  FfnWs w;
  int64_t off = 0;
  auto take = [&](int64_t bytes) { int64_t o = off; off = align_up(off + std::max<int64_t>(bytes, 0), 256); return o; };
  w.wgu = take((int64_t)p.split * 2 * d_ff * d->d_model * 2);
  w.xtt = take(p.n_t_rows * d->d_model * 2);
  w.h = take(p.n_t_rows * (int64_t)d_ff * 2);
  w.total = off;
  return w;
}

mtfm_status v2_checks(const mtfm_batch* batch, const mtfm_dims* dims, const void* meta_d, Ctx* c) {
  TRY(plan_meta(batch, &c->plan));
  TRY(check_dims(dims));
  if (dims->dtype != MTFM_BF16) return MTFM_E_UNSUPPORTED;
  if (!meta_d) return MTFM_E_NULL;
  TRY(check_batch_device(batch, c->plan));
  c->b = batch;
  c->meta = meta_ptrs(c->plan, meta_d);
  return MTFM_OK;
}

mtfm_status check_ffn(const mtfm_dims* d, int d_ff, int split, const mtfm_ffn_w* w) {
  if (!w || !w->ln_g || !w->ln_b || !w->w_gate || !w->w_up || !w->w_down) return MTFM_E_NULL;
  if (d_ff <= 0 || d_ff % 32 != 0) return MTFM_E_UNSUPPORTED;
  if (split > 1 && (d->d_model % split != 0 || (d->d_model / split) % 8 != 0 || split * d->d_model / 8 > 1024))
    return MTFM_E_UNSUPPORTED;
  return MTFM_OK;
}

// Token FFN + mixing of one target layer on the T rows of x (packed, in place).
mtfm_status run_token_ffn(const Ctx& c, const mtfm_dims* d, int d_ff, const mtfm_ffn_w* w, void* x, char* ws,
                          const FfnWs& L) {
  const MetaPlan& p = c.plan;
  const int S = p.split, D = d->d_model;
  if (p.n_t_rows == 0) return MTFM_OK;
  {
    RepackArgs r{};
    r.gate = (const bf16*)w->w_gate; r.up = (const bf16*)w->w_up; r.out = (bf16*)(ws + L.wgu);
    r.S = S; r.F = d_ff; r.D = D;
    TimedLaunch t(MTFM_K_V2, c.s);
    TRY(launch_repack_gate_up(r, c.s));
  }
  GlnArgs g1{};
  g1.rows = (int32_t)p.n_t_rows; g1.D = D; g1.x = x; g1.ldx = D; g1.y = ws + L.xtt; g1.ldy = D;
  g1.xlist = c.meta.parent_row; g1.xdiv = S;
  g1.gamma = w->ln_g; g1.beta = w->ln_b; g1.type = nullptr; g1.type_const = TT_T; g1.eps = d->ln_eps;
  TRY(timed_gln(g1, MTFM_BF16, c.s));

  GemmArgs gu{};
  gu.M = (int32_t)p.n_parents; gu.N = 2 * d_ff; gu.K = D; gu.groups = S;
  gu.A = ws + L.xtt; gu.lda = D; gu.amap = RowMap{nullptr, S, 0}; gu.amap_zadd = 1;
  gu.B[0] = ws + L.wgu; gu.bn[0] = 2 * d_ff; gu.bz[0] = (int64_t)2 * d_ff * D; gu.ldb = D;
  gu.cmap = RowMap{nullptr, S, 0}; gu.cmap_zadd = 1;
  gu.epi = EPI_SWIGLU; gu.out = ws + L.h; gu.ldo = d_ff;
  TRY(timed_gemm(MTFM_K_V2, gu, MTFM_BF16, c.s));

  GemmArgs gd{};
  gd.M = (int32_t)p.n_parents; gd.N = D; gd.K = d_ff; gd.groups = S;
  gd.A = ws + L.h; gd.lda = d_ff; gd.amap = RowMap{nullptr, S, 0}; gd.amap_zadd = 1;
  gd.B[0] = w->w_down; gd.bn[0] = D; gd.bz[0] = (int64_t)D * d_ff; gd.ldb = d_ff;
  gd.cmap = RowMap{c.meta.parent_row, 0, 0}; gd.cmap_zadd = 1;
  gd.epi = EPI_RESID; gd.resid = x; gd.ldr = D; gd.out = x; gd.ldo = D;
  TRY(timed_gemm(MTFM_K_V2, gd, MTFM_BF16, c.s));

  TokenRowsArgs m{};
  m.x = (bf16*)x; m.ldx = D; m.parent_row = c.meta.parent_row; m.n_parents = (int32_t)p.n_parents; m.S = S; m.D = D;
  TimedLaunch t(MTFM_K_V2, c.s);
  return launch_token_mix(m, c.s);
}

}  // namespace

// ---------------------------------------------------------------------------
// Request-level serving with user-side K/V reuse ([explainer] §5.2.3: K/V
// cache sharing across serving micro-batches; [blog] §3.4 and §4: one
// user-level sample shares the long-sequence attention among all of its
// targets).  H and R rows never attend to T rows, so their values through the
// whole stack, and every layer's K and V of them, do not depend on the
// candidates: one context pass per user fills a cache of each layer's K and
// V^T of the context rows; each candidate batch then runs only its T rows
// through the 16 layers against that cache.
namespace {

struct KvCacheLayout {
  int64_t ldvt = 0, k = 0, per_layer = 0, total = 0;
};

// Per layer: K [ctx rows][G*dh], then V^T [G*dh][ldvt] (bf16), 256-B aligned.
KvCacheLayout kv_cache_layout(const MetaPlan& p, const mtfm_dims* d, int n_layers) {
  const int64_t gd = (int64_t)d->n_kv_heads * d->head_dim;
  KvCacheLayout c;
  c.ldvt = vt_ld(p.n_ctx_rows);
  c.k = align_up(p.n_ctx_rows * gd * 2, 256);
  c.per_layer = c.k + align_up(gd * c.ldvt * 2, 256);
  c.total = c.per_layer * n_layers;
  return c;
}

KvOut kv_of(const KvCacheLayout& c, char* cache, int layer) {
  KvOut o;
  o.k = cache + layer * c.per_layer;
  o.vt = cache + layer * c.per_layer + c.k;
  o.ldvt = c.ldvt;
  return o;
}

// Tile descriptors whose key base [7] is the user's first context row in the
// cache (context rows of all users back to back) instead of its packed row.
__global__ void rebase_tiles_kernel(const int32_t* in, int n, const int32_t* ctx_off, int32_t* out) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n * 8) return;
  const int t = i >> 3, f = i & 7;
  out[i] = f == TD_UROW0 ? ctx_off[in[8 * t + TD_USER]] : in[i];
}

struct ServeWs {
  int64_t tiles = 0, xtt = 0, zt = 0, a = 0, y = 0, apart = 0, total = 0;
  int32_t ksplit = 1;   // key splits of the target attention (fp32 partials of A at apart)
};

ServeWs serve_ws(const MetaPlan& p, const mtfm_dims* d) {
  const int64_t hd = (int64_t)d->n_q_heads * d->head_dim, gd = (int64_t)d->n_kv_heads * d->head_dim;
  const int64_t zw = 2 * hd + 2 * gd, T = p.n_t_rows;
  ServeWs w;
  int64_t off = 0;
  auto take = [&](int64_t bytes) { int64_t o = off; off = align_up(off + std::max<int64_t>(bytes, 0), 256); return o; };
  w.tiles = take(p.n_target_tiles * 8 * 4);
  w.xtt = take(T * d->d_model * 2);
  w.zt = take(T * zw * 2);
  w.a = take(T * hd * 2);
  w.y = take(T * hd * 2);
  w.ksplit = target_key_splits(p, d);
  w.apart = take(w.ksplit > 1 ? w.ksplit * T * hd * 4 : 0);
  w.total = off;
  return w;
}

// One layer over the T rows (T-row order: sub-token z of parent m at m * S + z)
// against that layer's cached context K / V^T.  fw (a full layer: one U|Q|K|V
// projection for every sub-token) or tw (a target layer: per-sub-token Q).
mtfm_status serve_rows(const Ctx& c, const mtfm_dims* d, const mtfm_full_w* fw, const mtfm_target_w* tw,
                       const KvOut& kv, const int32_t* tiles, void* x, char* ws, const ServeWs& L) {
  const MetaPlan& p = c.plan;
  const int dt = MTFM_BF16;
  const int64_t es = 2;
  const int H = d->n_q_heads, G = d->n_kv_heads, dh = d->head_dim, D = d->d_model;
  const int hd = H * dh, gd = G * dh, zw = 2 * hd + 2 * gd;
  const int S = p.split;
  char* xtt = ws + L.xtt;
  char* zt = ws + L.zt;
  char* a = ws + L.a;
  char* y = ws + L.y;

  GlnArgs g1{};
  g1.rows = (int32_t)p.n_t_rows; g1.D = D; g1.x = x; g1.ldx = D; g1.y = xtt; g1.ldy = D;
  g1.gamma = fw ? fw->ln1_g : tw->ln1_g; g1.beta = fw ? fw->ln1_b : tw->ln1_b;
  g1.type = nullptr; g1.type_const = TT_T; g1.eps = d->ln_eps;
  // a candidate pass is T-row work alone: its small normalised outputs stay in
  // L2 for the projection that reads them next (cached stores; the backbone's
  // T-row passes measured slower with them, beside its all-row streams)
  g1.temporal = 1;
  TRY(timed_gln(g1, dt, c.s, MTFM_K_GLN_T));

  GemmArgs gt{};
  gt.K = D; gt.A = xtt; gt.lda = D; gt.ldb = D;
  gt.epi = EPI_SILU_SPLIT;
  gt.dst[0] = zt; gt.ld[0] = zw; gt.cend[0] = hd; gt.scale[0] = 1.f;
  gt.dst[1] = zt + hd * es; gt.ld[1] = zw; gt.cend[1] = 2 * hd; gt.scale[1] = q_scale(dh);
  gt.dst[2] = zt + 2 * hd * es; gt.ld[2] = zw; gt.cend[2] = zw; gt.scale[2] = 1.f;
  gt.cend[3] = zw;
  gt.N = zw;
  if (fw) {
    gt.M = (int32_t)p.n_t_rows; gt.groups = 1;
    gt.amap = identity_map(); gt.cmap = identity_map();
    gt.B[0] = fw->w_uqkv; gt.bn[0] = zw;
    gt.bs24 = fw->w_uqkv_s24; gt.bs24_rows = zw;
  } else {
    gt.M = (int32_t)p.n_parents; gt.groups = S;
    gt.amap = RowMap{nullptr, S, 0}; gt.amap_zadd = 1;
    gt.cmap = RowMap{nullptr, S, 0}; gt.cmap_zadd = 1;
    gt.B[0] = tw->w_u; gt.bn[0] = hd;
    gt.B[1] = tw->w_q; gt.bn[1] = hd; gt.bz[1] = (int64_t)hd * D;
    gt.B[2] = tw->w_kv; gt.bn[2] = 2 * gd;
    gt.bs24 = tw->w_t_s24; gt.bs24_rows = S * zw; gt.bs24_zrows = zw;
  }
  TRY(timed_gemm(MTFM_K_GEMM_T, gt, dt, c.s));

  AttnArgs aa{};
  aa.q = zt + hd * es; aa.ldq = zw;
  aa.k = kv.k; aa.ldk = gd;
  aa.v = nullptr; aa.ldv = 0;
  aa.vt = kv.vt; aa.ldvt = kv.ldvt; aa.n_key_rows = (int32_t)p.n_ctx_rows; aa.max_user_rows = p.max_user_rows;
  aa.kd = zt + 2 * hd * es; aa.ldkd = zw;
  aa.vd = zt + (2 * hd + gd) * es; aa.ldvd = zw;
  aa.a = a; aa.lda = hd;
  aa.tiles = tiles; aa.ntiles = (int32_t)p.n_target_tiles;   // the sorted tiles, rebased on the cache
  aa.order = c.meta.target_order; aa.n_order = (int32_t)p.n_target_order;
  aa.qperm = c.meta.tsort_q; aa.gperm = c.meta.tsort_g;
  aa.p = c.meta.p; aa.n = c.meta.n; aa.lens = c.b->lens_d;
  aa.H = H; aa.G = G; aa.dh = dh; aa.out_scale = kLn2;
  aa.per_group = 1;
  float* parts = L.ksplit > 1 ? (float*)(ws + L.apart) : nullptr;
  if (parts) { aa.ksplit = L.ksplit; aa.a_part = parts; aa.part_stride = p.n_t_rows * hd; }
  TRY(timed_attention(MTFM_K_ATTN_TARGET, aa, dt, c.s));

  TRY(target_gated_gln(c, d, fw ? fw->ln2_g : tw->ln2_g, fw ? fw->ln2_b : tw->ln2_b, a, zt, zw, y, dt, parts,
                       L.ksplit, true));

  GemmArgs go{};
  go.M = (int32_t)p.n_t_rows; go.N = D; go.K = hd; go.groups = 1;
  go.A = y; go.lda = hd; go.amap = identity_map();
  go.B[0] = fw ? fw->w_o : tw->w_o; go.bn[0] = D; go.ldb = hd;
  go.bs24 = fw ? fw->w_o_s24 : tw->w_o_s24; go.bs24_rows = D;
  go.cmap = identity_map();
  go.epi = EPI_RESID; go.resid = x; go.ldr = D; go.out = x; go.ldo = D;
  TRY(timed_gemm(MTFM_K_GEMM_OUT_T, go, dt, c.s));
  return MTFM_OK;
}

mtfm_status serve_checks(const mtfm_batch* batch, const mtfm_dims* dims, int32_t n_blocks, int32_t k_target,
                         const void* meta_d, const mtfm_full_w* full, const mtfm_target_w* tgt, Ctx* c) {
  if (n_blocks < 0 || k_target < 0) return MTFM_E_DIMS;
  TRY(plan_meta(batch, &c->plan));
  TRY(check_dims(dims));
  if (dims->dtype != MTFM_BF16 || k_target > 4) return MTFM_E_UNSUPPORTED;
  if (!meta_d) return MTFM_E_NULL;
  TRY(check_batch_device(batch, c->plan));
  if (n_blocks > 0 && !full) return MTFM_E_NULL;
  if (n_blocks > 0 && k_target > 0 && !tgt) return MTFM_E_NULL;
  for (int b = 0; b < n_blocks; ++b) {
    TRY(check_full_w(&full[b], dims));
    for (int t = 0; t < k_target; ++t) TRY(check_target_w(&tgt[b * k_target + t], dims));
  }
  c->b = batch;
  c->meta = meta_ptrs(c->plan, meta_d);
  return MTFM_OK;
}

}  // namespace

// Argument checks of the candidate pass (everything but the workspace).
mtfm_status serve_targets_check(const mtfm_batch* batch, const mtfm_dims* dims, int32_t n_blocks, int32_t k_target,
                                const void* meta_d, const mtfm_full_w* full, const mtfm_target_w* tgt,
                                const void* kv_cache, size_t cache_bytes, const void* x_t, Ctx* c) {
  TRY(serve_checks(batch, dims, n_blocks, k_target, meta_d, full, tgt, c));
  const KvCacheLayout K = kv_cache_layout(c->plan, dims, n_blocks * (1 + k_target));
  if (c->plan.n_t_rows > 0 && (!x_t || !kv_cache)) return MTFM_E_NULL;
  if (cache_bytes < (size_t)K.total) return MTFM_E_WORKSPACE;
  return MTFM_OK;
}

int64_t serve_targets_ws_bytes(const MetaPlan& p, const mtfm_dims* d) { return serve_ws(p, d).total; }

// The candidate pass on checked arguments with a workspace of at least
// serve_targets_ws_bytes bytes.
mtfm_status serve_targets_run(const Ctx& c, const mtfm_dims* dims, int32_t n_blocks, int32_t k_target,
                              const mtfm_full_w* full, const mtfm_target_w* tgt, const void* kv_cache, void* x_t,
                              char* w) {
  if (c.plan.n_t_rows == 0 || n_blocks == 0) return MTFM_OK;
  const KvCacheLayout K = kv_cache_layout(c.plan, dims, n_blocks * (1 + k_target));
  const ServeWs L = serve_ws(c.plan, dims);
  int32_t* tiles = (int32_t*)(w + L.tiles);
  {
    const int n = (int)c.plan.n_target_tiles;
    rebase_tiles_kernel<<<(n * 8 + 255) / 256, 256, 0, c.s>>>(c.meta.target_tiles_sorted, n,
                                                               c.meta.user + UT_CTX * (c.plan.n_users + 1), tiles);
    MTFM_LAUNCH_CHECK("rebase_tiles");
  }
  char* cache = (char*)kv_cache;
  const int per = 1 + k_target;
  for (int b = 0; b < n_blocks; ++b) {
    TRY(serve_rows(c, dims, &full[b], nullptr, kv_of(K, cache, b * per), tiles, x_t, w, L));
    for (int t = 0; t < k_target; ++t)
      TRY(serve_rows(c, dims, nullptr, &tgt[b * k_target + t], kv_of(K, cache, b * per + 1 + t), tiles, x_t, w, L));
  }
  return MTFM_OK;
}

// Backward through the whole stack: one forward pass keeps every layer's input
// (bf16, as the forward hands it on), then the layers' backward run from the
// last to the first, each taking the next layer's input gradient as its
// upstream gradient.  Workspace: the largest single-layer workspace, the
// inputs of layers 1 .. L-1, one gradient buffer (the caller's dx is the
// other one of the pair), then (full size only) the kept intermediates of
// layers 0 .. L-2.
namespace {

// With the full workspace the forward pass also keeps each layer's
// intermediates (X~, the projections and their pre-activations, the
// attention output), so no layer backward recomputes them; with only the
// minimum (the regions before `keep`) every layer backward recomputes them.
struct BackboneBwdWs {
  int64_t layer = 0, stash = 0, xbytes = 0, gbuf = 0, keep = 0, total = 0;
  int per = 1;
  int64_t R = 0, T = 0, D = 0, hd = 0, gd2 = 0, zw = 0;
  static int64_t al(int64_t b) { return align_up(std::max<int64_t>(b, 0), 256); }
  int64_t kfull() const { return al(R * D * 2) + 2 * al(R * zw * 2) + al(R * hd * 2); }
  int64_t ktarget() const { return al(R * D * 2) + 2 * al(R * gd2 * 2) + 2 * al(T * zw * 2) + al(T * hd * 2); }
  int64_t keep_off(int l) const {   // kept intermediates of layer l (l < L - 1)
    const int nf = (l + per - 1) / per;   // full layers before l
    return keep + nf * kfull() + (l - nf) * ktarget();
  }
  FwdKeep keep_of(char* w, int l) const {
    FwdKeep k;
    char* b = w + keep_off(l);
    k.xt = b; b += al(R * D * 2);
    if (l % per == 0) {
      k.z = b; b += al(R * zw * 2);
      k.hpre = b; b += al(R * zw * 2);
      k.a = b;
    } else {
      k.kv = b; b += al(R * gd2 * 2);
      k.kvpre = b; b += al(R * gd2 * 2);
      k.z = b; b += al(T * zw * 2);
      k.hpre = b; b += al(T * zw * 2);
      k.a = b;
    }
    return k;
  }
};

BackboneBwdWs backbone_bwd_ws(const MetaPlan& p, const mtfm_dims* d, int n_blocks, int k_target) {
  BackboneBwdWs w;
  const int n_layers = n_blocks * (1 + k_target);
  int64_t off = 0;
  auto take = [&](int64_t bytes) { int64_t o = off; off = align_up(off + std::max<int64_t>(bytes, 0), 256); return o; };
  const int64_t lw = std::max(std::max(layer_ws(p, d, MTFM_OP_FULL).total, layer_ws(p, d, MTFM_OP_TARGET).total),
                              std::max(bwd_ws_bytes(p, d, MTFM_OP_FULL_BWD), bwd_ws_bytes(p, d, MTFM_OP_TARGET_BWD)));
  w.layer = take(lw);
  w.xbytes = align_up(p.n_rows * d->d_model * elem_size(d->dtype), 256);
  w.stash = take(std::max(n_layers - 1, 0) * w.xbytes);
  w.gbuf = take(w.xbytes);
  w.per = 1 + k_target;
  w.R = p.n_rows; w.T = p.n_t_rows; w.D = d->d_model;
  w.hd = (int64_t)d->n_q_heads * d->head_dim;
  w.gd2 = 2 * (int64_t)d->n_kv_heads * d->head_dim;
  w.zw = 2 * w.hd + w.gd2;
  w.keep = off;
  w.total = n_layers > 1 ? w.keep_off(n_layers - 1) : off;
  return w;
}

}  // namespace

extern "C" {

size_t mtfm_meta_bytes(const mtfm_batch* batch) {
  MetaPlan p;
  if (plan_meta(batch, &p) != MTFM_OK) return 0;
  return (size_t)p.lay.total_bytes;
}

mtfm_status mtfm_meta_layout_of(const mtfm_batch* batch, mtfm_meta_layout* layout) {
  if (!layout) return MTFM_E_NULL;
  MetaPlan p;
  TRY(plan_meta(batch, &p));
  *layout = p.lay;
  return MTFM_OK;
}

mtfm_status mtfm_mask_build(const mtfm_batch* batch, void* meta_d, size_t meta_bytes, void* stream) {
  MetaPlan p;
  TRY(plan_meta(batch, &p));
  if (!meta_d) return MTFM_E_NULL;
  TRY(check_batch_device(batch, p));
  if (meta_bytes < (size_t)p.lay.total_bytes) return MTFM_E_WORKSPACE;
  TimedLaunch t(MTFM_K_MASK, (hipStream_t)stream);
  return launch_mask_build(batch, p, meta_d, (hipStream_t)stream);
}

size_t mtfm_workspace_bytes(const mtfm_batch* batch, const mtfm_dims* dims, int32_t op) {
  MetaPlan p;
  if (plan_meta(batch, &p) != MTFM_OK || check_dims(dims) != MTFM_OK) return 0;
  switch (op) {
    case MTFM_OP_FULL: return (size_t)layer_ws(p, dims, MTFM_OP_FULL).total;
    case MTFM_OP_TARGET: return (size_t)layer_ws(p, dims, MTFM_OP_TARGET).total;
    case MTFM_OP_BACKBONE:
      return (size_t)std::max(layer_ws(p, dims, MTFM_OP_FULL).total, layer_ws(p, dims, MTFM_OP_TARGET).total);
    case MTFM_OP_FULL_BWD: return (size_t)bwd_ws_bytes(p, dims, MTFM_OP_FULL_BWD);
    case MTFM_OP_TARGET_BWD: return (size_t)bwd_ws_bytes(p, dims, MTFM_OP_TARGET_BWD);
    default: return 0;
  }
}

mtfm_status mtfm_workspace_probe(const mtfm_batch* batch, const mtfm_dims* dims, int32_t op, int64_t* off_a,
                                 int64_t* off_y) {
  if (!off_a || !off_y) return MTFM_E_NULL;
  MetaPlan p;
  TRY(plan_meta(batch, &p));
  TRY(check_dims(dims));
  if (op != MTFM_OP_FULL && op != MTFM_OP_TARGET) return MTFM_E_UNSUPPORTED;
  const LayerWs L = layer_ws(p, dims, op);
  *off_a = L.a;
  *off_y = L.y;
  return MTFM_OK;
}

mtfm_status mtfm_attn_full(const mtfm_batch* batch, const mtfm_dims* dims, const void* meta_d, const mtfm_full_w* w,
                           const void* x_in, void* x_out, void* ws, size_t ws_bytes, void* stream) {
  Ctx c;
  TRY(prepare(batch, dims, meta_d, x_in, x_out, ws, ws_bytes, MTFM_OP_FULL, &c, stream));
  TRY(check_full_w(w, dims));
  c.write_a = true;
  return run_full(c, dims, w, x_in, x_out, (char*)ws);
}

mtfm_status mtfm_attn_target(const mtfm_batch* batch, const mtfm_dims* dims, const void* meta_d,
                             const mtfm_target_w* w, const void* x_in, void* x_out, void* ws, size_t ws_bytes,
                             void* stream) {
  Ctx c;
  TRY(prepare(batch, dims, meta_d, x_in, x_out, ws, ws_bytes, MTFM_OP_TARGET, &c, stream));
  TRY(check_target_w(w, dims));
  c.write_a = true;
  return run_target(c, dims, w, x_in, x_out, (char*)ws);
}

mtfm_status mtfm_backbone_fwd(const mtfm_batch* batch, const mtfm_dims* dims, int32_t n_blocks, int32_t k_target,
                              const void* meta_d, const mtfm_full_w* full, const mtfm_target_w* tgt,
                              void* x_inout, void* ws, size_t ws_bytes, void* stream) {
  Ctx c;
  TRY(prepare(batch, dims, meta_d, x_inout, x_inout, ws, ws_bytes, MTFM_OP_BACKBONE, &c, stream));
  if (n_blocks < 0 || k_target < 0) return MTFM_E_DIMS;
  if (n_blocks > 0 && !full) return MTFM_E_NULL;
  if (n_blocks > 0 && k_target > 0 && !tgt) return MTFM_E_NULL;
  for (int b = 0; b < n_blocks; ++b) {
    TRY(check_full_w(&full[b], dims));
    for (int t = 0; t < k_target; ++t) TRY(check_target_w(&tgt[b * k_target + t], dims));
  }
  const bool hoist = dims->dtype == MTFM_BF16 && k_target >= 1 && k_target <= 4 &&
                     ws_bytes >= (size_t)backbone_ws(c.plan, dims, k_target).total;
  if (hoist) {
    const BackboneWs L = backbone_ws(c.plan, dims, k_target);
    char* w = (char*)ws;
    for (int b = 0; b < n_blocks; ++b) {
      TRY(run_full(c, dims, &full[b], x_inout, x_inout, w + L.full));
      const mtfm_target_w* tw = &tgt[b * k_target];
      if (c.plan.n_t_rows == 0) continue;   // target layers change T rows only
      TRY(run_target_context(c, dims, tw, k_target, x_inout, w, L));
      for (int t = 0; t < k_target; ++t) TRY(run_target_rows(c, dims, &tw[t], x_inout, w, L, t));
    }
    return MTFM_OK;
  }
  for (int b = 0; b < n_blocks; ++b) {
    TRY(run_full(c, dims, &full[b], x_inout, x_inout, (char*)ws));
    for (int t = 0; t < k_target; ++t) TRY(run_target(c, dims, &tgt[b * k_target + t], x_inout, x_inout, (char*)ws));
  }
  return MTFM_OK;
}

size_t mtfm_backbone_workspace_bytes(const mtfm_batch* batch, const mtfm_dims* dims, int32_t k_target) {
  MetaPlan p;
  if (k_target < 0 || plan_meta(batch, &p) != MTFM_OK || check_dims(dims) != MTFM_OK) return 0;
  const size_t base = mtfm_workspace_bytes(batch, dims, MTFM_OP_BACKBONE);
  if (dims->dtype != MTFM_BF16 || k_target < 1 || k_target > 4) return base;
  return std::max(base, (size_t)backbone_ws(p, dims, k_target).total);
}

mtfm_status mtfm_attn_full_bwd(const mtfm_batch* batch, const mtfm_dims* dims, const void* meta_d,
                               const mtfm_full_w* w, const void* x_in, const void* dy, void* dx,
                               const mtfm_full_grad* g, void* ws, size_t ws_bytes, void* stream) {
  Ctx c;
  TRY(prepare(batch, dims, meta_d, x_in, dx, ws, ws_bytes, MTFM_OP_FULL_BWD, &c, stream));
  TRY(check_full_w(w));
  if (!dy || !g || !g->ln1_g || !g->ln1_b || !g->w_uqkv || !g->ln2_g || !g->ln2_b || !g->w_o) return MTFM_E_NULL;
  if (dx == x_in || dx == dy) return MTFM_E_DIMS;
  return run_full_bwd(c, dims, w, x_in, dy, dx, g, (char*)ws);
}

mtfm_status mtfm_attn_target_bwd(const mtfm_batch* batch, const mtfm_dims* dims, const void* meta_d,
                                 const mtfm_target_w* w, const void* x_in, const void* dy, void* dx,
                                 const mtfm_target_grad* g, void* ws, size_t ws_bytes, void* stream) {
  Ctx c;
  TRY(prepare(batch, dims, meta_d, x_in, dx, ws, ws_bytes, MTFM_OP_TARGET_BWD, &c, stream));
  TRY(check_target_w(w));
  if (!dy || !g || !g->ln1_g || !g->ln1_b || !g->w_u || !g->w_q || !g->w_kv || !g->ln2_g || !g->ln2_b || !g->w_o)
    return MTFM_E_NULL;
  if (dx == x_in || dx == dy) return MTFM_E_DIMS;
  return run_target_bwd(c, dims, w, x_in, dy, dx, g, (char*)ws);
}

// ---------------------------------------------------------------------------


size_t mtfm_backbone_bwd_workspace_bytes(const mtfm_batch* batch, const mtfm_dims* dims, int32_t n_blocks,
                                         int32_t k_target) {
  MetaPlan p;
  if (n_blocks < 0 || k_target < 0 || plan_meta(batch, &p) != MTFM_OK || check_dims(dims) != MTFM_OK) return 0;
  if (bwd_ws_bytes(p, dims, MTFM_OP_FULL_BWD) == 0) return 0;   // shapes the backward does not support
  return (size_t)backbone_bwd_ws(p, dims, n_blocks, k_target).total;
}

size_t mtfm_backbone_bwd_min_workspace_bytes(const mtfm_batch* batch, const mtfm_dims* dims, int32_t n_blocks,
                                             int32_t k_target) {
  MetaPlan p;
  if (n_blocks < 0 || k_target < 0 || plan_meta(batch, &p) != MTFM_OK || check_dims(dims) != MTFM_OK) return 0;
  if (bwd_ws_bytes(p, dims, MTFM_OP_FULL_BWD) == 0) return 0;
  return (size_t)backbone_bwd_ws(p, dims, n_blocks, k_target).keep;
}

mtfm_status mtfm_backbone_bwd(const mtfm_batch* batch, const mtfm_dims* dims, int32_t n_blocks, int32_t k_target,
                              const void* meta_d, const mtfm_full_w* full, const mtfm_target_w* tgt,
                              const void* x_in, const void* dy, void* dx, const mtfm_full_grad* full_g,
                              const mtfm_target_grad* tgt_g, void* ws, size_t ws_bytes, void* stream) {
  if (n_blocks < 0 || k_target < 0) return MTFM_E_DIMS;
  Ctx c;
  TRY(plan_meta(batch, &c.plan));
  TRY(check_dims(dims));
  if (!meta_d || !x_in || !dy || !dx) return MTFM_E_NULL;
  if (dx == x_in || dx == dy) return MTFM_E_DIMS;
  TRY(check_batch_device(batch, c.plan));
  if (bwd_ws_bytes(c.plan, dims, MTFM_OP_FULL_BWD) == 0) return MTFM_E_UNSUPPORTED;
  if (n_blocks > 0 && (!full || !full_g)) return MTFM_E_NULL;
  if (n_blocks > 0 && k_target > 0 && (!tgt || !tgt_g)) return MTFM_E_NULL;
  for (int b = 0; b < n_blocks; ++b) {
    TRY(check_full_w(&full[b]));
    const mtfm_full_grad& g = full_g[b];
    if (!g.ln1_g || !g.ln1_b || !g.w_uqkv || !g.ln2_g || !g.ln2_b || !g.w_o) return MTFM_E_NULL;
    for (int t = 0; t < k_target; ++t) {
      TRY(check_target_w(&tgt[b * k_target + t]));
      const mtfm_target_grad& h = tgt_g[b * k_target + t];
      if (!h.ln1_g || !h.ln1_b || !h.w_u || !h.w_q || !h.w_kv || !h.ln2_g || !h.ln2_b || !h.w_o) return MTFM_E_NULL;
    }
  }
  const int L = n_blocks * (1 + k_target);
  const BackboneBwdWs W = backbone_bwd_ws(c.plan, dims, n_blocks, k_target);
  if (W.keep > 0 && !ws) return MTFM_E_NULL;
  if (ws_bytes < (size_t)W.keep) return MTFM_E_WORKSPACE;
  const bool keep_mode = ws_bytes >= (size_t)W.total;
  c.b = batch;
  c.meta = meta_ptrs(c.plan, meta_d);
  c.s = (hipStream_t)stream;
  char* w = (char*)ws;
  const size_t xb = (size_t)c.plan.n_rows * dims->d_model * elem_size(dims->dtype);
  if (L == 0) {   // the empty stack is the identity
    if (xb == 0) return MTFM_OK;
    const hipError_t e = hipMemcpyAsync(dx, dy, xb, hipMemcpyDeviceToDevice, c.s);
    return e == hipSuccess ? MTFM_OK : hip_fail(e, "hipMemcpyAsync");
  }
  const int per = 1 + k_target;
  auto input_of = [&](int l) -> const void* { return l == 0 ? x_in : (const void*)(w + W.stash + (l - 1) * W.xbytes); };
  // gradient buffers alternate so that layer 0 writes dx
  auto grad_buf = [&](int l) -> void* { return (l % 2 == 0) ? dx : (void*)(w + W.gbuf); };
  // intermediates of layer l kept by the forward pass (keep mode; none for the
  // last layer, whose forward is not run here: its backward recomputes them)
  FwdKeep kl;
  auto keep_of = [&](int l) -> const FwdKeep* {
    if (!keep_mode || l + 1 >= L) return nullptr;
    kl = W.keep_of(w, l);
    return &kl;
  };
  for (int l = 0; l + 1 < L; ++l) {
    void* out = w + W.stash + l * W.xbytes;
    const int b = l / per, t = l % per;
    // the training pass computes with the dense weights (packed sparse ones are inference-only)
    if (t == 0) {
      mtfm_full_w fw = full[b];
      fw.w_uqkv_s24 = fw.w_o_s24 = nullptr;
      TRY(run_full(c, dims, &fw, input_of(l), out, w + W.layer, nullptr, keep_of(l)));
    } else {
      mtfm_target_w tw = tgt[b * k_target + t - 1];
      tw.w_t_s24 = tw.w_kv_s24 = tw.w_o_s24 = nullptr;
      TRY(run_target(c, dims, &tw, input_of(l), out, w + W.layer, keep_of(l)));
    }
  }
  for (int l = L - 1; l >= 0; --l) {
    const void* g_in = l == L - 1 ? dy : grad_buf(l + 1);
    void* g_out = grad_buf(l);
    const int b = l / per, t = l % per;
    if (t == 0) TRY(run_full_bwd(c, dims, &full[b], input_of(l), g_in, g_out, &full_g[b], w + W.layer, keep_of(l)));
    else TRY(run_target_bwd(c, dims, &tgt[b * k_target + t - 1], input_of(l), g_in, g_out,
                            &tgt_g[b * k_target + t - 1], w + W.layer, keep_of(l)));
  }
  return MTFM_OK;
}

mtfm_status mtfm_autosplit(const mtfm_batch* batch, const mtfm_dims* dims, int32_t d_in, const void* meta_d,
                           const void* feats, const void* w_split, void* x, void* stream) {
  Ctx c;
  TRY(v2_checks(batch, dims, meta_d, &c));
  c.s = (hipStream_t)stream;
  if (d_in <= 0 || d_in % 32 != 0) return MTFM_E_UNSUPPORTED;
  if (c.plan.n_parents == 0) return MTFM_OK;
  if (!feats || !w_split || !x) return MTFM_E_NULL;
  GemmArgs g{};
  g.M = (int32_t)c.plan.n_parents; g.N = c.plan.split * dims->d_model; g.K = d_in; g.groups = 1;
  g.A = feats; g.lda = d_in; g.amap = identity_map();
  g.B[0] = w_split; g.bn[0] = g.N; g.ldb = d_in;
  // output row m = parent m's S sub-token rows, contiguous in the packed matrix
  g.cmap = RowMap{c.meta.parent_row, 0, 0};
  g.epi = EPI_STORE; g.out = x; g.ldo = dims->d_model;
  return timed_gemm(MTFM_K_V2, g, MTFM_BF16, c.s);
}

size_t mtfm_token_ffn_workspace_bytes(const mtfm_batch* batch, const mtfm_dims* dims, int32_t d_ff) {
  MetaPlan p;
  if (d_ff <= 0 || plan_meta(batch, &p) != MTFM_OK || check_dims(dims) != MTFM_OK) return 0;
  return (size_t)ffn_ws(p, dims, d_ff).total;
}

mtfm_status mtfm_token_ffn(const mtfm_batch* batch, const mtfm_dims* dims, int32_t d_ff, const void* meta_d,
                           const mtfm_ffn_w* w, void* x, void* ws, size_t ws_bytes, void* stream) {
  Ctx c;
  TRY(v2_checks(batch, dims, meta_d, &c));
  c.s = (hipStream_t)stream;
  TRY(check_ffn(dims, d_ff, c.plan.split, w));
  const FfnWs L = ffn_ws(c.plan, dims, d_ff);
  if (c.plan.n_t_rows > 0 && (!x || !ws)) return MTFM_E_NULL;
  if (ws_bytes < (size_t)L.total) return MTFM_E_WORKSPACE;
  return run_token_ffn(c, dims, d_ff, w, x, (char*)ws, L);
}

mtfm_status mtfm_token_pool(const mtfm_batch* batch, const mtfm_dims* dims, const void* meta_d, const void* x,
                            void* out, void* stream) {
  Ctx c;
  TRY(v2_checks(batch, dims, meta_d, &c));
  c.s = (hipStream_t)stream;
  if (c.plan.n_parents == 0) return MTFM_OK;
  if (!x || !out) return MTFM_E_NULL;
  TokenRowsArgs a{};
  a.x = (bf16*)x; a.ldx = dims->d_model; a.parent_row = c.meta.parent_row; a.n_parents = (int32_t)c.plan.n_parents;
  a.S = c.plan.split; a.D = dims->d_model; a.out = (bf16*)out; a.ldo = dims->d_model;
  TimedLaunch t(MTFM_K_V2, c.s);
  return launch_token_pool(a, c.s);
}

size_t mtfm_backbone_v2_workspace_bytes(const mtfm_batch* batch, const mtfm_dims* dims, int32_t k_target,
                                        int32_t d_ff) {
  MetaPlan p;
  if (k_target < 1 || k_target > 4 || d_ff <= 0 || plan_meta(batch, &p) != MTFM_OK || check_dims(dims) != MTFM_OK)
    return 0;
  return (size_t)(align_up(backbone_ws(p, dims, k_target).total, 256) + ffn_ws(p, dims, d_ff).total);
}

mtfm_status mtfm_backbone_v2_fwd(const mtfm_batch* batch, const mtfm_dims* dims, int32_t n_blocks, int32_t k_target,
                                 int32_t d_ff, const void* meta_d, const mtfm_full_w* full, const mtfm_target_w* tgt,
                                 const mtfm_ffn_w* ffn, void* x_inout, void* ws, size_t ws_bytes, void* stream) {
  Ctx c;
  TRY(v2_checks(batch, dims, meta_d, &c));
  c.s = (hipStream_t)stream;
  if (n_blocks < 0) return MTFM_E_DIMS;
  if (k_target < 1 || k_target > 4) return MTFM_E_UNSUPPORTED;
  if (n_blocks > 0 && (!full || !tgt || !ffn)) return MTFM_E_NULL;
  for (int b = 0; b < n_blocks; ++b) {
    TRY(check_full_w(&full[b], dims));
    for (int t = 0; t < k_target; ++t) {
      TRY(check_target_w(&tgt[b * k_target + t], dims));
      TRY(check_ffn(dims, d_ff, c.plan.split, &ffn[b * k_target + t]));
    }
  }
  const BackboneWs L = backbone_ws(c.plan, dims, k_target);
  const int64_t foff = align_up(L.total, 256);
  const FfnWs F = ffn_ws(c.plan, dims, d_ff);
  if (c.plan.n_rows > 0 && (!x_inout || !ws)) return MTFM_E_NULL;
  if (ws_bytes < (size_t)(foff + F.total)) return MTFM_E_WORKSPACE;
  char* w = (char*)ws;
  for (int b = 0; b < n_blocks; ++b) {
    TRY(run_full(c, dims, &full[b], x_inout, x_inout, w + L.full));
    const mtfm_target_w* tw = &tgt[b * k_target];
    if (c.plan.n_t_rows == 0) continue;   // target layers and FFNs change T rows only
    TRY(run_target_context(c, dims, tw, k_target, x_inout, w, L));
    for (int t = 0; t < k_target; ++t) {
      TRY(run_target_rows(c, dims, &tw[t], x_inout, w, L, t));
      TRY(run_token_ffn(c, dims, d_ff, &ffn[b * k_target + t], x_inout, w + foff, F));
    }
  }
  return MTFM_OK;
}

size_t mtfm_kv_cache_bytes(const mtfm_batch* batch, const mtfm_dims* dims, int32_t n_blocks, int32_t k_target) {
  MetaPlan p;
  if (n_blocks < 0 || k_target < 0 || plan_meta(batch, &p) != MTFM_OK || check_dims(dims) != MTFM_OK) return 0;
  if (dims->dtype != MTFM_BF16) return 0;
  return (size_t)kv_cache_layout(p, dims, n_blocks * (1 + k_target)).total;
}

size_t mtfm_serve_workspace_bytes(const mtfm_batch* batch, const mtfm_dims* dims, int32_t k_target, int32_t phase) {
  MetaPlan p;
  if (k_target < 0 || k_target > 4 || plan_meta(batch, &p) != MTFM_OK || check_dims(dims) != MTFM_OK) return 0;
  if (dims->dtype != MTFM_BF16) return 0;
  if (phase == MTFM_SERVE_CONTEXT) return (size_t)backbone_ws(p, dims, k_target).total;
  if (phase == MTFM_SERVE_TARGETS) return (size_t)serve_ws(p, dims).total;
  return 0;
}

mtfm_status mtfm_serve_context(const mtfm_batch* batch, const mtfm_dims* dims, int32_t n_blocks, int32_t k_target,
                               const void* meta_d, const mtfm_full_w* full, const mtfm_target_w* tgt,
                               void* x_inout, void* kv_cache, size_t cache_bytes, void* ws, size_t ws_bytes,
                               void* stream) {
  Ctx c;
  TRY(serve_checks(batch, dims, n_blocks, k_target, meta_d, full, tgt, &c));
  c.s = (hipStream_t)stream;
  if (c.plan.n_t_rows != 0) {
    set_last_error("mtfm_serve_context: the context batch must hold no T rows");
    return MTFM_E_DIMS;
  }
  const KvCacheLayout K = kv_cache_layout(c.plan, dims, n_blocks * (1 + k_target));
  const BackboneWs L = backbone_ws(c.plan, dims, k_target);
  if (c.plan.n_rows > 0 && (!x_inout || !kv_cache || (L.total > 0 && !ws))) return MTFM_E_NULL;
  if (cache_bytes < (size_t)K.total || ws_bytes < (size_t)L.total) return MTFM_E_WORKSPACE;
  if (c.plan.n_rows == 0) return MTFM_OK;
  char* w = (char*)ws;
  char* cache = (char*)kv_cache;
  const int per = 1 + k_target;
  for (int b = 0; b < n_blocks; ++b) {
    const KvOut kf = kv_of(K, cache, b * per);
    TRY(run_full(c, dims, &full[b], x_inout, x_inout, w + L.full, &kf));
    if (k_target == 0) continue;
    KvOut kt[4];
    for (int t = 0; t < k_target; ++t) kt[t] = kv_of(K, cache, b * per + 1 + t);
    TRY(run_target_context(c, dims, &tgt[b * k_target], k_target, x_inout, w, L, kt));
  }
  return MTFM_OK;
}

mtfm_status mtfm_serve_targets(const mtfm_batch* batch, const mtfm_dims* dims, int32_t n_blocks, int32_t k_target,
                               const void* meta_d, const mtfm_full_w* full, const mtfm_target_w* tgt,
                               const void* kv_cache, size_t cache_bytes, void* x_t, void* ws, size_t ws_bytes,
                               void* stream) {
  Ctx c;
  TRY(serve_targets_check(batch, dims, n_blocks, k_target, meta_d, full, tgt, kv_cache, cache_bytes, x_t, &c));
  if (c.plan.n_t_rows > 0 && !ws) return MTFM_E_NULL;
  if (ws_bytes < (size_t)serve_ws(c.plan, dims).total) return MTFM_E_WORKSPACE;
  c.s = (hipStream_t)stream;
  return serve_targets_run(c, dims, n_blocks, k_target, full, tgt, kv_cache, x_t, (char*)ws);
}

const char* mtfm_status_str(int32_t status) {
  switch (status) {
    case MTFM_OK: return "MTFM_OK";
    case MTFM_E_NULL: return "MTFM_E_NULL";
    case MTFM_E_DIMS: return "MTFM_E_DIMS";
    case MTFM_E_UNSUPPORTED: return "MTFM_E_UNSUPPORTED";
    case MTFM_E_WORKSPACE: return "MTFM_E_WORKSPACE";
    case MTFM_E_HIP: return "MTFM_E_HIP";
    default: return "MTFM_E_UNKNOWN";
  }
}

const char* mtfm_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
