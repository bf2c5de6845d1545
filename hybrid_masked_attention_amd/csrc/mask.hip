// Mask-metadata builder: token types and timestamps -> per-row visible
// prefixes and per-tile skip lists.
//
// The dynamic mask ([explainer] §4.1.1, worked matrix in §8.2; [blog] §3.2)
// makes every row's visible context (H then R columns) a prefix [0, p_i):
//   H row: p = L_H;  R row j: p = L_H + j + 1 (causal, self included);
//   T row of parent t: p = L_H + #{R actions with time < e_t}, plus itself.
// Because the actions are sorted by time, the count is a lower-bound binary
// search.  [blog] §6.1 stores the mask preprocessed as a one-dimensional
// jagged array and §6.2 pre-scans it into the list of key blocks that hold
// any visible key; here those are p_i / n_i per row and, per 64-row query
// tile, the number of leading fully visible key tiles and the end of the
// visible key tiles (a min / max of p over the tile's rows).
//
// Integer-only: results are bit-exact by construction.

#include "common.h"

namespace {

constexpr int kScanThreads = 1024;

// Per-user quantities whose exclusive prefix sums form the user table.
MTFM_DEV void user_counts(const int32_t* lens, int u, int split, int32_t out[UT_COUNT]) {
  const int lh = lens[3 * u], lr = lens[3 * u + 1], lt = lens[3 * u + 2];
  const int rows = lh + lr + split * lt;
  out[UT_ROW] = rows;
  out[UT_ACT] = lr;
  out[UT_PARENT] = lt;
  out[UT_CTX] = lh + lr;
  out[UT_FTILE] = (rows + kTile - 1) / kTile;
  out[UT_TTILE] = (split * lt + kTile - 1) / kTile;
  out[UT_TROW] = split * lt;
  out[UT_KTILE] = (lh + lr + kTile - 1) / kTile;
}

// One workgroup: exclusive prefix sums of the per-user counts.
__global__ __launch_bounds__(kScanThreads) void user_scan_kernel(const int32_t* __restrict__ lens, int n_users,
                                                                  int split, int32_t* __restrict__ table) {
  __shared__ int32_t part[UT_COUNT][kScanThreads];
  const int t = threadIdx.x;
  const int chunk = (n_users + kScanThreads - 1) / kScanThreads;
  const int u0 = min(t * chunk, n_users), u1 = min(u0 + chunk, n_users);
  int32_t sum[UT_COUNT] = {};
  for (int u = u0; u < u1; ++u) {
    int32_t c[UT_COUNT];
    user_counts(lens, u, split, c);
    for (int k = 0; k < UT_COUNT; ++k) sum[k] += c[k];
  }
  for (int k = 0; k < UT_COUNT; ++k) part[k][t] = sum[k];
  __syncthreads();
  // exclusive scan of part[k][0..1024) by the first UT_COUNT waves, one table row each
  const int wave = t >> 6, lane = t & 63;
  if (wave < UT_COUNT) {
    int32_t* row = part[wave];
    int32_t acc = 0;
    for (int i = 0; i < kScanThreads / 64; ++i) acc += row[lane * (kScanThreads / 64) + i];
    int32_t incl = acc;
    for (int o = 1; o < 64; o <<= 1) {
      int32_t v = __shfl_up(incl, o, 64);
      if (lane >= o) incl += v;
    }
    int32_t run = incl - acc;
    for (int i = 0; i < kScanThreads / 64; ++i) {
      int32_t v = row[lane * (kScanThreads / 64) + i];
      row[lane * (kScanThreads / 64) + i] = run;
      run += v;
    }
    if (lane == 63) table[wave * (n_users + 1) + n_users] = incl;
  }
  __syncthreads();
  for (int k = 0; k < UT_COUNT; ++k) {
    int32_t run = part[k][t];
    for (int u = u0; u < u1; ++u) {
      int32_t c[UT_COUNT];
      user_counts(lens, u, split, c);
      table[k * (n_users + 1) + u] = run;
      run += c[k];
    }
  }
}

// Number of entries of the ascending array a[0, n) that are < x.
MTFM_DEV int lower_bound(const int32_t* a, int n, int x) {
  int lo = 0, hi = n;
  while (lo < hi) {
    int mid = (lo + hi) >> 1;
    if (a[mid] < x) lo = mid + 1; else hi = mid;
  }
  return lo;
}

MTFM_DEV void tile_bounds(int pmin, int pmax, int l_ctx, int* full_end, int* end) {
  const int nkt = (l_ctx + kTile - 1) / kTile;
  *full_end = (pmin >= l_ctx) ? nkt : pmin / kTile;
  *end = (pmax + kTile - 1) / kTile;
}

// One wave per full-layer query tile: per-row metadata, row lists, tile descriptor.
__global__ __launch_bounds__(64) void rows_full_tiles_kernel(const int32_t* __restrict__ lens, int n_users, int split,
                                                             const int32_t* __restrict__ ts_r,
                                                             const int32_t* __restrict__ ts_t,
                                                             const int32_t* __restrict__ table,
                                                             int32_t* __restrict__ p_out, int32_t* __restrict__ n_out,
                                                             uint8_t* __restrict__ type_out,
                                                             int32_t* __restrict__ tiles,
                                                             int32_t* __restrict__ ctx_rows,
                                                             int32_t* __restrict__ parent_row) {
  const int stride = n_users + 1;
  const int b = blockIdx.x;
  const int u = upper_index(table + UT_FTILE * stride, n_users, b);
  const int a = b - table[UT_FTILE * stride + u];
  const int lh = lens[3 * u], lr = lens[3 * u + 1], lt = lens[3 * u + 2];
  const int lc = lh + lr, rows = lc + split * lt;
  const int row0 = table[UT_ROW * stride + u];
  const int r = a * kTile + threadIdx.x;
  int pmin = INT32_MAX, pmax = 0;
  if (r < rows) {
    const int g = row0 + r;
    int p, self, type;
    if (r < lh) {
      type = TT_H; p = lh; self = 0;
    } else if (r < lc) {
      type = TT_R; p = r + 1; self = 0;
    } else {
      type = TT_T; self = 1;
      const int j = (r - lc) / split;
      const int pidx = table[UT_PARENT * stride + u] + j;
      const int e = ts_t[pidx];
      p = lh + lower_bound(ts_r + table[UT_ACT * stride + u], lr, e);
      if ((r - lc) % split == 0) parent_row[pidx] = g;
    }
    if (r < lc) ctx_rows[table[UT_CTX * stride + u] + r] = g;
    p_out[g] = p;
    n_out[g] = p + self;
    type_out[g] = (uint8_t)type;
    pmin = p; pmax = p;
  }
  pmin = wave_min(pmin);
  pmax = wave_max(pmax);
  if (threadIdx.x == 0) {
    int fe, e;
    tile_bounds(pmin, pmax, lc, &fe, &e);
    int32_t* d = tiles + 8 * b;
    d[TD_USER] = u; d[TD_ROW0] = a * kTile; d[TD_NROWS] = min(kTile, rows - a * kTile);
    d[TD_FULL_END] = fe; d[TD_END] = e;
    d[TD_GROW0] = row0 + a * kTile; d[TD_QROW0] = row0 + a * kTile; d[TD_UROW0] = row0;
  }
}

// One workgroup per user: its T rows in ascending order of the visible prefix
// p (ties by row; a parent's S sub-tokens share p and stay together), by
// counting.  Only the order of the query rows changes, which no row's result
// depends on; the target tiles over this order cut fewer key tiles (rows of
// similar p share a slice).  Users with more than kTSortMaxRows T rows keep
// their own order.
__global__ __launch_bounds__(256) void tsort_kernel(const int32_t* __restrict__ lens, int n_users, int split,
                                                     const int32_t* __restrict__ table,
                                                     const int32_t* __restrict__ p_in, int32_t* __restrict__ tsq,
                                                     int32_t* __restrict__ tsg) {
  __shared__ int32_t ps[kTSortMaxRows];   // the user's prefixes, read from LDS by every comparison
  const int stride = n_users + 1;
  const int u = blockIdx.x;
  const int lc = lens[3 * u] + lens[3 * u + 1], nt = split * lens[3 * u + 2];
  const int g0 = table[UT_ROW * stride + u] + lc, t0 = table[UT_TROW * stride + u];
  const bool sort = nt <= kTSortMaxRows;   // the same for the whole workgroup
  if (sort) {
    for (int i = threadIdx.x; i < nt; i += blockDim.x) ps[i] = p_in[g0 + i];
    __syncthreads();
  }
  for (int i = threadIdx.x; i < nt; i += blockDim.x) {
    int rank = i;
    if (sort) {
      const int pi = ps[i];
      rank = 0;
      for (int j = 0; j < nt; ++j) {
        const int pj = ps[j];
        rank += (pj < pi) || (pj == pi && j < i);
      }
    }
    tsq[t0 + rank] = t0 + i;
    tsg[t0 + rank] = g0 + i;
  }
}

// One wave per target-layer query tile (T rows only); reads p written above.
// With tsg, the tile's rows are the positions of the sorted order (tsg gives
// their packed rows) and its query-row fields hold the position.
__global__ __launch_bounds__(64) void target_tiles_kernel(const int32_t* __restrict__ lens, int n_users, int split,
                                                          const int32_t* __restrict__ table,
                                                          const int32_t* __restrict__ p_in,
                                                          const int32_t* __restrict__ tsg,
                                                          int32_t* __restrict__ tiles) {
  const int stride = n_users + 1;
  const int b = blockIdx.x;
  const int u = upper_index(table + UT_TTILE * stride, n_users, b);
  const int a = b - table[UT_TTILE * stride + u];
  const int lh = lens[3 * u], lr = lens[3 * u + 1], lt = lens[3 * u + 2];
  const int lc = lh + lr, nt = split * lt;
  const int row0 = table[UT_ROW * stride + u];
  const int rt = a * kTile + threadIdx.x;
  int pmin = INT32_MAX, pmax = 0;
  if (rt < nt) {
    const int p = p_in[tsg ? tsg[table[UT_TROW * stride + u] + rt] : row0 + lc + rt];
    pmin = p; pmax = p;
  }
  pmin = wave_min(pmin);
  pmax = wave_max(pmax);
  if (threadIdx.x == 0) {
    int fe, e;
    tile_bounds(pmin, pmax, lc, &fe, &e);
    int32_t* d = tiles + 8 * b;
    d[TD_USER] = u; d[TD_ROW0] = lc + a * kTile; d[TD_NROWS] = min(kTile, nt - a * kTile);
    d[TD_FULL_END] = fe; d[TD_END] = e;
    d[TD_GROW0] = row0 + lc + a * kTile;
    d[TD_QROW0] = table[UT_TROW * stride + u] + a * kTile;
    d[TD_UROW0] = row0;
  }
}

// One workgroup: the attention work order of both layers (ranking, dealing
// to the XCDs and the per-XCD lists as described with order_xcd).  Users are
// ranked by counting, O(n^2) over at most kOrderMaxUsers users in LDS, with
// the workgroup's threads split over (user, share of the other users) pairs.
// Every entry of an order array is written once: a slice id or, past the end
// of its XCD's list, -1.
__global__ __launch_bounds__(kScanThreads) void work_order_kernel(const int32_t* __restrict__ lens, int n_users,
                                                                  int split, const int32_t* __restrict__ table,
                                                                  int32_t* __restrict__ order_full, int n_full,
                                                                  int32_t* __restrict__ order_target, int n_target) {
  __shared__ int64_t work[kOrderMaxUsers];
  __shared__ int32_t rank[kOrderMaxUsers];
  __shared__ int32_t off[kOrderMaxUsers];
  __shared__ int32_t nsl[kOrderMaxUsers];
  __shared__ int32_t count[8];
  const int t = threadIdx.x, n = n_users, stride = n_users + 1;
  const int P = n > 0 && n < kScanThreads ? kScanThreads / n : 1;   // threads per user
  for (int layer = OL_FULL; layer <= OL_TARGET; ++layer) {
    int32_t* order = layer == OL_FULL ? order_full : order_target;
    const int len = layer == OL_FULL ? n_full : n_target;
    if (len == 0) continue;
    for (int u = t; u < n; u += kScanThreads) {
      work[u] = order_user_work(lens, u, split, layer);
      nsl[u] = order_slices(lens, u, split, layer);
      rank[u] = 0;
      off[u] = 0;
    }
    if (t < 8) count[t] = 0;
    __syncthreads();
    for (int i = t; i < n * P; i += kScanThreads) {
      const int u = i / P, j = i % P;
      const int64_t wu = work[u];
      int r = 0;
      for (int v = j; v < n; v += P) r += (work[v] > wu) || (work[v] == wu && v < u);
      atomicAdd(&rank[u], r);
    }
    __syncthreads();
    for (int i = t; i < n * P; i += kScanThreads) {
      const int u = i / P, j = i % P;
      const int ru = rank[u], x = order_xcd(ru);
      int o = 0;   // slices of the users dealt to XCD x ahead of u
      for (int v = j; v < n; v += P) o += (order_xcd(rank[v]) == x && rank[v] < ru) ? nsl[v] : 0;
      atomicAdd(&off[u], o);
      if (j == 0) atomicAdd(&count[x], nsl[u]);
    }
    __syncthreads();
    const int32_t* first_tile = table + (layer == OL_FULL ? UT_FTILE : UT_TTILE) * stride;
    for (int i = t; i < n * P; i += kScanThreads) {
      const int u = i / P, j = i % P;
      const int x = order_xcd(rank[u]), ns = nsl[u], o = off[u], sid0 = 2 * first_tile[u];
      for (int k = j; k < ns; k += P) {
        const int e = 8 * (o + k) + x;
        MTFM_DCHECK_LANE(e < len, "work order entry within the planned length");
        if (e < len) order[e] = sid0 + ns - 1 - k;
      }
    }
    for (int e = t; e < len; e += kScanThreads)
      if ((e >> 3) >= count[e & 7]) order[e] = -1;
    __syncthreads();   // LDS is reused by the next layer
  }
}

}  // namespace

mtfm_status launch_mask_build(const mtfm_batch* b, const MetaPlan& plan, void* meta_d, hipStream_t s) {
  char* base = static_cast<char*>(meta_d);
  int32_t* table = reinterpret_cast<int32_t*>(base + plan.lay.off_user);
  int32_t* p = reinterpret_cast<int32_t*>(base + plan.lay.off_p);
  int32_t* n = reinterpret_cast<int32_t*>(base + plan.lay.off_n);
  uint8_t* type = reinterpret_cast<uint8_t*>(base + plan.lay.off_type);
  int32_t* ft = reinterpret_cast<int32_t*>(base + plan.lay.off_full_tiles);
  int32_t* tt = reinterpret_cast<int32_t*>(base + plan.lay.off_target_tiles);
  int32_t* ctx = reinterpret_cast<int32_t*>(base + plan.lay.off_ctx_rows);
  int32_t* par = reinterpret_cast<int32_t*>(base + plan.lay.off_parent_row);

  user_scan_kernel<<<1, kScanThreads, 0, s>>>(b->lens_d, plan.n_users, plan.split, table);
  MTFM_LAUNCH_CHECK("user_scan_kernel");
  if (plan.n_full_tiles > 0) {
    rows_full_tiles_kernel<<<(unsigned)plan.n_full_tiles, 64, 0, s>>>(b->lens_d, plan.n_users, plan.split, b->ts_r_d,
                                                                      b->ts_t_d, table, p, n, type, ft, ctx, par);
    MTFM_LAUNCH_CHECK("rows_full_tiles_kernel");
  }
  if (plan.n_full_order > 0 || plan.n_target_order > 0) {
    work_order_kernel<<<1, kScanThreads, 0, s>>>(
        b->lens_d, plan.n_users, plan.split, table, reinterpret_cast<int32_t*>(base + plan.lay.off_full_order),
        (int)plan.n_full_order, reinterpret_cast<int32_t*>(base + plan.lay.off_target_order),
        (int)plan.n_target_order);
    MTFM_LAUNCH_CHECK("work_order_kernel");
  }
  if (plan.n_target_tiles > 0) {
    int32_t* tsq = reinterpret_cast<int32_t*>(base + plan.lay.off_tsort_q);
    int32_t* tsg = reinterpret_cast<int32_t*>(base + plan.lay.off_tsort_g);
    int32_t* tts = reinterpret_cast<int32_t*>(base + plan.lay.off_target_tiles_sorted);
    target_tiles_kernel<<<(unsigned)plan.n_target_tiles, 64, 0, s>>>(b->lens_d, plan.n_users, plan.split, table, p,
                                                                       nullptr, tt);
    MTFM_LAUNCH_CHECK("target_tiles_kernel");
    tsort_kernel<<<(unsigned)plan.n_users, 256, 0, s>>>(b->lens_d, plan.n_users, plan.split, table, p, tsq, tsg);
    MTFM_LAUNCH_CHECK("tsort_kernel");
    target_tiles_kernel<<<(unsigned)plan.n_target_tiles, 64, 0, s>>>(b->lens_d, plan.n_users, plan.split, table, p,
                                                                       tsg, tts);
    MTFM_LAUNCH_CHECK("target_tiles_kernel (sorted)");
  }
  return MTFM_OK;
}
