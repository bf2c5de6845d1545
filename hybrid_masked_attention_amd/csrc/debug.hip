// Debug entry points: the dense visibility mask of one user from the
// metadata, and a device-side check of the batch's data-level contracts.
// Neither is on the hot path.

#include <algorithm>

#include "common.h"

namespace {

// Visibility of (query i, key j) inside one user, from its rows' metadata:
// context keys j < lctx are visible iff j < p_i (the visible context is a
// prefix); a T key (j >= lctx) is visible only to itself, when self_i = 1.
__global__ __launch_bounds__(256) void mask_dense_kernel(const int32_t* p, const int32_t* n, int64_t row0, int N,
                                                         int lctx, uint8_t* out) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)N * N) return;
  const int i = (int)(idx / N), j = (int)(idx % N);
  const int pi = p[row0 + i], self = n[row0 + i] - pi;
  const bool vis = j < lctx ? j < pi : (j == i && self > 0);
  out[idx] = vis ? 1 : 0;
}

// Order-sensitive mix of one user's lengths (the host computes the same sum).
__host__ __device__ inline uint32_t lens_mix(uint32_t u, uint32_t lh, uint32_t lr, uint32_t lt) {
  uint32_t x = lh * 0x9E3779B1u + lr * 0x85EBCA77u + lt * 0xC2B2AE3Du + u * 0x27D4EB2Fu;
  x ^= x >> 15;
  x *= 0x2C1B3C6Du;
  x ^= x >> 12;
  return x;
}

// One workgroup walks the users in chunks of 256: a scan of the device R
// lengths gives each user's action range (clamped to the host total, so bad
// lengths never move a read out of the array), whose times must ascend.
__global__ __launch_bounds__(256) void validate_kernel(const int32_t* lens, int32_t n_users, const int32_t* ts_r,
                                                       int64_t total_r, uint32_t hash_host, int32_t* flags) {
  __shared__ int64_t scan[256];
  __shared__ uint32_t hsum;
  __shared__ int32_t bad;
  __shared__ int64_t base;
  const int tid = threadIdx.x;
  if (tid == 0) { hsum = 0; bad = 0; base = 0; }
  __syncthreads();
  uint32_t h = 0;
  for (int c = 0; c < n_users; c += 256) {
    const int u = c + tid;
    int32_t lh = 0, lr = 0, lt = 0;
    if (u < n_users) {
      lh = lens[3 * u]; lr = lens[3 * u + 1]; lt = lens[3 * u + 2];
      if (lh < 0 || lr < 0 || lt < 0) atomicOr(&bad, MTFM_BAD_LENGTHS);
      h += lens_mix((uint32_t)u, (uint32_t)lh, (uint32_t)lr, (uint32_t)lt);
    }
    const int64_t mine = max(lr, 0);
    scan[tid] = mine;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {   // inclusive scan
      const int64_t add = tid >= off ? scan[tid - off] : 0;
      __syncthreads();
      scan[tid] += add;
      __syncthreads();
    }
    const int64_t r1 = base + scan[tid], r0 = r1 - mine;
    const int64_t a = min(max(r0, (int64_t)0), total_r), b = min(max(r1, (int64_t)0), total_r);
    for (int64_t k = a + 1; k < b; ++k)
      if (ts_r[k - 1] > ts_r[k]) { atomicOr(&bad, MTFM_BAD_ACTION_ORDER); break; }
    __syncthreads();
    if (tid == 255) base += scan[255];
    __syncthreads();
  }
  atomicAdd(&hsum, h);
  __syncthreads();
  if (tid == 0) {
    int32_t f = bad;
    if (hsum != hash_host || base != total_r) f |= MTFM_BAD_LENGTHS;
    *flags = f;
  }
}

}  // namespace

extern "C" {

mtfm_status mtfm_mask_dense(const mtfm_batch* batch, const void* meta_d, int32_t user, uint8_t* mask_d,
                            void* stream) {
  MetaPlan p;
  const mtfm_status st = plan_meta(batch, &p);
  if (st != MTFM_OK) return st;
  if (user < 0 || user >= p.n_users) return MTFM_E_DIMS;
  int64_t row0 = 0;
  for (int u = 0; u < user; ++u)
    row0 += batch->lens_h[3 * u] + batch->lens_h[3 * u + 1] + (int64_t)p.split * batch->lens_h[3 * u + 2];
  const int lctx = batch->lens_h[3 * user] + batch->lens_h[3 * user + 1];
  const int64_t N = lctx + (int64_t)p.split * batch->lens_h[3 * user + 2];
  if (N == 0) return MTFM_OK;
  if (!meta_d || !mask_d) return MTFM_E_NULL;
  if (N * N > ((int64_t)1 << 31) * 256) return MTFM_E_DIMS;
  const MetaPtrs m = meta_ptrs(p, meta_d);
  mask_dense_kernel<<<(unsigned)((N * N + 255) / 256), 256, 0, (hipStream_t)stream>>>(m.p, m.n, row0, (int)N, lctx,
                                                                                      mask_d);
  MTFM_LAUNCH_CHECK("mask_dense");
  return MTFM_OK;
}

mtfm_status mtfm_validate_batch(const mtfm_batch* batch, int32_t* flags_d, void* stream) {
  MetaPlan p;
  const mtfm_status st = plan_meta(batch, &p);
  if (st != MTFM_OK) return st;
  if (!flags_d) return MTFM_E_NULL;
  if (p.n_users > 0 && !batch->lens_d) return MTFM_E_NULL;
  int64_t total_r = 0;
  uint32_t hash = 0;
  for (int u = 0; u < p.n_users; ++u) {
    total_r += batch->lens_h[3 * u + 1];
    hash += lens_mix((uint32_t)u, (uint32_t)batch->lens_h[3 * u], (uint32_t)batch->lens_h[3 * u + 1],
                     (uint32_t)batch->lens_h[3 * u + 2]);
  }
  if (total_r > 0 && !batch->ts_r_d) return MTFM_E_NULL;
  validate_kernel<<<1, 256, 0, (hipStream_t)stream>>>(batch->lens_d, p.n_users, batch->ts_r_d, total_r, hash,
                                                      flags_d);
  MTFM_LAUNCH_CHECK("validate_batch");
  return MTFM_OK;
}

}  // extern "C"
