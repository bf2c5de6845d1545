// 2:4 structured pruning and packing of projection weights ([explainer]
// §5.2.1: of every 4 consecutive weights the 2 smaller are set to zero, so
// that sparse matrix hardware can skip them).
//
// Groups of 4 run along a weight row (the reduction axis of y = x W^T).  A
// group keeps its two entries of largest magnitude; of equal magnitudes the
// lower position is kept.  The kept values are laid out in the lane order of
// gfx950's v_smfmac_f32_32x32x32_bf16 sparse operand, so the sparse GEMM loads
// them with one 16-byte and one 2-byte load per lane and K step:
//
//   rows R (the stacked segments, in order), K % 32 == 0, K step ks = k / 32;
//   slice (ks, r, h), h = 0, 1, index i = (ks * R + r) * 2 + h, covers the
//   groups q of row r's K step ks with q % 4 in {0, 1} (h = 0) or {2, 3}
//   (h = 1), in ascending q: groups 2h, 2h + 1, 2h + 4, 2h + 5;
//   values at byte i * 16: per group (slot pair j = 0..3) its two kept
//           entries in ascending position;
//   indexes at byte R * K + i * 2: bits 4 j .. 4 j + 1 and 4 j + 2 .. 4 j + 3
//           hold the positions (0..3) within group j of the two kept entries.

#include "common.h"

namespace {

constexpr int kMaxSegs = 16;

struct PackArgs {
  const bf16* seg[kMaxSegs];
  int32_t seg_rows[kMaxSegs];
  int32_t n_segs, rows, K;
  char* out;
};

__global__ __launch_bounds__(256) void s24_pack_kernel(PackArgs a) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t slices = (int64_t)a.rows * (a.K / 32) * 2;
  if (i >= slices) return;
  const int h = (int)(i & 1);
  const int64_t rr = i >> 1;
  const int r = (int)(rr % a.rows), ks = (int)(rr / a.rows);
  int rs = r, sg = 0;
  while (sg + 1 < a.n_segs && rs >= a.seg_rows[sg]) { rs -= a.seg_rows[sg]; ++sg; }
  const bf16* src = a.seg[sg] + (int64_t)rs * a.K + (int64_t)ks * 32;
  bf16x8 v;
  uint32_t idx = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int q = 2 * h + j + (j >= 2 ? 2 : 0);
    const bf16x4 x = *(const bf16x4*)(src + 4 * q);
    float mag[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) mag[e] = fabsf((float)x[e]);
    // an entry stays if fewer than two others rank before it (larger
    // magnitude, or equal magnitude at a lower position)
    int kept[2] = {0, 1}, nk = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      int before = 0;
#pragma unroll
      for (int o = 0; o < 4; ++o) before += (mag[o] > mag[e]) || (mag[o] == mag[e] && o < e);
      if (before < 2 && nk < 2) kept[nk++] = e;
    }
    v[2 * j] = x[kept[0]];
    v[2 * j + 1] = x[kept[1]];
    idx |= (uint32_t)kept[0] << (4 * j) | (uint32_t)kept[1] << (4 * j + 2);
  }
  *(bf16x8*)(a.out + i * 16) = v;
  *(uint16_t*)(a.out + (int64_t)a.rows * a.K + i * 2) = (uint16_t)idx;
}

}  // namespace

extern "C" {

size_t mtfm_s24_pack_bytes(int32_t rows, int32_t k) {
  if (rows <= 0 || k <= 0 || k % 32 != 0) return 0;
  return (size_t)rows * k + (size_t)rows * k / 8;
}

mtfm_status mtfm_s24_pack(const void* const* w_segs, const int32_t* seg_rows, int32_t n_segs, int32_t k,
                          void* packed, size_t packed_bytes, void* stream) {
  if (!w_segs || !seg_rows || !packed) return MTFM_E_NULL;
  if (n_segs < 1 || n_segs > kMaxSegs || k <= 0 || k % 32 != 0) return MTFM_E_DIMS;
  PackArgs a{};
  int64_t rows = 0;
  for (int s = 0; s < n_segs; ++s) {
    if (seg_rows[s] < 0) return MTFM_E_DIMS;
    if (seg_rows[s] > 0 && !w_segs[s]) return MTFM_E_NULL;
    if (((uintptr_t)w_segs[s] & 15) != 0) return MTFM_E_UNSUPPORTED;
    a.seg[s] = (const bf16*)w_segs[s];
    a.seg_rows[s] = seg_rows[s];
    rows += seg_rows[s];
  }
  if (rows == 0) return MTFM_OK;
  if (rows > 0x7fffffff / 2) return MTFM_E_DIMS;
  if (((uintptr_t)packed & 15) != 0) return MTFM_E_UNSUPPORTED;
  if (packed_bytes < mtfm_s24_pack_bytes((int32_t)rows, k)) {
    set_last_error("s24_pack: packed buffer smaller than mtfm_s24_pack_bytes(rows, k)");
    return MTFM_E_WORKSPACE;
  }
  a.n_segs = n_segs; a.rows = (int32_t)rows; a.K = k; a.out = (char*)packed;
  const int64_t slices = rows * (k / 32) * 2;
  if (slices > ((int64_t)1 << 32) - 256) return MTFM_E_DIMS;   // one thread per slice, 32-bit grid
  s24_pack_kernel<<<(unsigned)((slices + 255) / 256), 256, 0, (hipStream_t)stream>>>(a);
  MTFM_LAUNCH_CHECK("s24_pack");
  return MTFM_OK;
}

}  // extern "C"
