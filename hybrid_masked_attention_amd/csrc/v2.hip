// V2 target side ([blog] §3.3.2): RankMixer token mixing of each parent's S
// sub-token rows, their mean pooling, and the interleave of SwiGLU gate/up
// weights that lets the projection GEMM's epilogue see a hidden unit's gate
// and up values in the same lane.  Row kernels, HBM-bound: every element is
// read once and written once.

#include <algorithm>

#include "v2.h"

namespace {

typedef __attribute__((__vector_size__(2 * sizeof(int64_t)))) int64_t piece_t;   // 16 bytes

// One workgroup per parent: its S rows are read whole into registers, then
// (after the barrier, so in place is safe) each 16-byte piece of chunk c of
// row z is written to chunk z of row c.
__global__ __launch_bounds__(256) void token_mix_kernel(TokenRowsArgs a) {
  constexpr int MAXP = 4;
  const int m = blockIdx.x;
  const int per_row = a.D / 8, pieces = a.S * per_row, cw = a.D / a.S;
  const int64_t r0 = a.parent_row[m];
  piece_t v[MAXP];
#pragma unroll
  for (int i = 0; i < MAXP; ++i) {
    const int p = threadIdx.x + 256 * i;
    if (p < pieces) v[i] = *(const piece_t*)(a.x + (r0 + p / per_row) * a.ldx + (p % per_row) * 8);
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < MAXP; ++i) {
    const int p = threadIdx.x + 256 * i;
    if (p >= pieces) continue;
    const int z = p / per_row, col = (p % per_row) * 8;
    const int c = col / cw, w = col % cw;
    *(piece_t*)(a.x + (r0 + c) * a.ldx + z * cw + w) = v[i];
  }
}

// One wave per parent: fp32 sum over sub-tokens in order, times 1/S.
__global__ __launch_bounds__(256) void token_pool_kernel(TokenRowsArgs a) {
  const int m = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (m >= a.n_parents) return;
  const int64_t r0 = a.parent_row[m];
  const float inv = 1.0f / (float)a.S;
  for (int c = lane * 8; c < a.D; c += 512) {
    float s[8] = {};
    for (int z = 0; z < a.S; ++z) {
      const bf16x8 v = *(const bf16x8*)(a.x + (r0 + z) * a.ldx + c);
#pragma unroll
      for (int e = 0; e < 8; ++e) s[e] += (float)v[e];
    }
    bf16x8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (bf16)(s[e] * inv);
    *(bf16x8*)(a.out + (int64_t)m * a.ldo + c) = o;
  }
}

__global__ __launch_bounds__(256) void repack_gate_up_kernel(RepackArgs a) {
  const int64_t per_row = a.D / 8;
  const int64_t total = (int64_t)a.S * 2 * a.F * per_row;
  for (int64_t i = blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    const int64_t row = i / per_row, col = (i % per_row) * 8;
    const int z = (int)(row / (2 * a.F)), r = (int)(row % (2 * a.F));
    const int blk = r / 32, unit = (blk / 2) * 32 + r % 32;
    const bf16* src = ((blk & 1) ? a.up : a.gate) + ((int64_t)z * a.F + unit) * a.D + col;
    *(piece_t*)(a.out + row * a.D + col) = *(const piece_t*)src;
  }
}

}  // namespace

mtfm_status launch_token_mix(const TokenRowsArgs& a, hipStream_t s) {
  if (a.n_parents <= 0 || a.S == 1) return MTFM_OK;
  if (a.D % a.S != 0 || (a.D / a.S) % 8 != 0 || a.S * a.D / 8 > 4 * 256 || a.ldx % 8 != 0) return MTFM_E_UNSUPPORTED;
  token_mix_kernel<<<a.n_parents, 256, 0, s>>>(a);
  MTFM_LAUNCH_CHECK("token_mix");
  return MTFM_OK;
}

mtfm_status launch_token_pool(const TokenRowsArgs& a, hipStream_t s) {
  if (a.n_parents <= 0) return MTFM_OK;
  if (a.D % 8 != 0 || a.ldx % 8 != 0 || a.ldo % 8 != 0 || ((uintptr_t)a.out & 15)) return MTFM_E_UNSUPPORTED;
  token_pool_kernel<<<(a.n_parents + 3) / 4, 256, 0, s>>>(a);
  MTFM_LAUNCH_CHECK("token_pool");
  return MTFM_OK;
}

mtfm_status launch_repack_gate_up(const RepackArgs& a, hipStream_t s) {
  if (a.S <= 0 || a.F <= 0) return MTFM_OK;
  if (a.F % 32 != 0 || a.D % 8 != 0) return MTFM_E_UNSUPPORTED;
  if (((uintptr_t)a.gate | (uintptr_t)a.up | (uintptr_t)a.out) & 15) return MTFM_E_UNSUPPORTED;
  const int64_t total = (int64_t)a.S * 2 * a.F * (a.D / 8);
  const unsigned blocks = (unsigned)std::min<int64_t>((total + 255) / 256, 4096);
  repack_gate_up_kernel<<<blocks, 256, 0, s>>>(a);
  MTFM_LAUNCH_CHECK("repack_gate_up");
  return MTFM_OK;
}
