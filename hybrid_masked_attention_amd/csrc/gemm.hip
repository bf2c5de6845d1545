// Projection GEMMs: bf16 MFMA (gfx950 v_mfma_f32_32x32x16_bf16, fp32
// accumulation) with fused epilogues, a weight-gradient (r-reduced) bf16
// GEMM, and an fp32 FMA kernel for the fp32 correctness path.
//
// The MFMA computes C^T (weights as the A operand) so that each lane ends up
// holding four consecutive output columns of one row; the column segment
// (U / Q / K / V) is uniform per 64-column wave tile.  Block ids are remapped
// so that consecutive logical tiles (which share A rows) land on the same XCD
// and hit its L2.

#include <algorithm>
#include <cstdlib>
#include <type_traits>

#include "gemm.h"

namespace {

constexpr int BM = 128, BN = 128;   // weight-gradient GEMM tile
constexpr float kLog2eF = 1.44269504088896340736f;

MTFM_DEV int64_t map_row(const RowMap& r, int m) {
  if (r.list) {
    if (r.div > 1) return (int64_t)r.list[m / r.div] + m % r.div + r.add;
    return (int64_t)r.list[m] + r.add;
  }
  return (int64_t)m * r.mul + r.add;
}

template <typename T>
MTFM_DEV const T* b_row_ptr(const GemmArgs& g, int z, int n) {
  if (n < g.bn[0]) return (const T*)g.B[0] + (int64_t)z * g.bz[0] + (int64_t)n * g.ldb;
  n -= g.bn[0];
  if (n < g.bn[1]) return (const T*)g.B[1] + (int64_t)z * g.bz[1] + (int64_t)n * g.ldb;
  n -= g.bn[1];
  return (const T*)g.B[2] + (int64_t)z * g.bz[2] + (int64_t)n * g.ldb;
}

MTFM_DEV float silu_fast(float x) {
  return x * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-x * kLog2eF));
}

// Scalar epilogue (fp32 path).
template <typename T>
MTFM_DEV void epilogue_one(const GemmArgs& g, const RowMap& cmap, int m, int n, float acc) {
  const int64_t crow = map_row(cmap, m);
  if (g.epi == EPI_SILU_SPLIT) {
    const float v = acc / (1.0f + __expf(-acc));
    int r = 0;
    while (r < 3 && n >= g.cend[r]) ++r;
    const int c0 = r ? g.cend[r - 1] : 0;
    ((T*)g.dst[r])[crow * g.ld[r] + (n - c0)] = from_f32<T>(v * g.scale[r]);
  } else if (g.epi == EPI_RESID) {
    const float res = to_f32(((const T*)g.resid)[crow * g.ldr + n]);
    ((T*)g.out)[crow * g.ldo + n] = from_f32<T>(acc + res);
  } else if (g.epi == EPI_STORE_F32) {
    float* o = (float*)g.out + crow * g.ldo + n;
    *o = g.accumulate ? *o + acc : acc;
  } else {
    ((T*)g.out)[crow * g.ldo + n] = from_f32<T>(acc);
  }
}

// ---------------------------------------------------------------------------
// bf16 kernel.  Tile 256 (m) x 128 (n), four waves in a 2 x 2 grid (wave tile
// 128 x 64 = 4 x 2 MFMA tiles), K steps of 32 in a two-stage LDS ring that is
// filled by buffer loads straight into LDS (no VGPR staging; rows past the end
// of a matrix read as zero); 48 KB of LDS lets three workgroups share a CU.  Each 64-byte LDS row keeps its four 16-byte
// chunks XOR-swizzled by row so that both the DMA writes and the MFMA
// fragment reads are free of bank conflicts.  Fragments are double buffered
// in registers: the next K slice is read while the current one multiplies.
// The epilogue stages the wave's output tile in the (then idle) LDS ring and
// writes whole 128-byte row segments with 16-byte stores.
constexpr int GBN = 128, GBK = 32, GS = 2, GWN = 2, GNW = 4;
constexpr int G_RPC = 16;                         // rows per 1 KB DMA chunk (4 x 16 B per row)
constexpr int G_LB = GBN / G_RPC / GNW;           // DMA instructions per wave per K step: B
constexpr int G_TN = 2, G_KK = GBK / 16;
constexpr int G_WC = 64;                          // wave tile columns
constexpr int G_EP_BYTES = 9216;                  // per-wave epilogue staging: 64 x 136 B, 32 x 272 B or 64 x 144 B

// Tile rows: 256 (wave tile 128 x 64, three workgroups per CU) for large M,
// 128 (wave tile 64 x 64, four per CU) when 256-row tiles would leave CUs idle.
// NS ring stages: GS, or four for grids smaller than the CU count (a lone
// workgroup per CU waits on each K step's loads; LDS is no constraint there).
template <int BM, int NS = GS> struct GShape {
  static constexpr int LA = BM / G_RPC / GNW;     // DMA instructions per wave per K step: A
  static constexpr int TM = BM / 64;              // MFMA row blocks per wave
  static constexpr int WR = BM / 2;               // wave tile rows
  static constexpr int STAGE = (BM + GBN) * GBK * 2;
  static constexpr int VMC0 = (NS - 1) * (LA + G_LB);
  static constexpr int WG_PER_CU = NS != GS ? 2 : (BM == 256 ? 3 : 4);
  static constexpr int LDS = NS * STAGE > GNW * G_EP_BYTES ? NS * STAGE : GNW * G_EP_BYTES;  // ring, then staging
};
constexpr uint32_t kOobOffset = 0x80000000u;      // voffset of a row past the end (reads zero)

typedef __attribute__((address_space(3))) void lds_void;

MTFM_DEV int g_swz(int r) { return (r >> 2) & 3; }

MTFM_DEV void lds_dma16(__amdgpu_buffer_rsrc_t r, lds_void* dst, uint32_t voff, uint32_t soff) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, voff, soff, 0, 0);
#endif
}

// Buffer resource of a wave-uniform base and size (readfirstlane keeps it in
// scalar registers even where the compiler cannot prove uniformity).
MTFM_DEV __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t b = (uint64_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  void* ub = (void*)(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(ub, (short)0, (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

// s_waitcnt immediates: vmcnt(n) alone, and vmcnt(n) with lgkmcnt(0)
template <int N> MTFM_DEV void wait_vm() { __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0f70); }
template <int N> MTFM_DEV void wait_vm_lgkm() { __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0070); }
MTFM_DEV void wait_lgkm() { __builtin_amdgcn_s_waitcnt(0xc07f); }
// Workgroup barrier without the memory-model waits that __syncthreads adds
// (those would also wait for the DMA loads still in flight).
MTFM_DEV void barrier_only() { asm volatile("s_barrier" ::: "memory"); }

typedef __attribute__((__vector_size__(2 * sizeof(int64_t)))) int64_t i64x2;
// The staged rows are written as bf16 and read back as 8-byte words: reads
// through this type may alias any store (no type-based reordering).
typedef int64_t __attribute__((may_alias)) i64_any;

struct NoPre {
  MTFM_DEV void operator()() const {}
};

// One pass of the staged epilogue: the wave's fp32 accumulators of MFMA row
// blocks [a0, a0 + NA) go through LDS as bf16 (OUTF32 = false; 136-byte rows)
// or fp32 (272-byte rows), then each lane handles one row and 8 consecutive
// columns, calling f(row_local, col_local, v[8]) with the values in fp32
// (or f(row_local, col_local, v[8], round) where f takes the read-back round
// i, row_local = 32 a0 + 8 i + lane / 8).  pre() runs first: loads that the
// pass consumes can be issued there, ahead of the LDS round trip.
template <bool OUTF32, int NA, int TM, typename F, typename Pre = NoPre>
MTFM_DEV void staged_pass(char* ep, const f32x16 (&acc)[G_TN][TM], int a0, int l32, int hi, int lane, F&& f,
                          Pre&& pre = Pre{}) {
  constexpr int RS = OUTF32 ? G_WC * 4 + 16 : G_WC * 2 + 8;
  pre();
  wave_lds_sync();   // the previous pass's reads of this buffer are done
#pragma unroll
  for (int a = 0; a < NA; ++a)
#pragma unroll
    for (int b = 0; b < G_TN; ++b)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        char* d = ep + (a * 32 + l32) * RS + (b * 32 + 8 * j + 4 * hi) * (OUTF32 ? 4 : 2);
        if constexpr (OUTF32) {
          f32x4 v;
#pragma unroll
          for (int q = 0; q < 4; ++q) v[q] = acc[b][a0 + a][4 * j + q];
          *(f32x4*)d = v;
        } else {
          bf16x4 v;
#pragma unroll
          for (int q = 0; q < 4; ++q) v[q] = (bf16)acc[b][a0 + a][4 * j + q];
          *(bf16x4*)d = v;
        }
      }
  wave_lds_sync();   // every lane's writes land before other lanes read them
  // read back: 8 lanes per row (8 columns each), 8 rows per round
#pragma unroll
  for (int i = 0; i < NA * 32 / 8; ++i) {
    const int r = i * 8 + (lane >> 3), c = (lane & 7) * 8;
    float v[8];
    if constexpr (OUTF32) {
      const f32x4 x0 = *(const f32x4*)(ep + r * RS + c * 4);
      const f32x4 x1 = *(const f32x4*)(ep + r * RS + c * 4 + 16);
#pragma unroll
      for (int q = 0; q < 4; ++q) { v[q] = x0[q]; v[4 + q] = x1[q]; }
    } else {
      const i64_any* src = (const i64_any*)(ep + r * RS + c * 2);
      i64x2 raw; raw[0] = src[0]; raw[1] = src[1];
      const bf16x8 x = __builtin_bit_cast(bf16x8, raw);
#pragma unroll
      for (int q = 0; q < 8; ++q) v[q] = (float)x[q];
    }
    if constexpr (std::is_invocable_v<F&, int, int, const float (&)[8], int>) f(a0 * 32 + r, c, v, i);
    else f(a0 * 32 + r, c, v);
  }
}

MTFM_DEV bf16x8 pack8(const float (&v)[8]) {
  bf16x8 o;
#pragma unroll
  for (int q = 0; q < 8; ++q) o[q] = (bf16)v[q];
  return o;
}

// ---------------------------------------------------------------------------
// 2:4 structured-sparse variant (SP = true; gfx950
// v_smfmac_f32_32x32x32_bf16): the pruned weights, packed by mtfm_s24_pack,
// are the instruction's sparse operand and the activations its dense one,
// so each instruction covers a K step of 32 at the MFMA cost of 16.  Row
// maps, the XCD-aware order and the epilogues are the dense kernel's.  The
// LDS ring holds activations only (three stages, filled two K steps ahead);
// each lane loads its packed weight slices (16 bytes of kept values and a
// 16-bit position word per K step and column block) straight from global
// memory into registers.
// Tile rows as in the dense kernel (256 for large M, 128 when that would
// leave CUs idle).  Weights are loaded one K step ahead into two register
// sets: 168 registers at 256 rows (three workgroups per CU, as the dense
// kernel) and 110 at 128 (four).  Two steps ahead in three sets needs 189
// registers at 256 rows, i.e. two workgroups per CU, and measured 8 % slower
// on the 241535-row projections: loads in flight per CU matter more here
// than the weights' prefetch depth.
constexpr int S24_NS = 3;                 // activation ring stages (loaded two K steps ahead)
constexpr int S24_WA = 1;                 // weight slices are loaded this many K steps ahead
constexpr int S24_WS = S24_WA + 1;        // weight register sets
constexpr int S24_U = S24_WS == S24_NS ? S24_NS : S24_NS * S24_WS;   // unroll: stage and set indexes constant
constexpr int S24_WL = 2 * G_TN;          // weight load instructions per wave per K step

template <int BM> struct S24Shape {
  static constexpr int STAGE = BM * GBK * 2;
  static constexpr int LDS = S24_NS * STAGE > GNW * G_EP_BYTES ? S24_NS * STAGE : GNW * G_EP_BYTES;
  static constexpr int WG_PER_CU = BM == 256 ? 3 : 4;
};

typedef __attribute__((__vector_size__(16 * sizeof(__bf16)))) __bf16 bf16x16;

template <int EPI, int GBM, bool SP, int NS = GS>
__global__ __launch_bounds__(256, (SP ? S24Shape<GBM>::WG_PER_CU : GShape<GBM, NS>::WG_PER_CU)) void gemm_bf16_kernel(GemmArgs g) {
  using SH = GShape<GBM, NS>;
  constexpr int G_LA = SH::LA, G_TM = SH::TM, G_WR = SH::WR, G_STAGE = SH::STAGE, G_VMC0 = SH::VMC0;
  constexpr int G_VMC = (NS - 2) * (G_LA + G_LB);
  __shared__ __attribute__((aligned(1024))) char lds[SP ? S24Shape<GBM>::LDS : SH::LDS];

  const int n_mt = (g.M + GBM - 1) / GBM, n_nt = (g.N + GBN - 1) / GBN;
  const int tiles_per_group = n_mt * n_nt;
  const int t = xcd_remap(blockIdx.x, gridDim.x);
  const int z = t / tiles_per_group, tt = t % tiles_per_group;
  const int m0 = (tt / n_nt) * GBM, n0 = (tt % n_nt) * GBN;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / GWN, wn = wave % GWN, l32 = lane & 31, hi = lane >> 5;
  const int rin = lane >> 2, slot = lane & 3;       // DMA lane: row within the chunk, 16-byte slot

  RowMap amap = g.amap; amap.add += z * g.amap_zadd;
  RowMap cmap = g.cmap; cmap.add += z * g.cmap_zadd;

  // A: one buffer resource per DMA instruction.  Contiguous row maps rebase
  // the resource on the chunk's first row (no 4 GiB limit); gathered rows
  // address the whole matrix (bounded on the host).
  __amdgpu_buffer_rsrc_t ra[G_LA];
  uint32_t aoff[G_LA];
#pragma unroll
  for (int i = 0; i < G_LA; ++i) {
    const int rs = (i * GNW + wave) * G_RPC;               // first tile row of the chunk
    const int r = rs + rin, m = m0 + r;
    const uint32_t cb = (uint32_t)((slot ^ g_swz(r)) * 16);
    if (amap.list) {
      ra[i] = make_rsrc(g.A, (uint32_t)(g.a_rows * g.lda * 2));
      MTFM_DCHECK_LANE(m >= g.M || (map_row(amap, m) >= 0 && map_row(amap, m) < g.a_rows), "GEMM gathered row");
      aoff[i] = m < g.M ? (uint32_t)(map_row(amap, m) * g.lda * 2) + cb : kOobOffset;
    } else {
      const int valid = min(max(g.M - (m0 + rs), 0), G_RPC);
      const int64_t row0 = (int64_t)(m0 + rs) * amap.mul + amap.add;
      const uint32_t bytes = valid ? (uint32_t)(((int64_t)(valid - 1) * amap.mul * g.lda + g.K) * 2) : 0u;
      ra[i] = make_rsrc((const bf16*)g.A + (valid ? row0 * g.lda : 0), bytes);
      aoff[i] = (uint32_t)(rin * amap.mul * g.lda * 2) + cb;
    }
  }
  f32x16 acc[G_TN][G_TM];
#pragma unroll
  for (int b = 0; b < G_TN; ++b)
#pragma unroll
    for (int a = 0; a < G_TM; ++a) acc[b][a] = f32x16{};
  if constexpr (!SP) {
    // B: the weight rows of a chunk lie in one segment (segment sizes are multiples of 16)
    __amdgpu_buffer_rsrc_t rb[G_LB];
    uint32_t boff[G_LB];
#pragma unroll
    for (int i = 0; i < G_LB; ++i) {
      const int rs = (i * GNW + wave) * G_RPC;
      const int r = rs + rin, n = n0 + rs;
      const int valid = min(max(g.N - n, 0), G_RPC);
      // (explicit selects keep the segment pointer in scalar registers)
      const void* bseg = g.B[0];
      int64_t bz = g.bz[0];
      int nn = n;
      if (nn >= g.bn[0]) {
        nn -= g.bn[0]; bseg = g.B[1]; bz = g.bz[1];
        if (nn >= g.bn[1]) { nn -= g.bn[1]; bseg = g.B[2]; bz = g.bz[2]; }
      }
      if (g.bgroup[0]) {   // per-group weight matrices
        bseg = z == 0 ? g.bgroup[0] : z == 1 ? g.bgroup[1] : z == 2 ? g.bgroup[2] : g.bgroup[3];
        bz = 0;
      }
      const bf16* base = (const bf16*)bseg + (int64_t)z * bz + (int64_t)nn * g.ldb;
      rb[i] = make_rsrc(valid ? base : (const bf16*)g.B[0], valid ? (uint32_t)(((int64_t)(valid - 1) * g.ldb + g.K) * 2) : 0u);
      boff[i] = (uint32_t)(rin * g.ldb * 2 + (slot ^ g_swz(r)) * 16);
    }
    auto issue = [&](int step, int stage) {
      char* base = lds + stage * G_STAGE;
      const uint32_t so = (uint32_t)step * GBK * 2;
#pragma unroll
      for (int i = 0; i < G_LA; ++i) lds_dma16(ra[i], (lds_void*)(base + (i * GNW + wave) * 1024), aoff[i], so);
#pragma unroll
      for (int i = 0; i < G_LB; ++i)
        lds_dma16(rb[i], (lds_void*)(base + GBM * GBK * 2 + (i * GNW + wave) * 1024), boff[i], so);
    };

    // fragment offsets within a stage: chunk (2 kk + hi) of row r sits at slot chunk ^ f(r)
    int arow[G_TM], af[G_TM], brow[G_TN], bfo[G_TN];
#pragma unroll
    for (int i = 0; i < G_TM; ++i) {
      const int r = wm * G_WR + i * 32 + l32;
      arow[i] = r * GBK * 2; af[i] = hi ^ g_swz(r);
    }
#pragma unroll
    for (int i = 0; i < G_TN; ++i) {
      const int r = wn * G_WC + i * 32 + l32;
      brow[i] = GBM * GBK * 2 + r * GBK * 2; bfo[i] = hi ^ g_swz(r);
    }
    bf16x8 fa[2][G_TM], fb[2][G_TN];
    auto read = [&](int stage, int kk, int buf) {
      const char* st = lds + stage * G_STAGE;
#pragma unroll
      for (int i = 0; i < G_TM; ++i) fa[buf][i] = *(const bf16x8*)(st + arow[i] + (((2 * kk) ^ af[i]) << 4));
#pragma unroll
      for (int i = 0; i < G_TN; ++i) fb[buf][i] = *(const bf16x8*)(st + brow[i] + (((2 * kk) ^ bfo[i]) << 4));
    };
    auto mma = [&](int buf) {   // C^T tiles: weights as the A operand, so a lane holds 4 consecutive columns
#pragma unroll
      for (int b = 0; b < G_TN; ++b)
#pragma unroll
        for (int a = 0; a < G_TM; ++a)
          acc[b][a] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[buf][b], fa[buf][a], acc[b][a], 0, 0, 0);
    };

    const int nk = g.K / GBK;
#pragma unroll
    for (int s = 0; s < NS; ++s)
      if (s < nk) issue(s, s);
    if (NS - 1 < nk) wait_vm<G_VMC0>();
    else wait_vm<0>();
    barrier_only();
    read(0, 0, 0);
    int stage = 0;
    for (int s = 0; s < nk - 1; ++s) {
#pragma unroll
      for (int kk = 0; kk < G_KK; ++kk) {
        const int cur = kk & 1;
        if (kk + 1 < G_KK) {
          read(stage, kk + 1, cur ^ 1);
        } else {
          // step s + 1 has landed once at most G_VMC newer DMA instructions are
          // outstanding; the barrier also tells every wave that this stage has
          // been read (lgkmcnt(0)) so it can be refilled with step s + NS
          if (s + NS - 1 < nk) wait_vm_lgkm<G_VMC>();
          else wait_vm_lgkm<0>();
          barrier_only();
          if (s + NS < nk) issue(s + NS, stage);
          stage = (stage + 1 == NS) ? 0 : stage + 1;
          read(stage, 0, cur ^ 1);
        }
        mma(cur);
      }
    }
#pragma unroll
    for (int kk = 0; kk < G_KK; ++kk) {
      const int cur = kk & 1;
      if (kk + 1 < G_KK) read(stage, kk + 1, cur ^ 1);
      mma(cur);
    }

  } else {
    constexpr int STAGE = S24Shape<GBM>::STAGE;
    // loads issued after step t's: step t + 1's (weights first, then activations)
    constexpr int VMC = S24_WA == 2 ? S24_WL + G_LA : G_LA;
    auto issue = [&](int step, int stage) {
      char* base = lds + stage * STAGE;
      const uint32_t so = (uint32_t)step * GBK * 2;
#pragma unroll
      for (int i = 0; i < G_LA; ++i) lds_dma16(ra[i], (lds_void*)(base + (i * GNW + wave) * 1024), aoff[i], so);
    };

    // packed weights: slice (step, row, half) of this lane's output column in
    // each 32-column block; columns past N repeat row N - 1 (never stored)
    const char* wvals = (const char*)g.bs24;
    int64_t zrows = g.bs24_zrows;
    if (g.bgroup[0]) {   // per-group packed matrices
      wvals = (const char*)(z == 0 ? g.bgroup[0] : z == 1 ? g.bgroup[1] : z == 2 ? g.bgroup[2] : g.bgroup[3]);
      zrows = 0;
    }
    const int64_t wrows = g.bs24_rows;
    const char* widx = wvals + wrows * g.K;
    int64_t wslice[G_TN];
#pragma unroll
    for (int b = 0; b < G_TN; ++b) {
      const int n = min(n0 + wn * G_WC + b * 32 + l32, g.N - 1);
      wslice[b] = ((int64_t)z * zrows + n) * 2 + hi;
    }
    bf16x8 wv[S24_WS][G_TN];
    int wi[S24_WS][G_TN];
    auto wload = [&](int step, int set) {
#pragma unroll
      for (int b = 0; b < G_TN; ++b) {
        const int64_t e = (int64_t)step * wrows * 2 + wslice[b];
        wv[set][b] = *(const bf16x8*)(wvals + e * 16);
        wi[set][b] = *(const uint16_t*)(widx + e * 2);
      }
    };

    // B operand of the sparse instruction: lane (row, half h) holds K entries
    // 16 h .. 16 h + 15 of its activation row = LDS chunks 2 h and 2 h + 1
    int arow[G_TM], af[G_TM];
#pragma unroll
    for (int i = 0; i < G_TM; ++i) {
      const int r = wm * G_WR + i * 32 + l32;
      arow[i] = r * GBK * 2; af[i] = g_swz(r);
    }

    // Issue order: activations of step 0, then per step j the weights of step
    // j + S24_WA and the activations of step j + 2, so that a step's loads are
    // followed only by the next step's.  Every step issues the same loads
    // (steps past the end re-read the last one into a stage no longer read):
    // with no branches around them the compiler's own wait counting stays as
    // loose as the explicit waits below.
    const int nk = g.K / GBK;
    issue(0, 0);
#pragma unroll
    for (int j = 0; j < S24_WA; ++j) wload(min(j, nk - 1), j);
    issue(min(1, nk - 1), 1);
    for (int s0 = 0; s0 < nk; s0 += S24_U) {
#pragma unroll
      for (int u = 0; u < S24_U; ++u) {
        const int t = s0 + u;
        if (t >= nk) break;
        const int st = u % S24_NS, ws = u % S24_WS;   // constants once the loop is unrolled
        // step t has landed once only step t + 1's loads may be outstanding;
        // the barrier also tells every wave that the previous stage has been
        // read, so it can take step t + 2
        wait_vm_lgkm<VMC>();
        barrier_only();
        wload(min(t + S24_WA, nk - 1), (u + S24_WA) % S24_WS);
        issue(min(t + 2, nk - 1), (u + 2) % S24_NS);
        const char* sb = lds + st * STAGE;
#pragma unroll
        for (int a = 0; a < G_TM; ++a) {
          const bf16x8 lo = *(const bf16x8*)(sb + arow[a] + (((2 * hi) ^ af[a]) << 4));
          const bf16x8 up = *(const bf16x8*)(sb + arow[a] + (((2 * hi + 1) ^ af[a]) << 4));
          const bf16x16 fa = __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
#pragma unroll
          for (int b = 0; b < G_TN; ++b)
            acc[b][a] = __builtin_amdgcn_smfmac_f32_32x32x32_bf16(wv[ws][b], fa, acc[b][a], wi[ws][b], 0, 0);
        }
      }
    }
    wait_vm<0>();   // the tail's loads land before the epilogue reuses the ring
  }

  // ---- epilogue: the ring is free once every wave has finished its reads
  wait_lgkm();
  barrier_only();
  char* ep = lds + wave * G_EP_BYTES;
  const int mw = m0 + wm * G_WR, nw = n0 + wn * G_WC;
  if (nw >= g.N) return;   // wave tile entirely past the last column (after the barrier)
  if constexpr (EPI == EPI_SILU_SPLIT) {
    // output segment of this wave's columns (selects, not a dynamic index into the arguments)
    void* dseg = g.dst[0];
    int64_t ldseg = g.ld[0];
    float sc = g.scale[0];
    int c0 = 0;
    const uint8_t* rtype = nullptr;   // segment 3 with a row filter: T rows only
    if (nw >= g.cend[0]) {
      c0 = g.cend[0]; dseg = g.dst[1]; ldseg = g.ld[1]; sc = g.scale[1];
      if (nw >= g.cend[1]) {
        c0 = g.cend[1]; dseg = g.dst[2]; ldseg = g.ld[2]; sc = g.scale[2];
        if (nw >= g.cend[2]) { c0 = g.cend[2]; dseg = g.dst[3]; ldseg = g.ld[3]; sc = g.scale[3]; rtype = g.seg3_type; }
      }
    }
    if (g.pre) {
#pragma unroll
      for (int h = 0; h < G_WR / 64; ++h)
        staged_pass<false, 2>(ep, acc, 2 * h, l32, hi, lane, [&](int rl, int cl, const float (&v)[8]) {
          const int m = mw + rl;
          if (m < g.M && nw + cl < g.N) *(bf16x8*)((bf16*)g.pre + map_row(cmap, m) * g.ldpre + nw + cl) = pack8(v);
        });
    }
#pragma unroll
    for (int b = 0; b < G_TN; ++b)
#pragma unroll
      for (int a = 0; a < G_TM; ++a)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[b][a][e] = silu_fast(acc[b][a][e]) * sc;
    if (dseg) {
#pragma unroll
      for (int h = 0; h < G_WR / 64; ++h)
        staged_pass<false, 2>(ep, acc, 2 * h, l32, hi, lane, [&](int rl, int cl, const float (&v)[8]) {
          const int m = mw + rl;
          if (m < g.M && nw + cl < g.N) {
            const int64_t crow = map_row(cmap, m);
            if (!rtype || rtype[crow] == TT_T) *(bf16x8*)((bf16*)dseg + crow * ldseg + (nw - c0) + cl) = pack8(v);
          }
        });
    }
    if (g.vt && nw >= g.vt_col0 && nw < g.vt_col0 + g.vt_cols) {
      // transposed copy, in two passes of 64 rows: LDS [64 columns][64 rows]
      // (144-byte rows), then each lane writes 8 consecutive slots of one
      // column: slots 16G + 8h + [0, 8) hold rows 16G + 4h + [0, 4) and
      // 16G + 8 + 4h + [0, 4)
      constexpr int RT = 64 * 2 + 16;
      const int64_t col0 = nw - g.vt_col0;
#pragma unroll
      for (int pass = 0; pass < G_WR / 64; ++pass) {
        wave_lds_sync();   // earlier passes' reads of the staging buffer are done
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
          for (int b = 0; b < G_TN; ++b)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              const int col = b * 32 + 8 * (e >> 2) + 4 * hi + (e & 3);
              *(bf16*)(ep + col * RT + (a * 32 + l32) * 2) = (bf16)acc[b][2 * pass + a][e];
            }
        wave_lds_sync();   // the transposed tile is complete before lanes read columns
#pragma unroll
        for (int i = 0; i < G_WC / 8; ++i) {
          const int col = i * 8 + (lane >> 3), sc = lane & 7;      // 8 lanes per column, 8 slots each
          const int r0 = (sc >> 1) * 16 + 4 * (sc & 1);
          const i64_any* s0 = (const i64_any*)(ep + col * RT + r0 * 2);
          const i64_any* s1 = (const i64_any*)(ep + col * RT + (r0 + 8) * 2);
          i64x2 v; v[0] = *s0; v[1] = *s1;
          const int64_t slot0 = (int64_t)mw + pass * 64 + sc * 8;
          if (slot0 < g.ldvt && nw + col < g.N)
            *(i64x2*)((bf16*)g.vt + (int64_t)z * g.vt_zstride + (col0 + col) * g.ldvt + slot0) = v;
        }
      }
    }
  } else if constexpr (EPI == EPI_SWIGLU) {
    // the wave tile's 32-column halves are the gate and up rows of the same 32 hidden
    // units: a lane holds both for the same row and units, so it writes SiLU(g) * u
    // as runs of four units
    const int u0 = nw / 2;
#pragma unroll
    for (int a = 0; a < G_TM; ++a) {
      const int m = mw + a * 32 + l32;
      if (m >= g.M) continue;
      bf16* orow = (bf16*)g.out + map_row(cmap, m) * g.ldo + u0 + 4 * hi;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf16x4 v;
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = (bf16)(silu_fast(acc[0][a][4 * j + q]) * acc[1][a][4 * j + q]);
        *(bf16x4*)(orow + 8 * j) = v;
      }
    }
  } else if constexpr (EPI == EPI_STORE) {
#pragma unroll
    for (int h = 0; h < G_WR / 64; ++h)
      staged_pass<false, 2>(ep, acc, 2 * h, l32, hi, lane, [&](int rl, int cl, const float (&v)[8]) {
        const int m = mw + rl;
        if (m < g.M && nw + cl < g.N) *(bf16x8*)((bf16*)g.out + map_row(cmap, m) * g.ldo + nw + cl) = pack8(v);
      });
  } else if constexpr (EPI == EPI_RESID) {
    // fp32 staging in four passes of 32 rows; a pass's residual segments are
    // loaded before its LDS round trip (their latency overlaps the staging)
#pragma unroll
    for (int h = 0; h < G_TM; ++h) {
      bf16x8 res[4];
      const int cl = (lane & 7) * 8;
      staged_pass<true, 1>(
          ep, acc, h, l32, hi, lane,
          [&](int rl, int, const float (&v)[8], int i) {
            const int m = mw + rl;
            if (m >= g.M || nw + cl >= g.N) return;
            float o[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) o[q] = v[q] + (float)res[i][q];
            *(bf16x8*)((bf16*)g.out + map_row(cmap, m) * g.ldo + nw + cl) = pack8(o);
          },
          [&]() {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int m = mw + h * 32 + i * 8 + (lane >> 3);
              res[i] = (m < g.M && nw + cl < g.N)
                           ? *(const bf16x8*)((const bf16*)g.resid + map_row(cmap, m) * g.ldr + nw + cl)
                           : bf16x8{};
            }
          });
    }
  } else {
    // fp32 staging in four passes of 32 rows
#pragma unroll
    for (int h = 0; h < G_TM; ++h) {
      staged_pass<true, 1>(ep, acc, h, l32, hi, lane, [&](int rl, int cl, const float (&v)[8]) {
        const int m = mw + rl;
        if (m >= g.M || nw + cl >= g.N) return;
        const int64_t crow = map_row(cmap, m);
        {
          float* d = (float*)g.out + crow * g.ldo + nw + cl;
          f32x4 o0, o1;
          if (g.accumulate) { o0 = *(const f32x4*)d; o1 = *(const f32x4*)(d + 4); }
          else { o0 = f32x4{}; o1 = f32x4{}; }
#pragma unroll
          for (int q = 0; q < 4; ++q) { o0[q] += v[q]; o1[q] += v[4 + q]; }
          *(f32x4*)d = o0;
          *(f32x4*)(d + 4) = o1;
        }
      });
    }
  }
}



// ---------------------------------------------------------------------------
// Weight-gradient GEMM.  Block tile 128 (m) x 128 (n), 32 rows of r per step:
// each thread loads a pair of rows r, r+1 at 8 consecutive m (or n) and
// writes them transposed into LDS as [m][r] so the MFMA operands (8
// consecutive r per lane) are 16-byte reads.  Grid: tiles x splits of r; a
// split writes its partial tile, the reduction adds splits in order.
constexpr int TBK = 32, T_STRIDE = TBK + 8;
constexpr int TN_ROWS_PER_SPLIT = 2048;

__global__ __launch_bounds__(256, 2) void gemm_tn_kernel(GemmTNArgs g, int n_split) {
  __shared__ __attribute__((aligned(16))) bf16 As[BM * T_STRIDE];
  __shared__ __attribute__((aligned(16))) bf16 Bs[BN * T_STRIDE];
  const int z = blockIdx.z;
  const int n_mt = (g.M + BM - 1) / BM, n_nt = (g.N + BN - 1) / BN;
  const int tiles = n_mt * n_nt;
  const int split = blockIdx.x / tiles, t = blockIdx.x % tiles;
  const int mt = t / n_nt, nt = t % n_nt;
  const int m0 = mt * BM, n0 = nt * BN;
  RowMap amap = g.amap; amap.add += z * g.amap_zadd;
  RowMap bmap = g.bmap; bmap.add += z * g.bmap_zadd;
  const bf16* A = (const bf16*)g.A + (int64_t)z * g.a_zoff;
  const bf16* B = (const bf16*)g.B;
  const int r_begin = split * TN_ROWS_PER_SPLIT, r_end = min(g.R, r_begin + TN_ROWS_PER_SPLIT);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, hi = lane >> 5;
  // staging item: row pair rp (16 pairs per step), 8-column chunk cc (16 chunks of 128)
  const int rp = tid >> 4, cc = tid & 15;

  f32x16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = f32x16{};

  for (int r0 = r_begin; r0 < r_end; r0 += TBK) {
    bf16x8 av[2], bv[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int r = r0 + 2 * rp + e;
      const bool ok = r < r_end;
      const int m = m0 + cc * 8, n = n0 + cc * 8;
      av[e] = (ok && m < g.M) ? *(const bf16x8*)(A + map_row(amap, r) * g.lda + m) : bf16x8{};
      bv[e] = (ok && n < g.N) ? *(const bf16x8*)(B + map_row(bmap, r) * g.ldb + n) : bf16x8{};
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      bf16x2 pa, pb;
      pa[0] = av[0][s]; pa[1] = av[1][s];
      pb[0] = bv[0][s]; pb[1] = bv[1][s];
      *(bf16x2*)(&As[(cc * 8 + s) * T_STRIDE + 2 * rp]) = pa;
      *(bf16x2*)(&Bs[(cc * 8 + s) * T_STRIDE + 2 * rp]) = pb;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < TBK / 16; ++kk) {
      bf16x8 af[2], bfr[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
        af[mb] = *(const bf16x8*)(&As[(wm * 64 + mb * 32 + l32) * T_STRIDE + kk * 16 + 8 * hi]);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
        bfr[nb] = *(const bf16x8*)(&Bs[(wn * 64 + nb * 32 + l32) * T_STRIDE + kk * 16 + 8 * hi]);
      // C^T tiles: lane = m, registers = four consecutive n
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
          acc[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[nb], af[mb], acc[nb][mb], 0, 0, 0);
    }
  }
  float* P = g.partial + ((int64_t)z * n_split + split) * (int64_t)g.M * g.N;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    const int m = m0 + wm * 64 + mb * 32 + l32;
    if (m >= g.M) continue;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int nblk = n0 + wn * 64 + nb * 32;
      if (nblk >= g.N) continue;
      float* dst = P + (int64_t)m * g.N + nblk + 4 * hi;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f32x4 v;
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = acc[nb][mb][4 * j + q];
        *(f32x4*)(dst + 8 * j) = v;
      }
    }
  }
}

// Weight-gradient GEMM, DMA form.  Same tiles, splits and partial layout as
// above; the 32-row steps of A and B are copied row-major into a three-stage
// LDS ring by buffer DMA (rows past the split's end and columns past M / N read
// as zeros), and the MFMA operands -- 8 consecutive r of one column per lane --
// come out of it through the transposing LDS read.  The split's row indices
// (row maps applied) sit in a table of their own, so reading them never waits
// for the DMA.
constexpr int TD_NS = 3;
static_assert(TN_ROWS_PER_SPLIT % 256 == 0, "row table fill");
constexpr int TD_TILE = 32 * 256;     // 32 rows x 128 bf16 columns
constexpr int TD_STAGE = 2 * TD_TILE;  // A, then B

// 16-byte unit u of tile row r sits at slot u ^ 4 (r % 4): the four rows of one
// transposing read then fall in four different quarters of the banks.
MTFM_DEV int td_swz(int r) { return (r & 3) << 2; }

typedef short td_i16x4 __attribute__((ext_vector_type(4)));

// The 16 transposing reads of one stage for one wave: fragment f (0, 1: A
// column blocks mb; 2, 3: B column blocks nb) at LDS address a[f], plus 4096 B
// for the second 16 rows (kk = 1) and 1024 B for rows 4..7 of each 8 (h = 1).
// One block with its own wait: the compiler would otherwise wait for every DMA
// in flight before each read (it cannot tell which ring stage a read touches).
MTFM_DEV void td_tr16(const uint32_t (&a)[4], td_i16x4 (&o)[2][4][2]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %16\n\t"
      "ds_read_b64_tr_b16 %1, %16 offset:1024\n\t"
      "ds_read_b64_tr_b16 %2, %17\n\t"
      "ds_read_b64_tr_b16 %3, %17 offset:1024\n\t"
      "ds_read_b64_tr_b16 %4, %18\n\t"
      "ds_read_b64_tr_b16 %5, %18 offset:1024\n\t"
      "ds_read_b64_tr_b16 %6, %19\n\t"
      "ds_read_b64_tr_b16 %7, %19 offset:1024\n\t"
      "ds_read_b64_tr_b16 %8, %16 offset:4096\n\t"
      "ds_read_b64_tr_b16 %9, %16 offset:5120\n\t"
      "ds_read_b64_tr_b16 %10, %17 offset:4096\n\t"
      "ds_read_b64_tr_b16 %11, %17 offset:5120\n\t"
      "ds_read_b64_tr_b16 %12, %18 offset:4096\n\t"
      "ds_read_b64_tr_b16 %13, %18 offset:5120\n\t"
      "ds_read_b64_tr_b16 %14, %19 offset:4096\n\t"
      "ds_read_b64_tr_b16 %15, %19 offset:5120\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o[0][0][0]), "=&v"(o[0][0][1]), "=&v"(o[0][1][0]), "=&v"(o[0][1][1]),
        "=&v"(o[0][2][0]), "=&v"(o[0][2][1]), "=&v"(o[0][3][0]), "=&v"(o[0][3][1]),
        "=&v"(o[1][0][0]), "=&v"(o[1][0][1]), "=&v"(o[1][1][0]), "=&v"(o[1][1][1]),
        "=&v"(o[1][2][0]), "=&v"(o[1][2][1]), "=&v"(o[1][3][0]), "=&v"(o[1][3][1])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3])
      : "memory");
}

__global__ __launch_bounds__(256, 2) void gemm_tn_dma_kernel(GemmTNArgs g, int n_split) {
  __shared__ __attribute__((aligned(1024))) char ring[TD_NS * TD_STAGE];
  __shared__ int32_t rowtab[2][TN_ROWS_PER_SPLIT];
  const int z = blockIdx.z;
  const int n_mt = (g.M + BM - 1) / BM, n_nt = (g.N + BN - 1) / BN;
  const int tiles = n_mt * n_nt;
  const int split = blockIdx.x / tiles, t = blockIdx.x % tiles;
  const int mt = t / n_nt, nt = t % n_nt;
  const int m0 = mt * BM, n0 = nt * BN;
  RowMap amap = g.amap; amap.add += z * g.amap_zadd;
  RowMap bmap = g.bmap; bmap.add += z * g.bmap_zadd;
  const int r_begin = split * TN_ROWS_PER_SPLIT, r_end = min(g.R, r_begin + TN_ROWS_PER_SPLIT);
  const int nrows = r_end - r_begin;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int hi = lane >> 5;

  {
    // all loads of the row lists first, then the table writes
    constexpr int PER = TN_ROWS_PER_SPLIT / 256;
    int32_t av[PER], bv[PER];
    auto fill = [&](const RowMap& m, int32_t (&v)[PER]) {
      if (m.list) {
        const int dv = max(m.div, 1);
#pragma unroll
        for (int k = 0; k < PER; ++k) {
          const int r = r_begin + min(tid + 256 * k, nrows - 1);   // entries past the end unused
          v[k] = m.list[r / dv] + r % dv + m.add;
        }
      } else {
#pragma unroll
        for (int k = 0; k < PER; ++k) v[k] = (r_begin + tid + 256 * k) * m.mul + m.add;
      }
    };
    if (nrows > 0) {
      fill(amap, av);
      fill(bmap, bv);
    }
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      rowtab[0][tid + 256 * k] = av[k];
      rowtab[1][tid + 256 * k] = bv[k];
    }
  }
  __syncthreads();

  const int64_t a_shift = (int64_t)z * g.a_zoff;
  const __amdgpu_buffer_rsrc_t ra =
      make_rsrc((const bf16*)g.A + a_shift, (uint32_t)(g.a_rows * g.lda * 2 - a_shift * 2));
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(g.B, (uint32_t)(g.b_rows * g.ldb * 2));
  // DMA lanes: chunk c (of 8 per tile) = rows 4c .. 4c + 3; lane -> row 4c + lane/16,
  // slot lane % 16, holding columns 8 (slot ^ swz(row)) .. + 7
  const int rq = lane >> 4;
  const int lu = (lane & 15) ^ td_swz(rq);
  const bool a_col = m0 + 8 * lu < g.M, b_col = n0 + 8 * lu < g.N;
  const int nst = (nrows + 31) >> 5;
  auto issue = [&](int st_i) {
    char* st = ring + (st_i % TD_NS) * TD_STAGE;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = i * 4 + wave;
      const int rr = st_i * 32 + 4 * c + rq;     // row within the split
      const bool ok = st_i < nst && rr < nrows;
      const uint32_t ao = ok && a_col ? (uint32_t)(rowtab[0][rr] * g.lda * 2 + (m0 + 8 * lu) * 2) : kOobOffset;
      const uint32_t bo = ok && b_col ? (uint32_t)(rowtab[1][rr] * g.ldb * 2 + (n0 + 8 * lu) * 2) : kOobOffset;
      lds_dma16(ra, (lds_void*)(st + c * 1024), ao, 0);
      lds_dma16(rb, (lds_void*)(st + TD_TILE + c * 1024), bo, 0);
    }
  };
#pragma unroll
  for (int s = 0; s < TD_NS - 1; ++s) issue(s);

  // transposing-read addresses: column block start + 16 ((lane/16) % 2) + 4 (lane % 4),
  // rows 8 hi + (lane/4) % 4 (+ 16 kk + 4 h as immediates, which keep row % 4)
  uint32_t tro[4];
  {
    const int r = 8 * hi + ((lane >> 2) & 3);
    const int cw = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const int col = (f < 2 ? wm * 64 + f * 32 : wn * 64 + (f - 2) * 32) + cw;
      tro[f] = (uint32_t)((f < 2 ? 0 : TD_TILE) + r * 256 + (((col >> 3) ^ td_swz(r)) << 4) + (col & 7) * 2);
    }
  }
  const uint32_t ring_addr = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)ring;

  f32x16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = f32x16{};

  for (int it = 0; it < nst; ++it) {
    wait_vm_lgkm<(TD_NS - 2) * 4>();
    barrier_only();
    issue(it + TD_NS - 1);
    uint32_t a4[4];
    const uint32_t sb = ring_addr + (uint32_t)((it % TD_NS) * TD_STAGE);
#pragma unroll
    for (int f = 0; f < 4; ++f) a4[f] = sb + tro[f];
    td_i16x4 fr[2][4][2];
    td_tr16(a4, fr);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      bf16x8 op[4];
#pragma unroll
      for (int f = 0; f < 4; ++f)
        op[f] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(fr[kk][f][0], fr[kk][f][1], 0, 1, 2, 3, 4, 5, 6, 7));
      // C^T tiles: lane = m, registers = four consecutive n
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
          acc[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[2 + nb], op[mb], acc[nb][mb], 0, 0, 0);
    }
  }
  wait_vm_lgkm<0>();   // the ring's trailing (empty) loads land before the workgroup ends
  const int l32 = lane & 31;
  float* P = g.partial + ((int64_t)z * n_split + split) * (int64_t)g.M * g.N;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    const int m = m0 + wm * 64 + mb * 32 + l32;
    if (m >= g.M) continue;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int nblk = n0 + wn * 64 + nb * 32;
      if (nblk >= g.N) continue;
      float* dst = P + (int64_t)m * g.N + nblk + 4 * hi;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f32x4 v;
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = acc[nb][mb][4 * j + q];
        *(f32x4*)(dst + 8 * j) = v;
      }
    }
  }
}

// C (+)= sum over splits of the partials, in split order.
__global__ __launch_bounds__(256) void gemm_tn_reduce_kernel(GemmTNArgs g, int n_split) {
  const int z = blockIdx.y;
  const int64_t mn = (int64_t)g.M * g.N;
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= mn) return;
  const float* P = g.partial + (int64_t)z * n_split * mn + i;
  f32x4 s = *(const f32x4*)P;
  for (int k = 1; k < n_split; ++k) {
    const f32x4 v = *(const f32x4*)(P + k * mn);
#pragma unroll
    for (int q = 0; q < 4; ++q) s[q] += v[q];
  }
  const int m = (int)(i / g.N), n = (int)(i % g.N);
  float* dst = g.C + (int64_t)z * g.c_zoff + (int64_t)m * g.ldc + n;
  if (g.accumulate) {
    const f32x4 o = *(const f32x4*)dst;
#pragma unroll
    for (int q = 0; q < 4; ++q) s[q] += o[q];
  }
  *(f32x4*)dst = s;
}

// fp32 path: one thread per output element (tiny correctness configs).
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs g) {
  const int z = blockIdx.z;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)g.M * g.N) return;
  const int m = (int)(idx / g.N), n = (int)(idx % g.N);
  RowMap amap = g.amap; amap.add += z * g.amap_zadd;
  RowMap cmap = g.cmap; cmap.add += z * g.cmap_zadd;
  const float* a = (const float*)g.A + map_row(amap, m) * g.lda;
  const float* b = b_row_ptr<float>(g, z, n);
  float acc = 0.f;
  for (int k = 0; k < g.K; ++k) acc = fmaf(a[k], b[k], acc);
  epilogue_one<float>(g, cmap, m, n, acc);
}

}  // namespace

// Compute units of the current device (cached per device id).
int device_cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cached[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

static bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

int64_t gemm_tn_partial_elems(int32_t M, int32_t N, int32_t R, int32_t groups) {
  const int64_t n_split = std::max<int64_t>(1, (R + TN_ROWS_PER_SPLIT - 1) / TN_ROWS_PER_SPLIT);
  return n_split * (int64_t)M * N * groups;
}

mtfm_status launch_gemm_tn(const GemmTNArgs& g, hipStream_t s) {
  if (g.M <= 0 || g.N <= 0 || g.groups <= 0) return MTFM_OK;
  if (g.M % 8 != 0 || g.N % 32 != 0 || g.lda % 8 != 0 || g.ldb % 8 != 0 || g.ldc % 4 != 0)
    return MTFM_E_UNSUPPORTED;
  const int n_split = std::max(1, (g.R + TN_ROWS_PER_SPLIT - 1) / TN_ROWS_PER_SPLIT);
  if (gemm_tn_partial_elems(g.M, g.N, g.R, g.groups) > g.partial_elems) return MTFM_E_WORKSPACE;
  const int tiles = ((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN);
  // the DMA form needs the operands' row counts (its loads are bounded by them,
  // with 32-bit offsets) and 16-byte aligned rows
  const int64_t a_bytes = g.a_rows * g.lda * 2, b_bytes = g.b_rows * g.ldb * 2;
  // (MTFM_GEMM_TN_STAGED=1 forces the register-staged kernel: both accumulate the
  // same rows in the same order, so they agree bit for bit)
  const char* forced = std::getenv("MTFM_GEMM_TN_STAGED");
  const bool dma = !(forced && forced[0] == '1') && g.a_rows > 0 && g.b_rows > 0 &&
                   a_bytes < (int64_t)kOobOffset && b_bytes < (int64_t)kOobOffset && g.a_zoff == 0 &&
                   aligned16(g.A) && aligned16(g.B);
  if (dma) {
    gemm_tn_dma_kernel<<<dim3(tiles * n_split, 1, g.groups), 256, 0, s>>>(g, n_split);
    MTFM_LAUNCH_CHECK("gemm_tn_dma");
  } else {
    gemm_tn_kernel<<<dim3(tiles * n_split, 1, g.groups), 256, 0, s>>>(g, n_split);
    MTFM_LAUNCH_CHECK("gemm_tn");
  }
  const int64_t mn4 = ((int64_t)g.M * g.N) / 4;
  gemm_tn_reduce_kernel<<<dim3((unsigned)((mn4 + 255) / 256), g.groups), 256, 0, s>>>(g, n_split);
  MTFM_LAUNCH_CHECK("gemm_tn_reduce");
  return MTFM_OK;
}

mtfm_status launch_gemm(const GemmArgs& g, int dtype, hipStream_t s) {
  if (g.M <= 0 || g.N <= 0 || g.groups <= 0) return MTFM_OK;
  if (dtype == MTFM_BF16) {
    // K in whole steps; 16-byte rows and stores; weight segments in whole DMA
    // chunks; output segments aligned to the 64-column wave tile
    if (g.K % GBK != 0 || g.N % 8 != 0 || g.lda % 8 != 0 || g.ldb % 8 != 0) return MTFM_E_UNSUPPORTED;
    if (!aligned16(g.A)) return MTFM_E_UNSUPPORTED;
    if (g.bs24) {
      // every group's rows inside the packed matrix
      if (!aligned16(g.bs24) || g.bs24_rows <= 0 || g.bs24_zrows < 0 ||
          (int64_t)(g.groups - 1) * g.bs24_zrows + g.N > g.bs24_rows)
        return MTFM_E_UNSUPPORTED;
    } else {
      if (!aligned16(g.B[0])) return MTFM_E_UNSUPPORTED;
      if (g.N > g.bn[0] && (g.bn[0] % G_RPC != 0 || !aligned16(g.B[1]))) return MTFM_E_UNSUPPORTED;
      if (g.N > g.bn[0] + g.bn[1] && (g.bn[1] % G_RPC != 0 || !aligned16(g.B[2]))) return MTFM_E_UNSUPPORTED;
    }
    if (g.amap.list) {
      // gathered rows address the whole A buffer through one 31-bit offset
      if (g.a_rows <= 0 || g.a_rows * g.lda * 2 + (int64_t)g.K * 2 >= (int64_t)kOobOffset) {
        set_last_error("gemm: gathered activation matrix exceeds 2 GiB");
        return MTFM_E_UNSUPPORTED;
      }
    }
    if (g.bgroup[0]) {
      // per-group weights: dense matrices of N rows, or packed ones of bs24_rows rows
      if (g.groups > 4 || g.bn[0] != g.N || (g.bs24 && g.bs24_zrows != 0)) return MTFM_E_UNSUPPORTED;
      for (int z = 0; z < g.groups; ++z) {
        if (!g.bgroup[z]) return MTFM_E_NULL;
        if (g.bs24 && !aligned16(g.bgroup[z])) return MTFM_E_UNSUPPORTED;
      }
    }
    if (g.epi == EPI_SILU_SPLIT) {
      for (int r = 0; r < 4; ++r) {
        if (g.cend[r] % G_WC != 0 && g.cend[r] < g.N) return MTFM_E_UNSUPPORTED;
        if (g.dst[r] && (!aligned16(g.dst[r]) || g.ld[r] % 8 != 0)) return MTFM_E_UNSUPPORTED;
      }
      if (g.pre && (!aligned16(g.pre) || g.ldpre % 8 != 0)) return MTFM_E_UNSUPPORTED;
      if (g.vt) {
        // rows map to themselves; whole 64-column wave tiles; slots up to ldvt covered by the grid
        // (groups: each its own copy at vt_zstride, covering its rows)
        if (g.amap.list || g.cmap.list || g.cmap.mul != 1 || g.cmap.add != 0) return MTFM_E_UNSUPPORTED;
        if (g.groups != 1 && (g.vt_zstride < (int64_t)g.vt_cols * g.ldvt || g.vt_zstride % 8 != 0))
          return MTFM_E_UNSUPPORTED;
        if (g.vt_col0 % G_WC != 0 || g.vt_cols % G_WC != 0 || !aligned16(g.vt) || g.ldvt % 64 != 0) return MTFM_E_UNSUPPORTED;
        if (g.ldvt < g.M) return MTFM_E_UNSUPPORTED;
      }
    } else if (g.epi == EPI_SWIGLU) {
      if (g.N % G_WC != 0 || ((uintptr_t)g.out & 7) || g.ldo % 4 != 0) return MTFM_E_UNSUPPORTED;
    } else {
      if (!aligned16(g.out) || g.ldo % 8 != 0) return MTFM_E_UNSUPPORTED;
      if (g.epi == EPI_RESID && (!aligned16(g.resid) || g.ldr % 8 != 0)) return MTFM_E_UNSUPPORTED;
    }
    // 256-row tiles unless they would not give every workgroup slot a tile
    const int64_t n_nt = (g.N + GBN - 1) / GBN;
    const int64_t tiles256 = (int64_t)((g.M + 255) / 256) * n_nt * g.groups;
    const bool small = tiles256 < 2 * (int64_t)GShape<256>::WG_PER_CU * device_cu_count();
    const int bm = small ? 128 : 256;
    if (g.vt && g.ldvt > (int64_t)((g.M + bm - 1) / bm) * bm) return MTFM_E_UNSUPPORTED;
    const int64_t tiles = (int64_t)((g.M + bm - 1) / bm) * n_nt * g.groups;
    if (tiles > 0x7fffffff) return MTFM_E_UNSUPPORTED;
    const dim3 grid((unsigned)tiles, 1, 1);
    if (g.bs24) {
      switch (g.epi * 2 + (small ? 1 : 0)) {
        case 2 * EPI_SILU_SPLIT: gemm_bf16_kernel<EPI_SILU_SPLIT, 256, true><<<grid, 256, 0, s>>>(g); break;
        case 2 * EPI_SILU_SPLIT + 1: gemm_bf16_kernel<EPI_SILU_SPLIT, 128, true><<<grid, 256, 0, s>>>(g); break;
        case 2 * EPI_RESID: gemm_bf16_kernel<EPI_RESID, 256, true><<<grid, 256, 0, s>>>(g); break;
        case 2 * EPI_RESID + 1: gemm_bf16_kernel<EPI_RESID, 128, true><<<grid, 256, 0, s>>>(g); break;
        default: return MTFM_E_UNSUPPORTED;   // the forward projections use these two epilogues
      }
      MTFM_LAUNCH_CHECK("gemm_s24");
      return MTFM_OK;
    }
    if (tiles < device_cu_count() && (g.epi == EPI_SILU_SPLIT || g.epi == EPI_RESID)) {
      // fewer workgroups than CUs (a few hundred rows): the four-stage ring
      if (g.epi == EPI_SILU_SPLIT) gemm_bf16_kernel<EPI_SILU_SPLIT, 128, false, 4><<<grid, 256, 0, s>>>(g);
      else gemm_bf16_kernel<EPI_RESID, 128, false, 4><<<grid, 256, 0, s>>>(g);
      MTFM_LAUNCH_CHECK("gemm");
      return MTFM_OK;
    }
    switch (g.epi * 2 + (small ? 1 : 0)) {
      case 2 * EPI_SILU_SPLIT: gemm_bf16_kernel<EPI_SILU_SPLIT, 256, false><<<grid, 256, 0, s>>>(g); break;
      case 2 * EPI_SILU_SPLIT + 1: gemm_bf16_kernel<EPI_SILU_SPLIT, 128, false><<<grid, 256, 0, s>>>(g); break;
      case 2 * EPI_RESID: gemm_bf16_kernel<EPI_RESID, 256, false><<<grid, 256, 0, s>>>(g); break;
      case 2 * EPI_RESID + 1: gemm_bf16_kernel<EPI_RESID, 128, false><<<grid, 256, 0, s>>>(g); break;
      case 2 * EPI_STORE_F32: gemm_bf16_kernel<EPI_STORE_F32, 256, false><<<grid, 256, 0, s>>>(g); break;
      case 2 * EPI_STORE_F32 + 1: gemm_bf16_kernel<EPI_STORE_F32, 128, false><<<grid, 256, 0, s>>>(g); break;
      case 2 * EPI_SWIGLU: gemm_bf16_kernel<EPI_SWIGLU, 256, false><<<grid, 256, 0, s>>>(g); break;
      case 2 * EPI_SWIGLU + 1: gemm_bf16_kernel<EPI_SWIGLU, 128, false><<<grid, 256, 0, s>>>(g); break;
      case 2 * EPI_STORE: gemm_bf16_kernel<EPI_STORE, 256, false><<<grid, 256, 0, s>>>(g); break;
      default: gemm_bf16_kernel<EPI_STORE, 128, false><<<grid, 256, 0, s>>>(g); break;
    }
  } else {
    if (g.epi == EPI_SWIGLU || g.bs24 || g.bgroup[0] || (g.vt && g.groups != 1)) return MTFM_E_UNSUPPORTED;
    const int64_t total = (int64_t)g.M * g.N;
    gemm_f32_kernel<<<dim3((unsigned)((total + 255) / 256), 1, g.groups), 256, 0, s>>>(g);
  }
  MTFM_LAUNCH_CHECK("gemm");
  return MTFM_OK;
}
