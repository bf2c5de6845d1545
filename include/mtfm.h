/*
 * mtfm.h - C ABI of libmtfm, the MI355X (gfx950) hot path of the hybrid
 * H/R/T masked-attention backbone.
 *
 * Pages cited (titles; sections as numbered on each page):
 *   [explainer] "美团推荐大模型 MTFM (Meituan Foundation Model) 深度硬核解析：跨场景推荐的终极答案？"
 *               (dingyadong.top)
 *   [blog]      "MTFM：美团统一推荐基座大模型在外卖多业务场景的落地实践" (Meituan tech blog,
 *               mirrored on dujian.net)
 *   [digest]    "外卖几条业务线共用一套精排骨干：美团 MTFM 免掉跨业务特征对齐，推理成本降 24%"
 *               (neodrop.ai)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Pointers named *_d are device pointers; *_h are host pointers.  The
 *    caller owns every buffer; the library never allocates device memory.
 *    Scratch space comes from a caller-provided workspace sized by
 *    mtfm_workspace_bytes(); per-batch mask metadata lives in a caller
 *    buffer sized by mtfm_meta_bytes().
 *  - All work is enqueued on `stream` (a hipStream_t; NULL = the null
 *    stream) and is asynchronous: no entry point synchronises the host or
 *    reads device memory back.  Grid sizes come from the host copy of the
 *    per-user lengths.
 *  - Arguments are validated on the host before anything is enqueued.  A
 *    status other than MTFM_OK means nothing was enqueued, except
 *    MTFM_E_HIP, which reports a failed launch (work enqueued before it may
 *    have run).
 *  - Data-level contracts are the caller's: action times ascending within
 *    each user, device lengths equal to the host lengths.
 *  - Rows of one user are packed H, R, T ([explainer] §2.1.3: X = (H; R; T));
 *    users follow one another with no padding ("jagged": [blog] §6.1).  With
 *    split S = 4 ([blog] §3.3.2, V2 target scale-up) each target parent
 *    contributes 4 consecutive T rows (target-major), all carrying that
 *    parent's exposure time.
 *  - Activations and projection weights have the layer's dtype (fp32 or
 *    bf16, row-major); group-LayerNorm parameters are always fp32.
 *  - Re-entrant for distinct workspaces and streams.
 */
#ifndef MTFM_H
#define MTFM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MTFM_OK = 0,
  MTFM_E_NULL = -1,        /* a required pointer is NULL */
  MTFM_E_DIMS = -2,        /* a size is negative, inconsistent or too large */
  MTFM_E_UNSUPPORTED = -3, /* valid, but not implemented (head_dim, H % G, split, dtype) */
  MTFM_E_WORKSPACE = -4,   /* meta or workspace buffer smaller than required */
  MTFM_E_HIP = -5          /* a HIP launch or runtime call failed */
} mtfm_status;

typedef enum { MTFM_F32 = 0, MTFM_BF16 = 1 } mtfm_dtype;

/* Query/key tile edge used by the mask metadata and the attention kernels. */
#define MTFM_TILE 64

/* A jagged user-level batch ([explainer] §3; [blog] §4.1: one sample per user
 * holding its history H, real-time actions R and exposed targets T). */
typedef struct {
  int32_t n_users;
  int32_t split;          /* T rows per target parent: 1 (V1) or 4 (V2) */
  const int32_t* lens_h;  /* host   [n_users][3] = {L_H, L_R, L_T parents}, all >= 0 */
  const int32_t* lens_d;  /* device copy of lens_h */
  const int32_t* ts_r_d;  /* device [sum L_R] action times, ascending within each user */
  const int32_t* ts_t_d;  /* device [sum L_T] exposure time of each target parent */
} mtfm_batch;

/* Layer shape.  H query heads share G key/value heads, r = H / G
 * ([explainer] §4.1, grouped-query attention). */
typedef struct {
  int32_t d_model;
  int32_t n_q_heads;   /* H */
  int32_t n_kv_heads;  /* G; H % G == 0 */
  int32_t head_dim;    /* dh: 32 or 64 */
  float ln_eps;        /* group-LayerNorm epsilon (the pages fix none; 1e-5 is used) */
  int32_t dtype;       /* mtfm_dtype of activations and projection weights */
} mtfm_dims;

/* Full-attention layer weights ([explainer] §4.1):
 *   X~ = GLN1(X);  [U|Q|K|V] = SiLU(X~ w_uqkv^T);  A_h = SiLU(Q_h K_g^T / sqrt(dh)) (.) M V_g / n
 *   X' = (GLN2(A) (.) U) w_o^T + X
 * GLN = LayerNorm over the row with affine parameters picked by the row's
 * token type H/R/T ([blog] §6.1: a [G, D] parameter matrix indexed per token). */
typedef struct {
  const float* ln1_g; const float* ln1_b;  /* [3][d_model], rows H, R, T */
  const void* w_uqkv;                      /* [2*H*dh + 2*G*dh][d_model], rows U|Q|K|V, heads contiguous */
  const float* ln2_g; const float* ln2_b;  /* [3][H*dh] */
  const void* w_o;                         /* [d_model][H*dh] */
  /* Optional 2:4 structured-sparse projections ([explainer] §5.2.1; bf16
   * only): if set, the forward and serving entry points compute that
   * projection with the pruned weights on the sparse matrix instructions
   * instead of reading the dense matrix.  Each is mtfm_s24_pack of the dense
   * matrix above (the pack prunes).  NULL = dense.  A set field must be
   * 16-byte aligned and needs bf16 dims (else E_UNSUPPORTED, checked before
   * anything is enqueued).  The backward entry points ignore them (training
   * keeps dense weights). */
  const void* w_uqkv_s24;                  /* pack of w_uqkv ([2*H*dh + 2*G*dh] rows, K = d_model) */
  const void* w_o_s24;                     /* pack of w_o ([d_model] rows, K = H*dh) */
} mtfm_full_w;

/* Target-attention layer weights ([explainer] §4.2; [blog] §3.3.2 per-sub-token Q):
 *   X~ = GLN1(X);  [K|V] = SiLU(X~ w_kv^T) on all rows;
 *   U_T = SiLU(X~_T w_u^T), Q_T = SiLU(X~_T w_q[k]^T) for sub-token k;
 *   X'_T = (GLN2(A_T) (.) U_T) w_o^T + X_T;  X'_{H,R} = X_{H,R}. */
typedef struct {
  const float* ln1_g; const float* ln1_b;  /* [3][d_model] */
  const void* w_u;                         /* [H*dh][d_model] */
  const void* w_q;                         /* [split][H*dh][d_model] */
  const void* w_kv;                        /* [2*G*dh][d_model], rows K|V */
  const float* ln2_g; const float* ln2_b;  /* [3][H*dh] */
  const void* w_o;                         /* [d_model][H*dh] */
  /* Optional 2:4 structured-sparse projections, as in mtfm_full_w: */
  const void* w_t_s24;                     /* pack of the T-row stack, per sub-token k = 0 .. split-1 the
                                              segments w_u, w_q[k], w_kv (split * (2*H*dh + 2*G*dh) rows) */
  const void* w_kv_s24;                    /* pack of w_kv (context rows' K|V) */
  const void* w_o_s24;                     /* pack of w_o */
} mtfm_target_w;

/* Gradients written by the backward entry points.  Weight and GLN-parameter
 * gradients are fp32 and overwritten (not accumulated); shapes as in the
 * matching weight struct. */
typedef struct {
  float* ln1_g; float* ln1_b; float* w_uqkv; float* ln2_g; float* ln2_b; float* w_o;
} mtfm_full_grad;

typedef struct {
  float* ln1_g; float* ln1_b; float* w_u; float* w_q; float* w_kv; float* ln2_g; float* ln2_b; float* w_o;
} mtfm_target_grad;

/* Byte offsets of the arrays inside the mask-metadata buffer (host-side
 * description; counts are element counts). */
typedef struct {
  int64_t n_rows;            /* total packed rows */
  int64_t n_t_rows;          /* total T rows (split * sum L_T) */
  int64_t n_parents;         /* sum L_T */
  int64_t n_ctx_rows;        /* total H + R rows */
  int64_t n_full_tiles;      /* query tiles of the full layer: sum ceil(N_u / 64) */
  int64_t n_target_tiles;    /* query tiles of the target layer: sum ceil(split L_T / 64) */
  int64_t n_key_tiles;       /* 64-key tiles of the users' context (H + R) rows */
  int64_t off_user;          /* int32 [8][n_users + 1]: row, action, parent, ctx-row, full-tile,
                                target-tile, T-row and context key-tile offsets of each user */
  int64_t off_p;             /* int32 [n_rows] visible context prefix p_i */
  int64_t off_n;             /* int32 [n_rows] visible key count n_i (p_i + self_i) */
  int64_t off_type;          /* uint8 [n_rows] token type 0 = H, 1 = R, 2 = T */
  int64_t off_full_tiles;    /* int32 [n_full_tiles][8] tile descriptors (below) */
  int64_t off_target_tiles;  /* int32 [n_target_tiles][8] */
  int64_t off_ctx_rows;      /* int32 [n_ctx_rows] packed row of each H/R row, users in order */
  int64_t off_parent_row;    /* int32 [n_parents] packed row of each parent's first T row */
  int64_t n_full_order;      /* work-order entries of the full / target layer's attention grid */
  int64_t n_target_order;    /*   (0 for batches over 2048 users: plain order) */
  int64_t off_full_order;    /* int32 [n_full_order]: entry 8 k + x = 2 tile + half of the k-th */
  int64_t off_target_order;  /*   32-row query slice XCD x takes, -1 past the end of its list */
  int64_t off_tsort_q;       /* int32 [n_t_rows]: each user's T rows in ascending order of their */
  int64_t off_tsort_g;       /*   prefix p (ties by row): T-row index / packed row at each position */
  int64_t off_target_tiles_sorted;  /* int32 [n_target_tiles][8]: target tiles over those positions */
  int64_t total_bytes;
} mtfm_meta_layout;
/* Tile descriptor, int32 x 8:
 *   [0] user, [1] first query row within the user, [2] rows in the tile (<= 64),
 *   [3] leading key tiles that are fully visible to every row of the tile,
 *   [4] one past the last key tile with any visible key,
 *   [5] packed row of the first query row, [6] row of the first query in the
 *   layer's query space (= [5] for the full layer; the T-row index for the
 *   target layer), [7] packed row of the user's first row.
 * Key tiles cover the user's context columns (H then R) from its first row in
 * steps of 64; tiles [0, [3]) are all visible, [[3], [4]) mixed, the rest
 * invisible.  A T row's only T key is itself, carried by n_i - p_i = 1. */

/* ---------------------------------------------------------------------------
 * Mask metadata ([explainer] §4.1.1 and the worked matrix of §8.2; [blog]
 * §3.2): H keys are visible to every query; H queries see only H; R queries
 * see H and R up to themselves (causal, self included); T queries see H, the
 * R actions strictly earlier than their exposure time, and themselves.
 * [blog] §6.1 preprocesses the mask into a one-dimensional jagged form and
 * §6.2 pre-scans it into an index of key blocks worth computing; here that is
 * the per-row prefix p_i plus the tile descriptors above.
 */

/* Bytes of metadata for this batch (0 on invalid arguments). */
size_t mtfm_meta_bytes(const mtfm_batch* batch);

/* Fill *layout with the array offsets of the metadata buffer.  Host only. */
mtfm_status mtfm_meta_layout_of(const mtfm_batch* batch, mtfm_meta_layout* layout);

/* Build the metadata of `batch` into meta_d (device, meta_bytes >= mtfm_meta_bytes).
 * Integer-only; the result is a pure function of lengths and timestamps and
 * is shared by every layer of a backbone.  Errors: E_NULL, E_DIMS (negative
 * lengths, split not 1 or 4, more than 2^31 - 1 rows), E_WORKSPACE, E_HIP. */
mtfm_status mtfm_mask_build(const mtfm_batch* batch, void* meta_d, size_t meta_bytes, void* stream);

/* Debug, tiny batches only: the dense visibility matrix of one user,
 * mask_d[i * N + j] = 1 if query row i of the user sees key row j (rows in the
 * user's packed order H, R, T; N = L_H + L_R + split * L_T), from the
 * metadata alone: a context key j < L_H + L_R is visible iff j < p_i, a T key
 * only to itself ([explainer] §8.2's worked matrix; [blog] §3.2).  mask_d:
 * device uint8 [N][N], caller-owned.  Errors: E_NULL, E_DIMS (no such user,
 * N^2 too large), E_HIP. */
mtfm_status mtfm_mask_dense(const mtfm_batch* batch, const void* meta_d, int32_t user, uint8_t* mask_d,
                            void* stream);

/* Debug: checks the batch's data-level contracts on the device and writes a
 * bit mask of the violations found to *flags_d (device int32; 0 = none):
 * MTFM_BAD_ACTION_ORDER if some user's action times do not ascend,
 * MTFM_BAD_LENGTHS if the device lengths differ from the host lengths (a
 * negative length, another total, or a mismatch of an order-sensitive hash of
 * the per-user lengths).  Reads only within the sizes the host lengths give,
 * whatever the device holds.  One workgroup; not meant for the hot path.
 * Errors: E_NULL, E_DIMS, E_HIP. */
#define MTFM_BAD_ACTION_ORDER 1
#define MTFM_BAD_LENGTHS 2
mtfm_status mtfm_validate_batch(const mtfm_batch* batch, int32_t* flags_d, void* stream);

/* ---------------------------------------------------------------------------
 * Layers.  x_in / x_out: device [n_rows][d_model] of dims->dtype.  meta_d:
 * the output of mtfm_mask_build for the same batch.  ws: device workspace of
 * at least mtfm_workspace_bytes(batch, dims, op) bytes.
 * Supported: head_dim 64 with bf16 (MFMA path; H / G of 1, 2, 4 or 8),
 * head_dim 32 or 64 with fp32; d_model and H * dh each one of 64, 128, 256,
 * 512 or 1024; H % G == 0.  Other shapes return MTFM_E_UNSUPPORTED before
 * anything is enqueued.  The backward entry points (bf16 only) further need
 * d_model and H * dh in {256, 512, 1024}.
 */
typedef enum {
  MTFM_OP_FULL = 0, MTFM_OP_TARGET = 1, MTFM_OP_BACKBONE = 2,
  MTFM_OP_FULL_BWD = 3, MTFM_OP_TARGET_BWD = 4
} mtfm_op;

size_t mtfm_workspace_bytes(const mtfm_batch* batch, const mtfm_dims* dims, int32_t op);

/* Byte offsets, inside the workspace, of the attention output A (before
 * GLN2, already divided by n) and of the gated Y = GLN2(A) (.) U left by the
 * last mtfm_attn_full / mtfm_attn_target call: [n_rows][H*dh] for the full
 * layer, [n_t_rows][H*dh] in T-row order for the target layer, in
 * dims->dtype.  Lets a caller check the attention and gating branches
 * separately.  (On the bf16 path the full layer's attention kernel applies
 * the gated GLN2 itself and stores A only for these single-layer calls.)
 * Host only. */
mtfm_status mtfm_workspace_probe(const mtfm_batch* batch, const mtfm_dims* dims, int32_t op,
                                 int64_t* off_a, int64_t* off_y);

/* Full-attention layer ([explainer] §4.1).  x_out may equal x_in. */
mtfm_status mtfm_attn_full(const mtfm_batch* batch, const mtfm_dims* dims, const void* meta_d,
                           const mtfm_full_w* w, const void* x_in, void* x_out,
                           void* ws, size_t ws_bytes, void* stream);

/* Target-attention layer ([explainer] §4.2): only T rows query; keys and
 * values come from every row under the mask's T rows; H and R rows of x_out
 * are copies of x_in (bit-exact).  x_out may equal x_in (then only T rows are
 * written). */
mtfm_status mtfm_attn_target(const mtfm_batch* batch, const mtfm_dims* dims, const void* meta_d,
                             const mtfm_target_w* w, const void* x_in, void* x_out,
                             void* ws, size_t ws_bytes, void* stream);

/* Hybrid backbone ([explainer] §4: B blocks of 1 full + K target layers;
 * [blog] §3.3.1: 16 layers = 4 x (1 + 3)).  full: [n_blocks] weights,
 * tgt: [n_blocks * k_target] weights in layer order.  In place on x_inout.
 * The metadata is built once per batch by the caller and reused by all layers. */
mtfm_status mtfm_backbone_fwd(const mtfm_batch* batch, const mtfm_dims* dims, int32_t n_blocks,
                              int32_t k_target, const void* meta_d, const mtfm_full_w* full,
                              const mtfm_target_w* tgt, void* x_inout, void* ws, size_t ws_bytes,
                              void* stream);

/* Workspace for mtfm_backbone_fwd with k_target target layers per block.
 * On the bf16 path with 1 <= k_target <= 4, the normalised context (H and R)
 * rows and the K/V of all target layers of a block are computed right after
 * the block's full layer, from one read of its output (a target layer never
 * changes H or R rows); each target layer then normalises only its T rows.
 * That needs this much workspace; with less (but at least
 * mtfm_workspace_bytes(batch, dims, MTFM_OP_BACKBONE)) the layers run one by
 * one.  Both orders compute the same values bit for bit, except with few T
 * rows against long contexts: there the hoisted order splits each T slice's
 * keys in the target attention over several workgroups (fp32 partials added
 * in a fixed order by the following normalisation), which agrees with the
 * one-by-one order to rounding.  Everything runs on `stream`.  Returns 0 on
 * invalid arguments.
 * Host only. */
size_t mtfm_backbone_workspace_bytes(const mtfm_batch* batch, const mtfm_dims* dims, int32_t k_target);

/* Backward of one full-attention layer: given x_in (the layer's input) and
 * dy = dL/dX', writes dx = dL/dX ([n_rows][d_model], dims->dtype) and the
 * fp32 weight/GLN gradients into *g.  Recomputes the forward internally.
 * dx must not alias x_in or dy. */
mtfm_status mtfm_attn_full_bwd(const mtfm_batch* batch, const mtfm_dims* dims, const void* meta_d,
                               const mtfm_full_w* w, const void* x_in, const void* dy, void* dx,
                               const mtfm_full_grad* g, void* ws, size_t ws_bytes, void* stream);

/* Backward of one target-attention layer, same conventions. */
mtfm_status mtfm_attn_target_bwd(const mtfm_batch* batch, const mtfm_dims* dims, const void* meta_d,
                                 const mtfm_target_w* w, const void* x_in, const void* dy, void* dx,
                                 const mtfm_target_grad* g, void* ws, size_t ws_bytes, void* stream);

/* Backward of the whole backbone (the training step's gradient pass): the
 * stack of mtfm_backbone_fwd, n_blocks x (1 full + k_target target layers)
 * ([explainer] §4; [blog] §3.3.1), differentiated layer by layer with the
 * chain rule.  Given x_in (the backbone's input) and dy = dL/dX_out, writes
 * dx = dL/dX_in and every layer's fp32 weight/GLN gradients (overwritten):
 * full_g[b] for the full layer of block b, tgt_g[b * k_target + t] for its
 * target layer t.  One forward pass keeps the inputs of layers 1 .. L-1 in
 * the workspace (bf16, as the forward passes them on); then each layer's
 * backward runs from the last to the first, the gradient handed between
 * layers stored in dims->dtype.  dx also serves as one of the two
 * intermediate gradient buffers, so it must not alias x_in or dy.
 * bf16 only (MTFM_E_UNSUPPORTED otherwise).
 * Workspace, two sizes: with at least
 * mtfm_backbone_bwd_workspace_bytes(batch, dims, n_blocks, k_target) bytes the
 * forward pass also keeps each layer's intermediates (normalised input,
 * projections and their pre-activations, attention output; about 21 GiB for
 * 160 users of ~1,500 rows at d_model 512), so no layer backward recomputes
 * them; with at
 * least mtfm_backbone_bwd_min_workspace_bytes(...) bytes (but less than the
 * full size) each layer backward recomputes them.  Both give the same
 * gradients bit for bit.  Fewer bytes than the minimum: MTFM_E_WORKSPACE.
 * Stream-ordered, no host synchronisation. */
size_t mtfm_backbone_bwd_workspace_bytes(const mtfm_batch* batch, const mtfm_dims* dims, int32_t n_blocks,
                                         int32_t k_target);
size_t mtfm_backbone_bwd_min_workspace_bytes(const mtfm_batch* batch, const mtfm_dims* dims, int32_t n_blocks,
                                             int32_t k_target);
mtfm_status mtfm_backbone_bwd(const mtfm_batch* batch, const mtfm_dims* dims, int32_t n_blocks, int32_t k_target,
                              const void* meta_d, const mtfm_full_w* full, const mtfm_target_w* tgt,
                              const void* x_in, const void* dy, void* dx, const mtfm_full_grad* full_g,
                              const mtfm_target_grad* tgt_g, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * V2 target side ([blog] §3.3.2 "Target Scale-Up"): a target becomes S = 4
 * sub-token rows (AutoSplit), every target layer gives each sub-token its own
 * SwiGLU FFN, RankMixer's zero-parameter token mixing crosses the sub-tokens,
 * and mean pooling ends the target side.  The page gives no formulas; the
 * readings: AutoSplit is a bias-free linear map of a parent's feature vector
 * to S * d_model values, sub-token z taking columns [z d, (z + 1) d); the FFN
 * is pre-normalised and residual,
 *   X_T <- X_T + W_down[z] (SiLU(W_gate[z] X~) (.) (W_up[z] X~)),
 *   X~ = LayerNorm(X_T) (biased variance, eps = dims->ln_eps) * ln_g[T] + ln_b[T],
 * bias-free, hidden width d_ff, applied to the T rows after each target layer
 * and followed by the mixing: each sub-token row is cut into S chunks of
 * d_model / S, and sub-token c becomes the concatenation over z = 0..S-1 of
 * chunk c of sub-token z (S = 1: nothing).  Pooling: one row per parent, the
 * mean of its S sub-token rows.  bf16 only; d_ff a multiple of 32; d_model / S
 * a multiple of 8. */
typedef struct {
  const float* ln_g; const float* ln_b;  /* [3][d_model]; the T row is used */
  const void* w_gate;                    /* [split][d_ff][d_model] */
  const void* w_up;                      /* [split][d_ff][d_model] */
  const void* w_down;                    /* [split][d_model][d_ff] */
} mtfm_ffn_w;

/* AutoSplit: feats [n_parents][d_in] (parents in batch order), w_split
 * [split * d_model][d_in] -> the T rows of x ([n_rows][d_model] packed rows;
 * only T rows are written).  d_in a multiple of 32. */
mtfm_status mtfm_autosplit(const mtfm_batch* batch, const mtfm_dims* dims, int32_t d_in, const void* meta_d,
                           const void* feats, const void* w_split, void* x, void* stream);

/* One target layer's token FFN and mixing on the T rows of x (packed rows, in
 * place); ws: mtfm_token_ffn_workspace_bytes. */
size_t mtfm_token_ffn_workspace_bytes(const mtfm_batch* batch, const mtfm_dims* dims, int32_t d_ff);
mtfm_status mtfm_token_ffn(const mtfm_batch* batch, const mtfm_dims* dims, int32_t d_ff, const void* meta_d,
                           const mtfm_ffn_w* w, void* x, void* ws, size_t ws_bytes, void* stream);

/* Mean pooling of each parent's sub-token rows of x into out [n_parents][d_model]. */
mtfm_status mtfm_token_pool(const mtfm_batch* batch, const mtfm_dims* dims, const void* meta_d, const void* x,
                            void* out, void* stream);

/* The V2 stack: mtfm_backbone_fwd's n_blocks x (1 full + k_target target
 * layers) with, after every target layer, that layer's token FFN and mixing
 * (ffn[b * k_target + t]).  1 <= k_target <= 4; ws:
 * mtfm_backbone_v2_workspace_bytes. */
size_t mtfm_backbone_v2_workspace_bytes(const mtfm_batch* batch, const mtfm_dims* dims, int32_t k_target,
                                        int32_t d_ff);
mtfm_status mtfm_backbone_v2_fwd(const mtfm_batch* batch, const mtfm_dims* dims, int32_t n_blocks, int32_t k_target,
                                 int32_t d_ff, const void* meta_d, const mtfm_full_w* full, const mtfm_target_w* tgt,
                                 const mtfm_ffn_w* ffn, void* x_inout, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Request-level serving with user-side K/V reuse ([explainer] §5.2.3: K/V
 * cache sharing across serving micro-batches; [blog] §3.4 and §4: one
 * user-level sample shares the long-sequence attention among its targets).
 * H and R rows never attend to T rows, so the context rows' values through
 * the stack and every layer's K and V of them do not depend on the
 * candidates.  Split the backbone in two:
 *
 *   mtfm_serve_context: once per set of users.  `batch` holds the users'
 *     context only (L_T = 0 for every user; lens and R timestamps as in the
 *     candidate batches to come).  Runs the stack of mtfm_backbone_fwd over
 *     the context rows (x_inout [n_rows][d_model], updated in place) and
 *     writes each layer's K and V^T of those rows into kv_cache.
 *   mtfm_serve_targets: per candidate batch.  `batch` holds the same users
 *     with the same L_H, L_R and R timestamps, plus any number of candidate
 *     parents L_T with their exposure times; meta_d is its mask metadata.
 *     x_t is [split * sum L_T][d_model] in T-row order (sub-token z of parent
 *     m at row m * split + z), updated in place through all layers, each T row
 *     attending to the cached context K/V of its user (visible prefix from
 *     the mask) and to itself.
 *
 * The T rows come out as mtfm_backbone_fwd would leave them for the batch
 * holding context and candidates together, to rounding (the cache packs the
 * context rows without the T rows between users, so the attention groups its
 * keys differently).  With few candidates against long contexts the target
 * attention splits each 32-row slice's keys over several workgroups (fp32
 * partials added in a fixed order by the following normalisation; up to 16
 * MiB of the workspace).  Cache layout, per layer l
 * in stack order (block b's full layer, then its target layers): K
 * [n_ctx_rows][G*dh], then V^T [G*dh][ldvt] with ldvt = n_ctx_rows rounded up
 * to 64 (bf16, 256-byte aligned pieces); context rows of all users back to
 * back, users in order.  bf16 only, k_target <= 4.  The caller owns the
 * cache; overlapping calls on the same cache or workspace race. */
typedef enum { MTFM_SERVE_CONTEXT = 0, MTFM_SERVE_TARGETS = 1 } mtfm_serve_phase;

size_t mtfm_kv_cache_bytes(const mtfm_batch* batch, const mtfm_dims* dims, int32_t n_blocks, int32_t k_target);
size_t mtfm_serve_workspace_bytes(const mtfm_batch* batch, const mtfm_dims* dims, int32_t k_target, int32_t phase);
mtfm_status mtfm_serve_context(const mtfm_batch* batch, const mtfm_dims* dims, int32_t n_blocks, int32_t k_target,
                               const void* meta_d, const mtfm_full_w* full, const mtfm_target_w* tgt,
                               void* x_inout, void* kv_cache, size_t cache_bytes, void* ws, size_t ws_bytes,
                               void* stream);
mtfm_status mtfm_serve_targets(const mtfm_batch* batch, const mtfm_dims* dims, int32_t n_blocks, int32_t k_target,
                               const void* meta_d, const mtfm_full_w* full, const mtfm_target_w* tgt,
                               const void* kv_cache, size_t cache_bytes, void* x_t, void* ws, size_t ws_bytes,
                               void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the
 * candidate pass of mtfm_serve_targets with the same arguments except the
 * workspace, which comes from a static device array inside the library, one
 * per GPU, of mtfm_serve_targets_noalloc_max_bytes() bytes (64 MiB: about
 * 11,900 T rows at d_model = H*dh = 512, G*dh = 128).  Computes exactly what
 * mtfm_serve_targets computes (same kernels and shapes, bit for bit).  Calls
 * no allocating routine; kernel timing (mtfm_timing_enable) is suspended
 * during the call.  A batch needing more than the array holds returns
 * MTFM_E_WORKSPACE before anything is enqueued.  The array is looked up on
 * the first call on each device; `stream` must belong to the current device
 * (else MTFM_E_UNSUPPORTED).  Every call on one GPU shares that GPU's array:
 * calls that overlap on one GPU (other host threads or streams) race; calls
 * ordered on one stream do not. */
size_t mtfm_serve_targets_noalloc_max_bytes(void);
mtfm_status mtfm_serve_targets_noalloc(const mtfm_batch* batch, const mtfm_dims* dims, int32_t n_blocks,
                                       int32_t k_target, const void* meta_d, const mtfm_full_w* full,
                                       const mtfm_target_w* tgt, const void* kv_cache, size_t cache_bytes, void* x_t,
                                       void* stream);

/* ---------------------------------------------------------------------------
 * Kernel timing (measurement aid).  While a kernel class is enabled, each of
 * its launches is bracketed by two HIP events recorded on the stream the
 * kernel is launched on; nothing else changes.  mtfm_timing_read waits for
 * the recorded events of one class, returns the number of launches and their
 * summed duration in milliseconds since the previous read, and resets that
 * class.  Process-wide state, guarded by a mutex.
 */
typedef enum {
  MTFM_K_MASK = 0,         /* mask-metadata builder */
  MTFM_K_GLN = 1,          /* group LayerNorm over all rows: the full layer's pre-norm (and its
                              gated post-norm on the fp32 path), the backward's and V2's */
  MTFM_K_GEMM_UQKV = 2,    /* full layer: U|Q|K|V projection */
  MTFM_K_ATTN_FULL = 3,    /* full layer: masked attention */
  MTFM_K_GEMM_OUT = 4,     /* full layer: output projection + residual (all rows) */
  MTFM_K_GEMM_KV = 5,      /* target layer: K|V projection of the H/R rows */
  MTFM_K_GEMM_T = 6,       /* target layer: U|Q|K|V projection of the T rows */
  MTFM_K_ATTN_TARGET = 7,  /* target layer: masked attention */
  MTFM_K_BWD = 8,          /* backward kernels */
  MTFM_K_V2 = 9,           /* V2 target side: AutoSplit, token FFN, mixing, pooling */
  MTFM_K_GLN_T = 10,       /* target layers: context pre-norm of a block's target layers, T-row
                              pre-norm and gated post-norm (also serving's T-row passes) */
  MTFM_K_GEMM_OUT_T = 11,  /* output projection + residual of the T rows (target layers, serving) */
  MTFM_K_COUNT = 12
} mtfm_kernel_class;

mtfm_status mtfm_timing_enable(uint32_t class_mask);  /* bit k enables class k; 0 disables all */
mtfm_status mtfm_timing_read(int32_t kernel_class, int64_t* launches, double* total_ms);

/* Human-readable name of a status. */
const char* mtfm_status_str(int32_t status);

/* Last HIP error text recorded by this thread (empty if none). */
const char* mtfm_last_error(void);

/* ---------------------------------------------------------------------------
 * 2:4 structured pruning and packing ([explainer] §5.2.1: in the linear
 * projections, of every 4 consecutive weights the 2 smaller are set to zero
 * for sparse matrix hardware).
 *
 * Groups of 4 run along a weight row (the reduction axis of y = x W^T).  A
 * group keeps its 2 entries of largest magnitude; of equal magnitudes the
 * lower position is kept.  The packed matrix holds, for the rows of the
 * given segments stacked in order (R rows, K columns, bf16, row-major, each
 * segment 16-byte aligned), the kept values and their positions in the
 * operand order of the sparse matrix instruction (K step ks = k / 32, slice
 * i = (ks * R + r) * 2 + h for half h = 0, 1 covering the groups q of the step
 * with q % 4 in {2h, 2h + 1}):
 *   byte i * 16: 8 bf16, the two kept entries of each of those 4 groups in
 *                ascending q, each pair in ascending position;
 *   byte R * K + i * 2: uint16, 2 bits per kept entry (its position 0..3 in
 *                its group), entry j at bits 2j .. 2j + 1.
 * The layout is what the forward kernels read; it is stated so that tests
 * can decode it.  K % 32 == 0, at most 16 segments. */
size_t mtfm_s24_pack_bytes(int32_t rows, int32_t k);   /* R * K * 9 / 8; 0 if k % 32 != 0 or a size <= 0 */
/* w_segs / seg_rows: host arrays of n_segs device pointers and row counts.
 * packed: device buffer of at least mtfm_s24_pack_bytes(sum rows, k) bytes
 * (else E_WORKSPACE), 16-byte aligned; caller-owned.  Enqueued on stream; the
 * sources must stay valid until it runs.  E_NULL, E_DIMS (k % 32, segment
 * count or rows), E_UNSUPPORTED (alignment), E_HIP. */
mtfm_status mtfm_s24_pack(const void* const* w_segs, const int32_t* seg_rows, int32_t n_segs, int32_t k,
                          void* packed, size_t packed_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MTFM_H */
