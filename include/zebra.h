/*
 * zebra.h -- C ABI of libzebra: the global multi-view attention stage of a
 * Zebra3D-style hybrid 3D reconstruction model, for AMD MI355X (gfx950).
 *
 * Source pages: "How Hybrid Attention Lets Feed-Forward 3D Models Scale to
 * Many Views" (wispaper.ai) and its translations. A global stage is either
 *   (a) tile-sparse softmax attention ("Linear-centered stages plus
 *       tile-sparse stages"): 8x8-patch key tiles, a selector keeping a
 *       key-tile fraction 1 - y per query tile, mean-K/V landmarks for the
 *       omitted tiles, special keys always visible, special query rows
 *       dense, every patch query keeps its self key; or
 *   (b) linear attention ("Speedup scales with the number of input views"):
 *       fused Q/K normalisation, 2D rotary and channel-softmax feature map,
 *       then the centred affine output correction ("A closed-form fit avoids
 *       retraining from scratch").
 *
 * Conventions for every entry point
 *   - Sequence layout: F frames; each frame holds S special tokens then an
 *     R x C patch grid in row-major order; N = F*(S+R*C) tokens. Q, K, V and
 *     the output are bfloat16 arrays indexed [token][head][channel]: element
 *     (n, h, c) of q, k and v sits at n*tok_stride + h*head_stride + c, of
 *     the output at n*out_tok_stride + h*out_head_stride + c (zebra_layout;
 *     0 selects the contiguous [N][H][64] strides). The 64 channels of a
 *     (token, head) row are contiguous. Head dim d must be 64; 1 <= R, C <=
 *     128; H >= 1.
 *   - Tiles: tile u = f*tpf + a*ceil(C/8) + b (tpf = ceil(R/8)*ceil(C/8))
 *     covers patch rows [8a, min(8a+8,R)) and columns [8b, min(8b+8,C));
 *     n_u = its patch count; T = F*tpf tiles. Lower index wins score ties.
 *   - Kept tiles per query tile: k = round-half-even((1-y)*T), 0 <= y <= 1.
 *   - All pointers in zebra_args are DEVICE pointers owned by the caller,
 *     except where a field says "host". Buffer sizes come from
 *     zebra_buffer_bytes(). The library allocates no device memory, keeps
 *     no global state and is re-entrant across streams.
 *   - Every call validates its arguments on the host before any launch and
 *     then enqueues kernels on `stream` (asynchronous, no implicit sync).
 *     Errors: a non-zero zebra_status; zebra_last_error() returns a
 *     thread-local message. No C++ exception crosses this ABI.
 */
#ifndef ZEBRA_H
#define ZEBRA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ZEBRA_OK = 0,
  ZEBRA_ERR_INVALID_ARG = 1, /* null pointer, bad size, y outside [0,1] ... */
  ZEBRA_ERR_UNSUPPORTED = 2, /* head_dim != 64, grid larger than 128x128 */
  ZEBRA_ERR_WORKSPACE = 3,   /* workspace smaller than zebra_buffer_bytes */
  ZEBRA_ERR_HIP = 4          /* a HIP launch reported an error */
} zebra_status;

typedef struct {
  int32_t frames;    /* F >= 1 */
  int32_t specials;  /* S >= 0 special tokens per frame */
  int32_t rows;      /* R, patch grid rows, 1..128 */
  int32_t cols;      /* C, patch grid columns, 1..128 */
  int32_t heads;     /* H >= 1 */
  int32_t head_dim;  /* d, must be 64 */
  /* Element strides of q, k, v (and the affine teacher) and of out, for
   * callers whose Q/K/V are views of a fused projection output ("Linear-
   * centered stages plus tile-sparse stages": the QKV projections are kept,
   * so the operator reads their output in place). 0 selects the contiguous
   * value (tok: heads*64, head: 64). Otherwise each must be a positive
   * multiple of 8 elements (16 bytes) and at least 64; the pointers must be
   * 16-byte aligned. Rows of different (token, head) pairs may not overlap
   * in out, nor overlap q, k or v. */
  int64_t tok_stride;
  int64_t head_stride;
  int64_t out_tok_stride;
  int64_t out_head_stride;
} zebra_layout;

/* Opaque stream handle: a hipStream_t (NULL = the default stream). */
typedef void* zebra_stream;

typedef struct {
  zebra_layout L;
  double y;            /* sparsity of a tile-sparse stage, 0 <= y <= 1 */

  const void* q;       /* bf16 [N][H][64] */
  const void* k;       /* bf16 [N][H][64] */
  const void* v;       /* bf16 [N][H][64] */
  void* out;           /* bf16 [N][H][64], written by the attention calls */

  /* Linear stage parameters (float32, may be NULL):
   * W [H][64][64] acting on column vectors (NULL: identity), b [H][64]
   * (NULL: 0), mu [H][64] (NULL: 0), RMSNorm gains gq, gk [H][64]
   * (NULL: 1). The correction is y_i = mu + W (o_i - mu) + b. */
  const float* W;
  const float* b;
  const float* mu;
  const float* gq;
  const float* gk;
  float rms_eps;       /* RMSNorm epsilon; <= 0 selects 1e-6 */
  float rope_base;     /* rotary base; <= 0 selects 100 */

  /* Tile-sparse stage buffers (sizes: zebra_buffer_bytes). */
  void* kt;            /* packed keys, tile-major (ZEBRA_BUF_KT) */
  void* vt;            /* packed values, tile-major (ZEBRA_BUF_VT) */
  void* ks;            /* packed special-token keys (ZEBRA_BUF_KS) */
  void* vs;            /* packed special-token values (ZEBRA_BUF_VS) */
  double* kbar;        /* mean key of every tile, fp64 [H][T][64] */
  float* vbar;         /* mean value of every tile, fp32 [H][T][64] */
  float* logn;         /* ln n_u, fp32 [T] */
  void* lm;            /* landmarks repacked for attention (ZEBRA_BUF_LM) */
  int32_t* sel;        /* kept key tiles of every query tile, ascending,
                          int32 [H][T][k] */
  uint32_t* selmask;   /* the same as a bitmap, [H][T][ceil(T/32)] */
  double* gap;         /* optional (NULL ok): relative gap between the k-th
                          and (k+1)-th ranked tile score, fp64 [H][T]; from
                          the fp64 scores when the two round to the same
                          fp32 value, else from the fp32-rounded scores
                          (within 1.2e-7); +inf when k = 0 or k = T */

  void* workspace;     /* scratch (ZEBRA_BUF_WORKSPACE bytes) */
  size_t workspace_bytes;
} zebra_args;

/* Which buffer zebra_buffer_bytes sizes. */
enum {
  ZEBRA_BUF_KT = 0,
  ZEBRA_BUF_VT = 1,
  ZEBRA_BUF_KS = 2,
  ZEBRA_BUF_VS = 3,
  ZEBRA_BUF_KBAR = 4,
  ZEBRA_BUF_VBAR = 5,
  ZEBRA_BUF_LOGN = 6,
  ZEBRA_BUF_LM = 7,
  ZEBRA_BUF_SEL = 8,
  ZEBRA_BUF_SELMASK = 9,
  ZEBRA_BUF_GAP = 10,
  ZEBRA_BUF_WORKSPACE = 11,     /* enough for every entry point below but zebra_sparse_attn_bwd */
  ZEBRA_BUF_BWD_WORKSPACE = 12  /* enough for every entry point, zebra_sparse_attn_bwd included */
};

/* Operation codes for zebra_validate. */
enum {
  ZEBRA_OP_PACK = 0,
  ZEBRA_OP_LANDMARKS = 1,
  ZEBRA_OP_SELECT = 2,
  ZEBRA_OP_SPARSE = 3,
  ZEBRA_OP_LINEAR = 4,
  ZEBRA_OP_DENSE = 5,
  ZEBRA_OP_AFFINE_STATS = 6,
  ZEBRA_OP_COVERAGE = 7,
  ZEBRA_OP_PROLOGUE = 8,
  ZEBRA_OP_FRAME = 9,
  ZEBRA_OP_LINEAR_BWD = 10,
  ZEBRA_OP_SPARSE_BWD = 11
};

/* Pack K and V into tile-major order ("Speedup scales with the number of
 * input views": the sparse-stage kernels pack the key/value sequence into
 * tile-major order). Reads k, v; writes kt, vt (each tile's tokens
 * row-major, zero-padded to a multiple of 32 slots) and ks, vs (all special
 * tokens in frame order, zero-padded to a multiple of 32). When kbar is
 * non-NULL (then vbar, logn and lm must be too) the same pass also writes
 * every landmark exactly as zebra_landmarks would from kt and vt, so K and V
 * are read once; zebra_landmarks need not be called after it. */
zebra_status zebra_pack_tiles(const zebra_args* a, zebra_stream stream);

/* Mean key/value landmark of every tile ("Linear-centered stages plus
 * tile-sparse stages": omitted tiles are summarised as mean key/value
 * landmarks). Reads kt, vt; writes kbar (exact fp64 mean of the bf16 keys),
 * vbar, logn = ln n_u and lm (landmark keys and values rounded to bf16, in
 * the attention kernel's layout). */
zebra_status zebra_landmarks(const zebra_args* a, zebra_stream stream);

/* Tile selector ("Linear-centered stages plus tile-sparse stages": keep a
 * key-tile fraction 1 - y per query tile). For every head and query tile t:
 * qbar_t = mean of its patch queries (fp64), score s_{t,u} = qbar_t . kbar_u
 * / 8 in fp64 for every key tile u of every frame, keep the top k by
 * (score descending, tile index ascending). Reads q, kbar; writes sel
 * (ascending), selmask and gap (if non-NULL). Uses the workspace. */
zebra_status zebra_select_tiles(const zebra_args* a, zebra_stream stream);

/* Tile-sparse attention ("Linear-centered stages plus tile-sparse stages").
 * Patch row i of query tile t: softmax over (1/8 scaling) the real tokens
 * of every kept tile, the landmark of every omitted tile (logit
 * q.kbar_u/8 + ln n_u, value vbar_u), every special key, and its own key
 * when tile t itself is not kept. Special rows: dense over all N keys.
 * Reads q, kt, vt, ks, vs, lm, logn, selmask; writes out. The padding slots
 * of kt, vt, ks and vs must hold zeros, as zebra_pack_tiles writes them (a
 * padding key then contributes nothing). Products use bf16 operands with
 * fp32 accumulation; the queries are scaled by log2(e)/8 and rounded to bf16
 * before the key products. Uses the workspace:
 * per-row softmax offsets, one flag per query tile (rows whose cheap logit
 * bound is too loose are recomputed with an exact online softmax), the
 * staging plans of one round of work units, and fp32 partial outputs of the
 * special rows, whose keys are split into segments. Launches one kernel
 * pair per round of as many workgroups as the device holds at once. */
zebra_status zebra_sparse_attn(const zebra_args* a, zebra_stream stream);

/* Backward of zebra_sparse_attn ("A closed-form fit avoids retraining from
 * scratch": an optional training stage after the conversion fine-tunes the
 * converted model, so gradients flow back through its tile-sparse stages).
 * For out as zebra_sparse_attn computes it at a->y, writes the gradients of
 * sum(dout * out) with respect to q, k and v. The tile selection passes no
 * gradient: the kept tiles are the forward's (sel, selmask). A landmark is
 * the mean of its tile, so each token of an omitted tile receives 1/n_u of
 * the landmark's key and value gradients (ln n_u is a constant); the
 * landmarks enter at full precision (kbar fp64 and vbar fp32, each as bf16
 * high and low parts; log2 n_u from lm). Reads q, k, v, kbar, vbar, lm, sel,
 * selmask,
 * i.e. call it after zebra_pack_tiles (with landmarks) and
 * zebra_select_tiles on the same q, k, v and y, and nothing that overwrites
 * them in between. dout: bf16, device, with the output's token and head
 * strides; dq, dk, dv: bf16, device, with q's strides, overlapping none of
 * the inputs. All four 16-byte aligned. The workspace must hold
 * ZEBRA_BUF_BWD_WORKSPACE bytes (per-row log-sum-exp and D, the transposed
 * kept-tile bitmap, partial gradients of the special keys and landmarks,
 * the landmarks' bf16 high and low parts, checkpoint counters that the call
 * zeroes itself; two calls must not share a workspace at once).
 * At most 32,768 tiles, fewer than 2^31 tokens, and 8 patch rows of q/k/v
 * and of dout spanning fewer than 2^31 elements (ZEBRA_ERR_UNSUPPORTED).
 * fp32 arithmetic with bf16 MFMA operands: logits and dP exact products
 * summed in fp32, P and the logit gradients rounded to bf16 for the
 * gradient products; each gradient rounded once to bf16. */
zebra_status zebra_sparse_attn_bwd(const zebra_args* a, const void* dout, void* dq, void* dk, void* dv,
                                   zebra_stream stream);

/* Linear attention with the centred affine correction. For each head:
 * phi(x) = softmax over the 64 channels of RoPE2D(RMSNorm(x)) (channels
 * [0,32) turn by the patch row, [32,64) by the column, pair (j, j+16)
 * by p * base^(-j/16); specials at (0,0)); S = sum_j phi(k_j) v_j^T,
 * z = sum_j phi(k_j) over all N tokens (fp32); o_i = phi(q_i)^T S /
 * phi(q_i)^T z; out_i = mu + W (o_i - mu) + b. Reads q, k, v, W, b, mu,
 * gq, gk; writes out. Uses the workspace. */
zebra_status zebra_linear_attn(const zebra_args* a, zebra_stream stream);

/* Backward of zebra_linear_attn ("A closed-form fit avoids retraining from
 * scratch": an optional training stage after the conversion fine-tunes the
 * converted model, so gradients flow back through its linear stages). For
 * out as zebra_linear_attn computes it, writes the gradients of
 * sum(dout * out) with respect to q, k and v. W, gq, gk, rms_eps and
 * rope_base are constants of the backward; b and mu do not change it and
 * are not read. dout: bf16, device, with the output's token and head
 * strides (a->L.out_tok_stride, out_head_stride); dq, dk, dv: bf16, device,
 * with q's strides, overlapping none of q, k, v and dout. All four 16-byte
 * aligned. Reads q, k, v, W, gq, gk; uses the workspace (the forward's KV
 * state, the gradient of that state, their partial sums). fp32 arithmetic;
 * products with the KV state and its gradient run on MFMA with both
 * operands split into bf16 high and low parts; sums over tokens in fp32
 * within a workgroup and in fp64 across workgroups; each gradient is
 * rounded once to bf16 (nearest even). */
zebra_status zebra_linear_attn_bwd(const zebra_args* a, const void* dout, void* dq, void* dk, void* dv,
                                   zebra_stream stream);

/* zebra_linear_attn for callers that cannot allocate memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same kernels and the same result, but the scratch they need (partial
 * KV states, their sum and the folded state) lives in a static device array
 * of ZEBRA_NOALLOC_SCRATCH_BYTES that the library holds on every device it
 * runs on until the process ends; a->workspace is ignored. Reads q, k, v, W,
 * b, mu, gq, gk; writes out. The caller passes inputs and outputs only.
 * Calls no allocating routine (the first call on a device looks up the
 * array's address once). Layouts needing more scratch than the maximum
 * (about 1,300 views of 37x37 patches at 16 heads) are rejected with
 * ZEBRA_ERR_WORKSPACE before any launch. Every call on a device shares that
 * device's array: calls that overlap on one device (other streams, other
 * threads) race and must be serialised by the caller. */
#define ZEBRA_NOALLOC_SCRATCH_BYTES (64u << 20)
zebra_status zebra_linear_attn_noalloc(const zebra_args* a, zebra_stream stream);

/* Dense softmax attention of every token over all N keys ("Global attention
 * dominates runtime as views grow"): the measurement baseline. Reads q, k,
 * v; writes kt, vt, ks, vs, kbar, vbar, logn, lm (it packs and builds the
 * per-tile key bounds first) and out; uses the workspace. */
zebra_status zebra_dense_attn(const zebra_args* a, zebra_stream stream);

/* Query/key prologue of a tile-sparse (or frame-wise) stage ("Linear-
 * centered stages plus tile-sparse stages": conversion keeps the
 * normalisation layers and positional encoding): for every token and head,
 * x -> RoPE2D(RMSNorm(x)) exactly as the linear stage applies it (per-head
 * RMSNorm over the 64 channels with eps a->rms_eps and gains a->gq / a->gk,
 * then the pair (j, j+16) of channels [0,32) turned by the patch row and of
 * [32,64) by the column, angle p * base^(-j/16), base a->rope_base, special
 * tokens at (0,0)). Reads q and k; writes q_out and k_out (bf16, device,
 * with the token and head strides of q, k and v, so that they can stand in
 * for q and k in the next call; each may equal its input). */
zebra_status zebra_qk_prologue(const zebra_args* a, void* q_out, void* k_out, zebra_stream stream);

/* Frame-wise softmax attention ("Global attention dominates runtime as
 * views grow": the backbones alternate frame-wise attention with global
 * attention): every token of a frame, special or patch, attends with
 * logits q.k/8 to all tokens of its own frame and no other. Reads q, k, v;
 * packs K/V into kt, vt, ks, vs first (as zebra_pack_tiles, without
 * landmarks); writes out. At most 65,535 frames. */
zebra_status zebra_frame_attn(const zebra_args* a, zebra_stream stream);

/* Attention-mass coverage diagnostic of a tile-sparse stage ("Sensitive
 * stages also concentrate their attention": stages are profiled by how
 * concentrated their attention mass is, and sparse selection covers most
 * of it where softmax matters). For every head and patch query tile t,
 * averaged over the tile's rows i:
 *   coverage[h][t] = share of row i's DENSE softmax mass (all N keys,
 *                    logits q.k/8) that falls on the tokens of the key
 *                    tiles t kept;
 *   lm_error[h][t] = 1 - L_i/E_i, E_i the exact mass of the omitted tiles'
 *                    tokens and L_i the mass their landmarks give them
 *                    (n_u exp(q.kbar_u/8), kbar rounded to bf16 as the
 *                    sparse kernel uses it); 0 if no tile is omitted. In
 *                    [0, 1) by Jensen's inequality (up to rounding).
 * Reads q, kt, ks, lm (zebra_pack_tiles with the landmark buffers, or
 * zebra_landmarks) and selmask (zebra_select_tiles at the stage's y);
 * writes coverage and lm_error, device float32 [H][T]. Dense work: two
 * passes of Q.K^T over every key. */
zebra_status zebra_coverage(const zebra_args* a, float* coverage, float* lm_error, zebra_stream stream);

/* Statistics of the closed-form centred affine fit of a linear stage ("A
 * closed-form fit avoids retraining from scratch": teacher softmax outputs
 * and the converted linear outputs, accumulated over tokens and heads (and,
 * over calls, scenes), for a regularised least-squares solve in fp64).
 * o = a->out (the linear stage's output with no correction: W, b, mu NULL),
 * t = teacher (same layout as q: bf16 [N][H][64]); both pooled over all
 * N x H rows. Adds into stats, a device array of ZEBRA_AFFINE_STATS doubles
 * that the caller zeroes before the first call: n, sum o [64], sum t [64],
 * sum o o^T [64][64] (row-major), sum o t^T [64][64] (row a = o channel).
 * Products are exact, summed in fp32 over a workgroup's tokens and in fp64
 * across workgroups. Uses the workspace. */
#define ZEBRA_AFFINE_STATS (1 + 2 * 64 + 2 * 64 * 64)
zebra_status zebra_affine_stats(const zebra_args* a, const void* teacher, double* stats, zebra_stream stream);

/* Host-only fp64 solve from those statistics (host copy, ZEBRA_AFFINE_STATS
 * doubles): mu = mean o, b = mean t - mu, and W minimising
 * sum |(t - mean t) - W (o - mu)|^2 + lambda |W|^2 with
 * lambda = lambda_rel * trace(G) / 64, G the centred Gram of o:
 * W^T = (G + lambda I)^-1 C, C = sum (o - mu)(t - mean t)^T (Cholesky).
 * Writes W [64][64] (row = output channel), b [64], mu [64] as fp32, the
 * form zebra_linear_attn takes per head (one fit shared by all heads).
 * Errors: NULL pointers, lambda_rel < 0, n < 1, G + lambda I not positive
 * definite (ZEBRA_ERR_INVALID_ARG). */
zebra_status zebra_affine_solve(const double* stats, double lambda_rel, float* W, float* b, float* mu);

/* Host-only argument check of operation `op` (ZEBRA_OP_*); no GPU call. */
zebra_status zebra_validate(const zebra_args* a, int op);

/* Bytes needed for buffer `which` (ZEBRA_BUF_*) at layout L and sparsity y;
 * 0 for an invalid layout. */
size_t zebra_buffer_bytes(const zebra_layout* L, double y, int which);

/* k = round-half-even((1-y)*T) clamped to [0,T]; -1 if invalid. */
int64_t zebra_keep_count(const zebra_layout* L, double y);

/* Number of tiles T; -1 if the layout is invalid. */
int64_t zebra_num_tiles(const zebra_layout* L);

/* Message of the last error on this thread ("" if none). */
const char* zebra_last_error(void);

/* Library version string. */
const char* zebra_version(void);

#ifdef __cplusplus
}
#endif
#endif /* ZEBRA_H */
