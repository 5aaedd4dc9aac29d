/*
 * csa2.h - C ABI of the CSA2 (Compressed Sparse Attention 2) decode / chunked-prefill
 * library for AMD Instinct MI355X (gfx950).
 *
 * What is computed (sources are the pages this library follows):
 *   "Detailed Notes On DeepSeek V4 Point 1 Flash In Simple Words" - sections
 *     "Compressed Sparse Attention 2 Or CSA2 In Simple Terms" (per-layer indexer scores
 *     the past entries, the top 512 are attended), "The Three Modes Full Reindex And
 *     Reuse", "Hierarchical Sparse Indexer In Simple Terms", "FP4 Main KV Cache To Halve
 *     Storage Again" (E2M1 main KV, dequantised before attention), "Model Setup Numbers
 *     Without Jargon" (32 indexer heads, Top-512, 64 attention heads of dim 512).
 *   "DeepSeek-V4.1-Flash 技术解读" (mengman.github.io) - 3.3 CSA2 (mode table; Reindex and
 *     Reuse borrow from the most recent Full / indexing layer), 3.4 Hierarchical Sparse
 *     Indexer, 3.5 FP4 Main KV Cache.
 *
 * Conventions shared by every call:
 *   - Every pointer argument is a DEVICE pointer unless marked "host".  All calls are
 *     asynchronous on `stream` (a hipStream_t; NULL = the null stream).
 *   - The caller owns every buffer.  No call allocates, frees or retains device memory
 *     (csa2_layer_group_noalloc uses a scratch array the library itself holds).
 *     Calls that take `ws` need a device workspace of at least the size the matching
 *     *_workspace_size() function reports; it needs no initialisation and its contents
 *     are undefined afterwards.  Calls that share one `ws` must be ordered on a stream.
 *   - Tensors are dense, row-major, innermost dimension contiguous.
 *   - Return value: CSA2_OK (0) or a negative csa2_status.  Arguments are validated on
 *     the host before anything is launched; on an error nothing is launched and no
 *     output is written.  Faults inside a kernel surface at the caller's next
 *     synchronisation; a launch failure returns CSA2_ERR_DEVICE.
 *   - The library runs on gfx950 only; other devices give CSA2_ERR_UNSUPPORTED.
 *
 * Number formats (bit-exact; see the quantise calls):
 *   E2M1: 4 bits = sign | 2 exponent bits (bias 1) | 1 mantissa bit; magnitudes
 *         0, 0.5, 1, 1.5, 2, 3, 4, 6.  Two codes per byte, even channel in the low nibble.
 *   E4M3: OCP "FN" 8-bit float (bias 7, max 448, no infinities, 0x7F/0xFF are NaN).
 *   Quantisation of x with scale s: code = nearest(fl32(x / s)), ties to the even code,
 *   saturating to the largest finite magnitude, sign kept (also for -0); s == 0 gives +0.
 */
#ifndef CSA2_H
#define CSA2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CSA2_OK = 0,
  CSA2_ERR_NULL = -1,        /* a required pointer is NULL */
  CSA2_ERR_SHAPE = -2,       /* a size is out of range or inconsistent */
  CSA2_ERR_DTYPE = -3,       /* unsupported dtype / format / precision enum value */
  CSA2_ERR_MODE = -4,        /* invalid layer-mode schedule */
  CSA2_ERR_WORKSPACE = -5,   /* workspace NULL or smaller than required */
  CSA2_ERR_UNSUPPORTED = -6, /* device is not gfx950, or a shape this build does not handle */
  CSA2_ERR_DEVICE = -7       /* a HIP runtime call or kernel launch failed */
} csa2_status;

typedef enum { CSA2_F32 = 0, CSA2_BF16 = 1 } csa2_dtype;
typedef enum {
  CSA2_FMT_FP4_PER_CHANNEL = 0,
  CSA2_FMT_FP8_PER_TOKEN = 1,
  CSA2_FMT_FP4_G16 = 2,
  CSA2_FMT_FP4_PER_TOKEN = 3
} csa2_fmt;
typedef enum { CSA2_SCALE_COMPUTE = 0, CSA2_SCALE_GIVEN = 1 } csa2_scale_policy;
typedef enum { CSA2_PREC_FP32 = 0, CSA2_PREC_FP8 = 1, CSA2_PREC_FP4 = 2 } csa2_index_prec;
typedef enum { CSA2_FULL = 0, CSA2_REINDEX = 1, CSA2_REUSE = 2 } csa2_mode;

/* Limits of this build. */
#define CSA2_MAX_K 2048      /* Top-K */
#define CSA2_MAX_D 512       /* main-KV dim */
#define CSA2_MAX_HQ 128      /* attention heads */
#define CSA2_MAX_DK 256      /* indexer dim (fp32 indexer); the fp8 indexer needs dk == 64 */
#define CSA2_MAX_H 64        /* indexer heads (fp32 indexer); the fp8 indexer needs H == 32 */
#define CSA2_MAX_WINDOW 128  /* sliding-window entries per query */
#define CSA2_MAX_GROUP_T 16  /* query tokens per sequence in a layer group */

/* Human-readable name of a csa2_status (static string). */
const char* csa2_status_string(int status);

/* CSA2_OK when the current HIP device is gfx950, else CSA2_ERR_UNSUPPORTED / _DEVICE. */
int csa2_device_check(void);

/*
 * Write side: quantise rows and store them in a cache.
 * Source: "FP4 Main KV Cache To Halve Storage Again" (main KV in E2M1 with scales,
 * quantised after RoPE) and 3.5 of the Chinese reading; the indexer stays low-bit.
 *
 *   x[b][t][c] at x + b*x_stride_b + t*x_stride_t + c (elements of x_dtype), b < B, t < T,
 *   c < D.  Row t of sequence b is written to cache row n0[b] + t (n0 NULL = 0); the
 *   caller guarantees 0 <= n0[b] and n0[b] + T <= n_max (rows outside [0, n_max) are
 *   skipped, never written).
 *
 *   CSA2_FMT_FP4_PER_CHANNEL: codes [B][n_max][D/2] (E2M1 pairs), scales [B][D] fp32, one
 *     scale per (sequence, channel).  CSA2_SCALE_COMPUTE: scales[b][c] =
 *     fl32(max_t |x[b][t][c]| / 6) over the T rows given, written to `scales`.
 *     CSA2_SCALE_GIVEN: `scales` is read (append to an existing cache; values beyond
 *     +-6 s saturate).  D even, 2 <= D.
 *   CSA2_FMT_FP8_PER_TOKEN: codes [B][n_max][D] (E4M3), scales [B][n_max] fp32, one scale
 *     per row: s = fl32(max_c |x| / 448) (scale_policy must be COMPUTE).  D <= 4096.
 *   CSA2_FMT_FP4_G16 (the pages' layout: one E4M3 scale per 16 channels of each entry, no
 *     global scale; "FP4 Main KV Cache To Halve Storage Again"): codes [B][n_max][D/2] as
 *     above, scales [B][n_max][D/16] uint8 (E4M3 bytes).  Per group of 16 channels of a row:
 *     sc = E4M3(fl32(max |x| / 6)) (nearest, ties to even, saturating at 448), code =
 *     E2M1(fl32(x / value(sc))) (values beyond 6 after the division saturate; sc = 0 gives
 *     code +0).  Every entry's scales come from the entry itself, so scale_policy is
 *     ignored.  D % 16 == 0.  288 B per entry at D = 512.
 *   CSA2_FMT_FP4_PER_TOKEN (4-bit indexer keys; the pages' indexer q/k are 4-bit, "FP4 Main
 *     KV Cache To Halve Storage Again"): codes [B][n_max][D/2] (E2M1 pairs, lower dim in the
 *     low nibble), scales [B][n_max] fp32: s = fl32(max_c |x| / 6), code = E2M1(fl32(x / s))
 *     (scale_policy must be COMPUTE).  D even, D <= 4096.
 */
int csa2_quantize_kv(int fmt, int scale_policy, int B, int T, int D, const void* x, int x_dtype,
                     int64_t x_stride_b, int64_t x_stride_t, const int32_t* n0, int64_t n_max, uint8_t* codes,
                     void* scales, void* stream);

/*
 * Gather + dequantise selected FP4 rows (the step before attention: the stored FP4 entries
 * are turned back into real values before attention, "FP4 Main KV Cache To Halve Storage
 * Again").
 *   kv_fmt CSA2_FMT_FP4_PER_CHANNEL: out[b][t][k][c] = fl32(E2M1(code) * scales[b][c]),
 *     scales fp32 [B][D];
 *   kv_fmt CSA2_FMT_FP4_G16: out = E2M1(code) * E4M3(scales[b][j][c / 16]) (exact), scales
 *     uint8 [B][n_max][D/16], D % 16 == 0;
 *   of cache row j = idx[b][t][k]; rows with idx outside [0, n_max) (e.g. the -1 padding)
 *   give 0.  out is fp32 [B][T][K][D].  Bit-exact.
 */
int csa2_gather_dequant(int kv_fmt, int B, int T, int K, int D, const uint8_t* codes, const void* scales,
                        int64_t n_max, const int32_t* idx, float* out, void* stream);

/*
 * Indexer scores (Full / Reindex layers).  Source: "Compressed Sparse Attention 2 Or CSA2
 * In Simple Terms" (a per-layer indexer with 32 query heads scores the past entries).
 * Score of query row (b,t) against cache row j:
 *   CSA2_PREC_FP32: score = sum_h w[b][t][h] * (q[b][t][h] . k[b][j])        (q, k fp32)
 *   CSA2_PREC_FP8 : the query is quantised per (b,t,h) to E4M3 with sq = max|q_h|/448,
 *                   score = k_scale[b][j] * sum_h w_h * sq_h * (q8_h . k8[b][j])
 *                   (k: E4M3 codes, k_scale fp32 per row; contraction on fp8 MFMA;
 *                   requires H == 32, dk == 64).
 *   CSA2_PREC_FP4 : the same with E2M1 on both sides: the query quantised per (b,t,h) with
 *                   sq = max|q_h|/6, k the packed E2M1 codes [B][n_max][dk/2] of
 *                   CSA2_FMT_FP4_PER_TOKEN with k_scale; contraction on the FP4 form of the
 *                   same MFMA; H == 32, dk == 64.  Not with csa2_hier_select.
 *   q: [B][T][H][dk] of q_dtype; w: [B][T][H] fp32; k: [B][n_max][dk]; k_scale:
 *   [B][n_max] (FP8) or NULL (FP32).
 * Visible columns: cand == NULL -> column j is cache row j (ncols = n_max); cand != NULL
 *   -> column c is cache row cand[b][t][c] (ncols = C; negative = invisible).  A row is
 *   visible iff it is < n_keys[b] and (q_limit == NULL or <= q_limit[b][t]) (causal limit
 *   of chunked prefill).  scores: [B][T][ncols] fp32, -inf where not visible.
 *   ws: csa2_index_score_workspace_size() bytes (currently 0; may be NULL).
 */
int csa2_index_score(int prec, int B, int T, int H, int dk, const void* q, int q_dtype, const float* w,
                     const void* k, const float* k_scale, int64_t n_max, const int32_t* n_keys,
                     const int32_t* q_limit, const int32_t* cand, int C, float* scores, void* ws, size_t ws_bytes,
                     void* stream);
size_t csa2_index_score_workspace_size(int B, int T, int64_t ncols);

/*
 * Top-K per query row.  Source: "Compressed Sparse Attention 2 Or CSA2 In Simple Terms"
 * (the indexer picks the top 512 entries).  Order: higher score first, ties to the lower
 * position.  A column is visible iff its score is > -inf (NaN is not) and, with `cand`,
 * its position cand[b][t][c] is >= 0.  Output idx_out [B][T][K] int32: the selected
 * positions (column index, or cand value) in ASCENDING order, padded with -1 when fewer
 * than K columns are visible; val_out [B][T][K] fp32 (nullable): their scores, -inf for
 * padding.  Positions must be distinct within a row.  1 <= K <= CSA2_MAX_K.
 * ws: csa2_topk_workspace_size() bytes.
 */
int csa2_topk(int B, int T, int64_t ncols, const float* scores, const int32_t* cand, int K, int32_t* idx_out,
              float* val_out, void* ws, size_t ws_bytes, void* stream);
size_t csa2_topk_workspace_size(int B, int T, int64_t ncols, int K);

/*
 * Fused score + Top-K (csa2_index_score then csa2_topk without returning the scores).
 * Same arguments and results as the two calls; scores are kept in `ws`.
 * ws: csa2_index_topk_workspace_size() bytes.
 */
int csa2_index_topk(int prec, int B, int T, int H, int dk, const void* q, int q_dtype, const float* w,
                    const void* k, const float* k_scale, int64_t n_max, const int32_t* n_keys,
                    const int32_t* q_limit, const int32_t* cand, int C, int K, int32_t* idx_out, float* val_out,
                    void* ws, size_t ws_bytes, void* stream);
size_t csa2_index_topk_workspace_size(int B, int T, int64_t ncols, int K);

/*
 * A layer's own sliding-window cache ("CSA2 In Simple Terms": every layer also attends to
 * the most recent tokens; window 128 in "Model Setup Numbers"; the window cache stays
 * 8-bit in "FP4 Main KV Cache To Halve Storage Again"; each layer keeps its own, 3.3 of
 * the Chinese reading).  codes [B][n_max][D] E4M3 with one fp32 scale per row, scales
 * [B][n_max] (the layout csa2_quantize_kv writes with CSA2_FMT_FP8_PER_TOKEN).  Query row
 * (b, t) attends to window rows [max(0, e - window), e), e = min(end[b][t], n_max), in the
 * same softmax as its selected entries (a ring buffer that holds exactly the window may
 * pass end = its fill count: the order of rows does not matter).  1 <= window <=
 * CSA2_MAX_WINDOW.
 */
typedef struct {
  const uint8_t* codes;
  const float* scales;
  int64_t n_max;
  const int32_t* end;    /* [B][T] */
  int window;
} csa2_swa;

/*
 * Sparse softmax attention over the selected FP4 entries.  Sources: "Compressed Sparse
 * Attention 2 Or CSA2 In Simple Terms" (attend to the selected entries), "FP4 Main KV
 * Cache To Halve Storage Again" (dequantise before attention), "Model Setup Numbers"
 * (64 heads of dim 512).  The whole dequantised entry v_j is both key and value:
 *   l_hj = softmax_scale * q_h . v_j over j in idx[b][t][*] (entries outside [0, n_max)
 *   skipped);  out_h = sum_j softmax(l_h)_j v_j;  lse_h = log sum_j exp(l_hj).
 *   No selected entry: out = 0, lse = -inf.
 *   q: [B][T][Hq][D] of q_dtype; kv_codes [B][n_max][D/2]; kv_scales as for
 *   csa2_gather_dequant of kv_fmt (fp32 [B][D] per channel, or uint8 [B][n_max][D/16] E4M3
 *   per 16 channels of each entry); idx [B][T][K]; out [B][T][Hq][D] of out_dtype; lse
 *   [B][T][Hq] fp32 (nullable).
 *   q_dtype CSA2_F32: fp32 arithmetic throughout (out_dtype must be CSA2_F32).
 *   q_dtype CSA2_BF16: fp16 MFMA with fp32 accumulation; needs Hq % 16 == 0 and D in
 *   {128, 256, 512}.  Per-channel scales are folded into the query (with an exact
 *   power-of-two prescale) and into the output; per-16-channel scales multiply the fp16
 *   key/value operands (E2M1 * E4M3 is exact in fp16).  Entries are processed in groups of
 *   512 whose partial softmax results are merged by log-sum-exp.
 *   swa (nullable): the layer's sliding-window entries, joining the same softmax (attended
 *   inside the selected entries' blocks when the grid is small, as at decode; otherwise
 *   the window's partial result is merged with the selected entries' by log-sum-exp).
 *   ws: csa2_sparse_attend_workspace_size() bytes (0 when K <= 512 without a window, or q
 *   is fp32; then ws may be NULL); `window` there is swa->window, or 0 without a window.
 *   The size covers a window's own partial slot whether or not the call needs it.
 */
int csa2_sparse_attend(int B, int T, int Hq, int D, const void* q, int q_dtype, int kv_fmt, const uint8_t* kv_codes,
                       const void* kv_scales, int64_t n_max, const int32_t* idx, int K, const csa2_swa* swa,
                       float softmax_scale, void* out, int out_dtype, float* lse, void* ws, size_t ws_bytes,
                       void* stream);
size_t csa2_sparse_attend_workspace_size(int B, int T, int Hq, int D, int K, int q_dtype, int window);

/*
 * Layer group: Full / Reindex / Reuse layers over one shared cache, run strictly in order.
 * Sources: "The Three Modes Full Reindex And Reuse" and 3.3 of the Chinese reading:
 *   FULL    - scores the shared indexer keys with its own query, takes a fresh Top-K.
 *             (Building the cache - csa2_quantize_kv - is the caller's write side.)
 *   REINDEX - borrows main KV and indexer keys of the most recent Full layer (here: the
 *             one shared cache), its own query and weights, a fresh Top-K.
 *   REUSE   - borrows main KV and the most recent indexing layer's Top-K unchanged.
 *   Every layer attends with its own attention query.
 * Schedule rule: layer 0 is FULL; REINDEX needs an earlier FULL; REUSE needs an earlier
 * FULL or REINDEX; otherwise CSA2_ERR_MODE.  Per-layer pointers (T = the group cache's
 * query tokens per sequence, 1 for plain decode): q_idx [B][T][H][dk] (q_dtype), w
 * [B][T][H], q_attn [B][T][Hq][D] (q_dtype), out [B][T][Hq][D] (out_dtype), lse [B][T][Hq]
 * (nullable), idx [B][T][K] written by FULL/REINDEX, ignored by REUSE (may be NULL there),
 * swa (nullable): the layer's own sliding-window cache (never shared; its window must not
 * exceed csa2_group_cache.window; its end is per query row).
 * With a candidate pool (csa2_group_cache.pool_blocks > 0), a REINDEX layer after a FULL
 * layer scores only the pool that the most recent FULL layer left; pool [B][T][pool_blocks
 * * pool_block] (nullable, FULL only) receives that pool's positions: selected blocks
 * ascending, positions ascending inside a block, -1 at or past the row's visible end
 * (n_keys, less T - 1 - t for row t) and for blocks missing when fewer than pool_blocks
 * blocks hold a visible position.
 */
typedef struct {
  int mode;              /* csa2_mode */
  const void* q_idx;     /* FULL/REINDEX */
  const float* w;        /* FULL/REINDEX */
  const void* q_attn;
  void* out;
  float* lse;
  int32_t* idx;          /* FULL/REINDEX: output; REUSE: ignored */
  int32_t* pool;         /* FULL with a pool: optional output; otherwise ignored */
  const csa2_swa* swa;   /* nullable */
} csa2_layer;

typedef struct {
  int B, H, dk, Hq, D, K;
  int64_t n_max;
  const int32_t* n_keys;   /* [B] */
  const uint8_t* kv_codes; /* [B][n_max][D/2] */
  const void* kv_scales;   /* fp32 [B][D], or uint8 [B][n_max][D/16] with kv_fmt CSA2_FMT_FP4_G16 */
  const void* k;           /* [B][n_max][dk] E4M3 codes (FP8) or fp32 (FP32) */
  const float* k_scale;    /* [B][n_max] (FP8) or NULL */
  int prec;                /* csa2_index_prec */
  int q_dtype, out_dtype;  /* csa2_dtype */
  float softmax_scale;
  /* Candidate pool ("Hierarchical Sparse Indexer In Simple Terms"): with pool_blocks > 0,
   * every Full layer also reduces its scores over blocks of pool_block consecutive positions
   * to the block maximum, keeps the pool_blocks best blocks (lowest block index on ties) and
   * the Reindex layers after it score only those blocks' positions.  0 = no pool (every
   * Reindex layer scores all n_keys entries).  1 <= pool_blocks <= CSA2_MAX_K. */
  int pool_block;
  int pool_blocks;
  int kv_fmt;              /* CSA2_FMT_FP4_PER_CHANNEL (0) or CSA2_FMT_FP4_G16 */
  int window;              /* largest sliding window of the layers (0: no layer has one) */
  /* Query tokens per sequence, 0 or 1 = plain decode.  T > 1 (draft verification: DSpark
   * proposes several tokens at once, "Detailed Notes", DSpark section): the T tokens' own
   * entries are the cache's last T, token t sees positions < n_keys[b] - (T - 1 - t), and
   * every per-layer tensor has T rows per sequence ([B][T][...]).  T <= CSA2_MAX_GROUP_T. */
  int T;
} csa2_group_cache;

int csa2_layer_group(const csa2_layer* layers, int n_layers, const csa2_group_cache* cache, void* ws,
                     size_t ws_bytes, void* stream);
size_t csa2_layer_group_workspace_size(const csa2_group_cache* cache, int n_layers);

/*
 * Layer group that allocates nothing, for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments (less the workspace), validation and results as csa2_layer_group; the
 * workspace is a device array of CSA2_NOALLOC_SCRATCH_BYTES inside the library, one per
 * GPU the library runs on, held until the process ends (its address is looked up on the
 * first call on each device).  No hipMalloc, hipFree or allocating library call is made.
 * Errors: those of csa2_layer_group; CSA2_ERR_WORKSPACE when
 * csa2_layer_group_workspace_size(cache, n_layers) exceeds CSA2_NOALLOC_SCRATCH_BYTES
 * (nothing is launched).  All calls on one GPU share that GPU's array, which keeps the
 * last call's contents (the call clears what must start at zero itself): calls that
 * overlap on one GPU (other streams, other threads) race on it and must be ordered.
 */
#define CSA2_NOALLOC_SCRATCH_BYTES (64u << 20)
int csa2_layer_group_noalloc(const csa2_layer* layers, int n_layers, const csa2_group_cache* cache, void* stream);

/*
 * Two-level indexer, coarse keys: the mean of each `block` consecutive dequantised E4M3
 * indexer keys, re-quantised to E4M3 with its own max/448 scale.  The mean is defined in
 * fp32: fl32((sum over the block's rows, in row order, of fl32(k_scale_j * E4M3(k8_jc))) /
 * count), each partial sum rounded to fp32, so the bytes are reproducible.  Blocks cover
 * [0, n_keys[b]); the last one may be partial; blocks past it are 0 with scale 0.
 * kb8 [B][nb_max][dk], kb_scale [B][nb_max], nb_max = ceil(n_max / block).  Bit-exact.
 * Source of the idea: "Hierarchical Sparse Indexer In Simple Terms" (rank blocks of
 * positions first, then score inside the kept blocks); this block-mean key is the form
 * used by the long-context configuration (the pages rank blocks by their max score).
 */
int csa2_coarse_keys(int B, int64_t n_max, const int32_t* n_keys, int dk, int block, const uint8_t* k8,
                     const float* k_scale, uint8_t* kb8, float* kb_scale, void* stream);

/*
 * Two-level Top-K over the coarse keys (decode, fp8 indexer): score the coarse keys, keep
 * the best `block_topk` blocks (ties to the lower block), score every position inside
 * them and keep the best K (ties to the lower position).  idx_out [B][1][K] ascending,
 * -1 padded; block_out [B][1][block_topk] (nullable) the kept blocks ascending.
 * ws: csa2_hier_select_workspace_size() bytes.  Each stage's scan lists its candidates for
 * the selection (four launches) when its rows span at most 128 score blocks; larger stages
 * (e.g. more than 32768 block keys for a single sequence) take the histogram selection
 * (seven launches).  Both give the same result.
 */
int csa2_hier_select(int B, int H, int dk, const void* q, int q_dtype, const float* w, const uint8_t* k8,
                     const float* k_scale, const uint8_t* kb8, const float* kb_scale, int64_t n_max,
                     const int32_t* n_keys, int block, int block_topk, int K, int32_t* idx_out, int32_t* block_out,
                     void* ws, size_t ws_bytes, void* stream);
size_t csa2_hier_select_workspace_size(int B, int64_t n_max, int block, int block_topk, int K);

/*
 * Measurement utility (not a step of the method): reads `bytes` of device memory at `src`
 * once with 16-byte nontemporal loads, `blocks` workgroups of 256 threads sweeping it, and
 * computes nothing the caller sees (sink [1] uint32 is written only in an impossible case).
 * Timing it gives the read bandwidth a streaming kernel reaches on this GPU, the ceiling
 * the indexer's key scan is compared with.  bytes a multiple of 16, src 16-byte aligned.
 */
int csa2_stream_probe(const void* src, int64_t bytes, int blocks, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* CSA2_H */
