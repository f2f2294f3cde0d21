/*
 * flux.h -- C ABI of the MI355X (gfx950) layer-routed hybrid attention library
 * (libflux.so).
 *
 * The method: Flux Attention adds a light Layer Router to a frozen LLM.  The
 * router pools the first and the last 100 prompt tokens, runs an MLP and
 * thresholds its output to a hard per-layer choice between Full Attention (FA)
 * and block-Sparse Attention (SA); the route is decided once at prefill and
 * reused by every decode step, and SA layers read only a minimal KV set.
 * (Flux Attention abstract, arXiv 2604.07394; technical summary on
 * gist.science, section 2 "Methodology".)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers marked [device] are HIP device pointers; [host] are host memory.
 *   The caller allocates and frees every buffer.  The library never
 *   allocates on these paths and keeps no mutable global state, except the
 *   device scratch array of flux_attn_decode_noalloc (one per GPU).
 * - bf16 tensors are passed as raw bf16 bit patterns (uint16_t).
 * - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *   Every call is asynchronous on `stream` and never synchronises it.
 * - All arguments are validated on the host before anything is launched; on
 *   failure a negative flux_status is returned and nothing is launched.  Data
 *   that lives on the device (lengths, routes, mask rows) cannot be checked on
 *   the host: kernels clamp routes, decode lengths and mask columns into
 *   range so that bad values give wrong numbers, never out-of-bounds
 *   accesses.  Offsets into other arrays are trusted and must be valid:
 *   prefill's cu_seqlens (they address the packed tensors) and a mask's
 *   row_ptr (it addresses col_idx).
 * - A launch failure reported by the HIP runtime returns FLUX_ERR_HIP.
 * - No C++ exception crosses this interface.
 */
#ifndef FLUX_H
#define FLUX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FLUX_OK = 0,
  FLUX_ERR_INVALID_ARG = -1,  /* null pointer, bad size or inconsistent shapes */
  FLUX_ERR_UNSUPPORTED = -2,  /* valid but not built (head_dim, block size ...) */
  FLUX_ERR_WORKSPACE = -3,    /* workspace missing or too small */
  FLUX_ERR_HIP = -4           /* the HIP runtime reported an error */
} flux_status;

typedef enum { FLUX_F32 = 0, FLUX_BF16 = 1 } flux_dtype;

/* Sparse Attention block pattern: block (i, j) of the mask is active iff
 * j <= i and (j < sink_blocks or j >= i - local_blocks + 1).
 * block_size in {64, 128}; sink_blocks >= 0; local_blocks >= 1 (counts the
 * diagonal block, so no row is ever empty). */
typedef struct {
  int32_t block_size;
  int32_t sink_blocks;
  int32_t local_blocks;
} flux_sa_params;

/* Text for a status code [host]. */
const char* flux_status_str(int32_t status);

/*
 * flux_route -- Layer Router: pooling, MLP and hard threshold.
 * (technical summary, section 2: the router pools the first and last 100
 * prompt tokens, an MLP context encoder maps them to a per-layer decision,
 * and inference thresholds the soft weight to 0/1.)
 *
 * For each request r with S = cu_seqlens[r+1] - cu_seqlens[r] rows:
 *   pooled = mean of hidden rows {0..min(100,S)-1} U {max(0,S-100)..S-1}
 *            (a set: rows in both ends count once), accumulated in fp32;
 *   z      = W2 * relu(W1 * pooled + b1) + b2       (fp32);
 *   route[r][l] = 1 (FA) if z[l] >= 0 else 0 (SA)   (sigmoid(z) >= 0.5).
 *
 * hidden      [device] [T][d_in] rows of all requests packed back to back,
 *             fp32 or bf16 per hidden_dtype (a flux_dtype value).
 * cu_seqlens  [device] int32 [n_req+1], prefix offsets into the rows; each
 *             request needs S >= 1 (S <= 0 yields pooled = 0).
 * w1, b1      [device] fp32 [h1][d_in], [h1]     (PyTorch Linear layout)
 * w2, b2      [device] fp32 [n_layers][h1], [n_layers]
 * route_out   [device] uint8 [n_req][n_layers]
 * logits_out  [device] fp32 [n_req][n_layers] or NULL
 * workspace   [device] >= flux_route_workspace_size(n_req, d_in, h1) bytes,
 *             any contents (holds the pooled vectors and hidden layers).
 * Limits: 1 <= n_req <= 65535, 1 <= d_in, h1, n_layers <= 65536.
 */
size_t flux_route_workspace_size(int32_t n_req, int32_t d_in, int32_t h1);
flux_status flux_route(const void* hidden, int32_t hidden_dtype,
                       const int32_t* cu_seqlens, int32_t n_req, int32_t d_in,
                       const float* w1, const float* b1, int32_t h1,
                       const float* w2, const float* b2, int32_t n_layers,
                       uint8_t* route_out, float* logits_out,
                       void* workspace, size_t workspace_bytes, void* stream);

/* Number of mask blocks for a sequence: ceil(seqlen / block_size) [host].
 * Returns a negative flux_status on invalid input. */
int64_t flux_mask_blocks(int32_t seqlen, flux_sa_params p);

/* Active blocks of the mask for `seqlen` tokens, in closed form [host]:
 * sum over rows i < nb of min(i+1, w) + max(0, min(s, i-w+1)).
 * Returns a negative flux_status on invalid input. */
int64_t flux_mask_nnz(int32_t seqlen, flux_sa_params p);

/*
 * flux_build_block_mask -- the SA block mask (integer, exact).
 * SA layers run block-sparse attention (Block-Sparse-Attention library, named
 * on the Flux Attention Qwen3-4B model card, "Sample Usage") and keep only a
 * minimal KV set (technical summary, section 2); the block pattern is the
 * sink + causal local window defined at flux_sa_params.
 *
 * With nb = flux_mask_blocks(seqlen, p) and nnz = flux_mask_nnz(seqlen, p):
 * mask_out [device] uint8 [nb][nb] dense mask, or NULL to skip it;
 * row_ptr  [device] int32 [nb+1];  col_idx [device] int32 [nnz], columns
 *          strictly increasing within a row (what the attention kernels read).
 * One mask built for the longest sequence serves every shorter one: entry
 * (i, j) does not depend on the length.  1 <= seqlen, nb <= 65536.
 */
flux_status flux_build_block_mask(int32_t seqlen, flux_sa_params p, uint8_t* mask_out,
                                  int32_t* row_ptr, int32_t* col_idx, void* stream);

/*
 * flux_build_block_mask_dynamic -- a content-aware SA block mask for one
 * sequence.  The pages only hint at a content-based pattern (the model
 * card's address slug); the "Daily Papers" page (hugingapi.com, search
 * "Head-Centric Sparse Attention") describes block importance from
 * coarse-grained attention between mean-pooled blocks (Prism abstract) and an
 * adaptive Top-tau block selection (RRAttention abstract).  The definition
 * built here:
 *   qbar[i][h], kbar[j][g]  means of the rows of block i of q / block j of k
 *                           (a shorter last block averages its own rows);
 *   P[i][j]  mean over the query heads h of the softmax over j <= i of
 *            softmax_scale * qbar[i][h] . kbar[j][h / (hq / hkv)];
 *   row i keeps its sink blocks (j < sink_blocks) and its diagonal block,
 *   then the other blocks j <= i by decreasing P (ties: smaller j first)
 *   while the mass taken is below tau and the row holds fewer than
 *   max_blocks blocks (max_blocks 0: no cap).
 * The output is the CSR form that flux_attn_prefill and flux_attn_decode read
 * as their SA mask (nb = ceil(seqlen / block_size) rows, columns increasing).
 * The selection is decided in fp32: a block whose cumulative mass lands within
 * rounding of tau may be kept by one implementation and not by another.
 *
 * q [device] bf16 [seqlen][hq][head_dim];  k [device] bf16 [seqlen][hkv][head_dim]
 * row_ptr  [device] int32 [nb+1], written;
 * col_idx  [device] int32 [col_capacity], col_capacity >= nb (nb + 1) / 2;
 *          the first row_ptr[nb] entries are written
 * workspace [device], 16-byte aligned, >= flux_dynamic_mask_workspace_size(...)
 *          bytes; owned by the caller, overwritten.
 * Supported: head_dim in {64, 128}, block_size in {64, 128}, hq % hkv == 0,
 *   hq / hkv <= 16, nb <= 1024.  tau >= 0 (tau >= 1 keeps every
 *   causal block unless capped), sink_blocks >= 0, max_blocks >= 0, scale > 0.
 */
typedef struct {
  int32_t block_size;   /* B: 64 or 128 */
  int32_t sink_blocks;  /* always-kept leading blocks */
  float tau;            /* probability mass a row must reach */
  int32_t max_blocks;   /* cap on blocks per row; 0 = none */
} flux_dyn_params;

size_t flux_dynamic_mask_workspace_size(int32_t seqlen, int32_t hq, int32_t hkv, int32_t head_dim,
                                        int32_t block_size);
flux_status flux_build_block_mask_dynamic(const uint16_t* q, const uint16_t* k, int32_t seqlen,
                                          int32_t hq, int32_t hkv, int32_t head_dim,
                                          float softmax_scale, flux_dyn_params p, int32_t* row_ptr,
                                          int32_t* col_idx, int64_t col_capacity, void* workspace,
                                          size_t workspace_bytes, void* stream);

/*
 * flux_attn_prefill -- one attention layer over a packed batch of prompts.
 * FA: causal softmax attention; SA: the same restricted to the active blocks
 * of the mask (abstract: each layer runs FA or SA; model card: SA is
 * block-sparse attention).  For request r, query head h reads KV head
 * h / (hq / hkv); key t is visible to query p iff t <= p and
 * (route[r][layer] == 1 or block (p / B, t / B) is in the mask).
 * Requests never attend to each other.  bf16 in/out, fp32 accumulation.
 *
 * q, out      [device] bf16 [T][hq][head_dim];  k, v [device] bf16 [T][hkv][head_dim]
 * cu_seqlens  [device] int32 [n_req+1], non-decreasing, cu_seqlens[n_req] = T
 *             (the kernels trust the offsets: they address q/k/v/out with
 *             them; a length above max_seqlen is cut to max_seqlen rows)
 * max_seqlen  [host] >= every request length
 * softmax_scale  > 0 (usually 1/sqrt(head_dim))
 * route       [device] uint8 [n_req][n_layers], read at [r][layer]; nonzero = FA
 * mask_row_ptr, mask_col_idx  [device] CSR of flux_build_block_mask for
 *             mask_blocks >= ceil(max_seqlen / block_size) rows; columns must
 *             be increasing within a row (columns past a row's diagonal are
 *             clamped to it).  Every workgroup reads its row's bounds; only SA
 *             layers read the columns.
 * workspace   [device] NULL, or FLUX_PREFILL_WORKSPACE_BYTES (16-byte
 *             aligned, owned by the caller) that are all zero before the call;
 *             the call leaves them all zero again when it completes (a
 *             one-workgroup kernel that follows the attention kernel on the
 *             stream clears them).  When ceil(max_seqlen / block_size) x hq
 *             x n_req is at least 768 and a multiple of 8, the last part of
 *             every XCD's share of the work is then handed out at run time,
 *             so XCDs that run faster than the others take over some of their
 *             work (other calls keep the fixed order).  Results are bitwise
 *             those without a workspace: only which workgroup computes a
 *             query block changes.  Calls that run at the same time need
 *             different workspaces.  A size below
 *             FLUX_PREFILL_WORKSPACE_BYTES or a misaligned pointer is
 *             FLUX_ERR_WORKSPACE.
 * Supported: head_dim in {64, 128}, block_size in {64, 128}, hq % hkv == 0,
 *            hq / hkv <= 16.  out may not alias q, k or v.
 */
#define FLUX_PREFILL_WORKSPACE_BYTES ((size_t)1024)

/* FLUX_PREFILL_WORKSPACE_BYTES [host]. */
size_t flux_attn_prefill_workspace_size(void);

flux_status flux_attn_prefill(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                              uint16_t* out, const int32_t* cu_seqlens, int32_t n_req,
                              int32_t max_seqlen, int32_t hq, int32_t hkv, int32_t head_dim,
                              float softmax_scale, const uint8_t* route, int32_t n_layers,
                              int32_t layer, const int32_t* mask_row_ptr,
                              const int32_t* mask_col_idx, int32_t mask_blocks,
                              flux_sa_params p, void* workspace, size_t workspace_bytes,
                              void* stream);

/*
 * flux_attn_prefill_heads -- flux_attn_prefill with one route decision per
 * (request, layer, kv head): route is uint8 [n_req][n_layers][hkv] and query
 * head h follows route[r][layer][h / (hq / hkv)].  Head-level routing is the
 * granularity the pages argue against on GPUs (load imbalance and
 * synchronisation long tails between heads; technical summary, sections 1
 * and 2); it is provided to measure that claim.  Everything else as
 * flux_attn_prefill, without the workspace (a fixed order that deals every
 * kv group to every XCD).
 */
flux_status flux_attn_prefill_heads(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                    uint16_t* out, const int32_t* cu_seqlens, int32_t n_req,
                                    int32_t max_seqlen, int32_t hq, int32_t hkv, int32_t head_dim,
                                    float softmax_scale, const uint8_t* route, int32_t n_layers,
                                    int32_t layer, const int32_t* mask_row_ptr,
                                    const int32_t* mask_col_idx, int32_t mask_blocks,
                                    flux_sa_params p, void* stream);

/*
 * flux_attn_prefill_soft -- the soft-routed forward of one layer:
 *   out = r * FA(q, k, v) + (1 - r) * SA(q, k, v),  r = r_soft[req][layer],
 * the convex combination of the two branches that the router's continuous
 * weight forms during training (technical summary, section 2, differentiable
 * soft routing).  One pass with one softmax state: the tiles of the mask's
 * blocks come first, then (1 - r) times their normalised result is parked
 * in `out` (rounded to bf16 once), the same state runs on over FA's other
 * causal tiles (the SA blocks are a subset of FA's), and r times the FA
 * result plus the parked part is written.  Forward only.
 * r_soft [device] fp32 [n_req][n_layers] (the caller's weights, e.g. a
 * Gumbel-softmax sample or sigmoid(z); any value is combined as given).
 * Everything else, the workspace included, as flux_attn_prefill (no route:
 * both branches are formed; the pass balances like an FA layer).
 */
flux_status flux_attn_prefill_soft(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                   uint16_t* out, const int32_t* cu_seqlens, int32_t n_req,
                                   int32_t max_seqlen, int32_t hq, int32_t hkv, int32_t head_dim,
                                   float softmax_scale, const float* r_soft, int32_t n_layers,
                                   int32_t layer, const int32_t* mask_row_ptr,
                                   const int32_t* mask_col_idx, int32_t mask_blocks,
                                   flux_sa_params p, void* workspace, size_t workspace_bytes,
                                   void* stream);

/* Workspace bytes flux_attn_decode needs for these sizes [host] (0 on invalid
 * input). */
size_t flux_attn_decode_workspace_size(int32_t n_seq, int32_t hq, int32_t hkv,
                                       int32_t head_dim, int32_t max_len);

/*
 * flux_attn_decode -- one decode step of one layer, split-KV over a work
 * list: every (sequence, kv head) visits U keys (FA: its N keys; SA: its
 * mask row's blocks), and the keys of all of them are cut into work items
 * of about the same size (about as many items as the GPU holds decode
 * workgroups at once, at most 1024, at least 256 keys each; a call with more
 * than 1024 (sequence, kv head) pairs takes one item per pair), so a long FA
 * sequence beside short SA sequences is split
 * finer than they are.  The plan is made on the device from the lengths and
 * routes of the call; the partial results of a pair's items are merged by
 * the log-sum-exp rule.
 * The route fixed at prefill is reused for every decode step; SA layers read
 * only the keys of their mask row and never the rest of the history
 * (technical summary, section 2, deployment paragraph).
 *
 * Sequence b holds N = seqlens[b] keys in its cache, the newest token (the
 * query's own) included, so the query is position N-1: FA reads keys
 * 0..N-1; SA reads the keys of mask row (N-1) / block_size.
 *
 * q, out      [device] bf16 [n_seq][hq][head_dim]
 * k_cache, v_cache [device] bf16 [n_seq][hkv][max_len][head_dim]
 * seqlens     [device] int32 [n_seq], each in [1, max_len] (clamped on device)
 * route       [device] uint8 [n_seq][n_layers], read at [b][layer]; 1 = FA
 * mask_*      as for flux_attn_prefill, mask_blocks >= ceil(max_len / block_size)
 * workspace   [device] 16-byte aligned, >= flux_attn_decode_workspace_size(...)
 *             bytes, any contents (nothing needs to start at zero); it holds
 *             the items' fp32 partials and the work plan between two kernels.
 *             When that size is 0 (every pair can only have one item: more
 *             than 1024 pairs, or too few keys to split) it may be NULL.
 * Supported: head_dim in {64, 128}, block_size in {64, 128}, hq % hkv == 0,
 *            hq / hkv <= 16.
 */
flux_status flux_attn_decode(const uint16_t* q, const uint16_t* k_cache,
                             const uint16_t* v_cache, uint16_t* out, const int32_t* seqlens,
                             int32_t n_seq, int32_t max_len, int32_t hq, int32_t hkv,
                             int32_t head_dim, float softmax_scale, const uint8_t* route,
                             int32_t n_layers, int32_t layer, const int32_t* mask_row_ptr,
                             const int32_t* mask_col_idx, int32_t mask_blocks,
                             flux_sa_params p, void* workspace, size_t workspace_bytes,
                             void* stream);

/*
 * flux_attn_decode_append -- one decode step of one layer with the new
 * token's K/V row appended in the same launch: the result and the caches
 * afterwards are those of flux_kv_append(k_new, v_new, seqlens, ..., compact
 * = 0) followed by flux_attn_decode (per (sequence, kv head), the one wave
 * that reads key seqlens[b] - 1 first stores the new row at that position
 * and waits for the store; sequences with seqlens[b] outside [1, max_len]
 * get no row, as in flux_kv_append).  Full caches only.
 * k_new, v_new  [device] bf16 [n_seq][hkv][head_dim], must not alias the
 *               caches or out; k_cache, v_cache [device] as for
 *               flux_attn_decode, written at one row per (sequence, kv head).
 * Everything else, including the workspace, as flux_attn_decode.
 */
flux_status flux_attn_decode_append(const uint16_t* q, const uint16_t* k_new,
                                    const uint16_t* v_new, uint16_t* k_cache, uint16_t* v_cache,
                                    uint16_t* out, const int32_t* seqlens, int32_t n_seq,
                                    int32_t max_len, int32_t hq, int32_t hkv, int32_t head_dim,
                                    float softmax_scale, const uint8_t* route, int32_t n_layers,
                                    int32_t layer, const int32_t* mask_row_ptr,
                                    const int32_t* mask_col_idx, int32_t mask_blocks,
                                    flux_sa_params p, void* workspace, size_t workspace_bytes,
                                    void* stream);

/*
 * flux_attn_decode_noalloc -- flux_attn_decode without a workspace argument,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation).  The
 * split partials and the work plan live in a device array of the library
 * (FLUX_DECODE_SCRATCH_BYTES, one copy per GPU, kept until the process ends;
 * its address is looked up once per device).  Nothing is allocated and
 * nothing needs to start at zero.  Calls on one GPU share that array: calls
 * that may overlap in time on one GPU (different streams, or host threads)
 * race and give wrong results; calls ordered on one stream are safe.
 * The array holds FLUX_DECODE_SCRATCH_BYTES (9 MiB); the largest workspace
 * any call that flux_attn_decode accepts can need is 8.2 MiB (1024 work
 * items x 16 query heads per kv head x head_dim 128), and a call needing
 * more than the array would return FLUX_ERR_WORKSPACE.  Everything else,
 * including the results (bit for bit), as flux_attn_decode.
 */
#define FLUX_DECODE_SCRATCH_BYTES ((size_t)9 << 20)
flux_status flux_attn_decode_noalloc(const uint16_t* q, const uint16_t* k_cache,
                                     const uint16_t* v_cache, uint16_t* out,
                                     const int32_t* seqlens, int32_t n_seq, int32_t max_len,
                                     int32_t hq, int32_t hkv, int32_t head_dim,
                                     float softmax_scale, const uint8_t* route, int32_t n_layers,
                                     int32_t layer, const int32_t* mask_row_ptr,
                                     const int32_t* mask_col_idx, int32_t mask_blocks,
                                     flux_sa_params p, void* stream);

/* flux_attn_decode_heads -- flux_attn_decode with route uint8
 * [n_seq][n_layers][hkv], one decision per kv head (see flux_attn_prefill_heads). */
flux_status flux_attn_decode_heads(const uint16_t* q, const uint16_t* k_cache,
                                   const uint16_t* v_cache, uint16_t* out, const int32_t* seqlens,
                                   int32_t n_seq, int32_t max_len, int32_t hq, int32_t hkv,
                                   int32_t head_dim, float softmax_scale, const uint8_t* route,
                                   int32_t n_layers, int32_t layer, const int32_t* mask_row_ptr,
                                   const int32_t* mask_col_idx, int32_t mask_blocks,
                                   flux_sa_params p, void* workspace, size_t workspace_bytes,
                                   void* stream);

/*
 * K/V caches for decode, and the compact SA-layer cache.
 * The route is decided once at prefill and reused by every decode step, and
 * SA layers read only their sink and window keys, never the rest of the
 * history (technical summary, section 2, deployment paragraph).  A cache is
 * [n_seq][hkv][rows][head_dim] bf16 with rows = flux_kv_rows(max_len, p,
 * compact):
 *   full    (compact = 0): rows = max_len, position t at row t;
 *   compact (compact = 1): rows = (sink_blocks + local_blocks) * block_size;
 *           positions t < sink_blocks*B at row t, every later position t at
 *           row sink_blocks*B + t mod (local_blocks*B) (a ring of the last
 *           local_blocks blocks).  This holds every key an SA decode step
 *           reads with the mask of flux_build_block_mask for the same p, and
 *           nothing else: at 32K context with 1 sink and 16 local blocks of
 *           128, 2176 rows instead of 32768.
 * Positions at or beyond max_len are never written (the writers skip them).
 */

/* Rows per (sequence, kv head) of a cache [host]; negative flux_status on
 * invalid input (compact must be 0 or 1; p is only used when compact). */
int64_t flux_kv_rows(int32_t max_len, flux_sa_params p, int32_t compact);

/*
 * flux_kv_store_prefill -- the prompts' K/V rows into decode caches.
 * k, v       [device] bf16 [T][hkv][head_dim], packed by cu_seqlens (the same
 *            tensors flux_attn_prefill reads); cu_seqlens [device] int32
 *            [n_req+1]; request r becomes sequence r of the caches.
 * k_cache, v_cache [device] bf16 [n_req][hkv][rows][head_dim]; full caches get
 *            every prompt position, compact caches the sink positions and the
 *            last local_blocks*B positions of each prompt.
 * Requires max_seqlen <= max_len; head_dim in {64, 128}; compact caches need
 * block_size in {64, 128}.  Rows not written keep their contents.
 */
flux_status flux_kv_store_prefill(const uint16_t* k, const uint16_t* v,
                                  const int32_t* cu_seqlens, int32_t n_req,
                                  int32_t max_seqlen, int32_t hkv, int32_t head_dim,
                                  uint16_t* k_cache, uint16_t* v_cache, int32_t max_len,
                                  int32_t compact, flux_sa_params p, void* stream);

/*
 * flux_kv_append -- one new K/V row per sequence (a decode step's token).
 * k_new, v_new [device] bf16 [n_seq][hkv][head_dim]; the row is written at
 * position seqlens[b] - 1, i.e. seqlens already counts the new token (the
 * convention of flux_attn_decode).  Sequences with seqlens[b] < 1 or
 * seqlens[b] > max_len are left alone.
 */
flux_status flux_kv_append(const uint16_t* k_new, const uint16_t* v_new, const int32_t* seqlens,
                           int32_t n_seq, int32_t hkv, int32_t head_dim, uint16_t* k_cache,
                           uint16_t* v_cache, int32_t max_len, int32_t compact,
                           flux_sa_params p, void* stream);

/*
 * flux_attn_decode_sa_compact -- flux_attn_decode for an SA layer whose caches
 * are compact.  Every sequence is treated as SA (a compact cache cannot serve
 * FA, so there is no route argument); keys are those of mask row
 * (seqlens[b] - 1) / block_size, read from their compact rows.  max_len is the
 * logical capacity (seqlens are clamped to it, the mask needs ceil(max_len /
 * block_size) rows and the workspace is flux_attn_decode_workspace_size(...,
 * max_len), as for flux_attn_decode); the result is bit-identical to
 * flux_attn_decode on full caches with the same keys.  The CSR must be the
 * flux_build_block_mask pattern of the same p.
 */
flux_status flux_attn_decode_sa_compact(const uint16_t* q, const uint16_t* k_cache,
                                        const uint16_t* v_cache, uint16_t* out,
                                        const int32_t* seqlens, int32_t n_seq, int32_t max_len,
                                        int32_t hq, int32_t hkv, int32_t head_dim,
                                        float softmax_scale, const int32_t* mask_row_ptr,
                                        const int32_t* mask_col_idx, int32_t mask_blocks,
                                        flux_sa_params p, void* workspace, size_t workspace_bytes,
                                        void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FLUX_H */
