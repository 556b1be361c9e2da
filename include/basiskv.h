/*
 * basiskv.h -- C ABI of libbasiskv.so: the BasisKV decode-time hot path on
 * AMD Instinct MI355X (gfx950).
 *
 * Method: "BasisKV: Value Latents for Communication and Key Routing"
 * (arXiv 2611.02583).  Per token and per physical KV head the cache holds a
 * Value latent z (width r_v), a Key residual code r (width r_q) and the exact
 * Key k (width head_dim) -- appendix Table 4.  A decode step
 *   (a0) compresses the new token's Key and Value into those three states,
 *   (a1) projects the queries onto the routing factors,
 *   (a2) scores every Key page from the latent's leading r_b dims plus the
 *        residual (the abstract's latent-based Key routing),
 *   (a3) keeps the top_k pages per KV head,
 *   (a4) computes exact softmax attention with the original Keys of the kept
 *        pages only and sums the cached latents with those weights, and
 *   (a5) maps the per-head latents to the model output through the fused
 *        latent-to-output matrix M = blockdiag(B) W_O (Figure 1: the output is
 *        rebuilt from the latents).
 *
 * Single-source routers: with dims.r_q = 0 there is no residual: no residual
 * pool (cache.r_pages may be NULL), and Q and E are not read (may be NULL);
 * with dims.r_b = 0 nothing is predicted from the latent and P is not read
 * (may be NULL): the residual code is the Key through E.
 *
 * Conventions shared by every entry point
 *   - Plain C, no exceptions; every call returns a basiskv_status.  Host-side
 *     validation runs before any launch: on a non-OK status nothing has been
 *     enqueued and outputs are untouched.
 *   - All memory is caller-owned and device-resident unless stated; the
 *     library never allocates, frees or synchronises.  Calls are asynchronous
 *     on `stream` (a hipStream_t; NULL = the default stream).  Calls on one
 *     stream are ordered; concurrent calls that share a workspace race.
 *   - `dims.dtype` is the storage format of queries, caches, factors, K/V
 *     inputs, M and y: BASISKV_F32 (float32) or BASISKV_BF16 (bfloat16); or
 *     BASISKV_BF16_FP8_E4M3: everything bf16 except the three cache pools,
 *     which hold FP8 E4M3 codes (appendix Table 13: BasisKV under an FP8
 *     E4M3 KV cache).  The codes are OCP E4M3FN (sign, 4 exponent bits with
 *     bias 7, 3 mantissa bits; largest finite magnitude 448; subnormal step
 *     2^-9; 0x7F and 0xFF are NaN; no infinities) with no scale factor.
 *     Arithmetic is float32 throughout (float32 accumulation; bf16 and E4M3
 *     values are widened exactly; stores round to nearest-even, and stores to
 *     E4M3 saturate at +-448).
 *   - Query head h uses KV head h / (n_q_heads / n_kv_heads).
 *   - Device-side indices are range-checked by the kernels: a block_table
 *     entry outside [0, num_phys_pages), a selected page outside the
 *     sequence, or a position outside [0, max_pages_per_seq * page_size) is
 *     skipped (treated as absent), never dereferenced.  seq_lens are clamped
 *     to [0, max_pages_per_seq * page_size].
 *
 * Paged cache layout (one pool per state, head-major):
 *   pool[n_kv_heads][num_phys_pages][width / CE][page_size][CE]
 * where CE = 16 / sizeof(element) (16 for E4M3, 8 for bf16, 4 for float32) and width is
 * r_v (z pool), r_q (r pool) or head_dim (k pool).  Token t of a page keeps its
 * 16-byte chunk c at ((c * page_size) + t) * 16 bytes from the page start, so
 * one wavefront with a token per lane reads page_size * 16 contiguous bytes per
 * chunk.  Logical page p of sequence b is physical page block_table[b][p].
 * Widths must be multiples of CE.
 *
 * Routing-first layout (dims.page_layout = BASISKV_LAYOUT_ROUTING_FIRST): the
 * latent and residual share one pool, cache.z_pages, whose pages hold
 * (r_v + r_q) / CE chunks in the order: the latent's first r_b / CE chunks, the
 * r_q / CE residual chunks, the latent's remaining chunks; cache.r_pages is
 * not used.  Routing then reads one contiguous run of (r_b + r_q) / CE chunks
 * per page (appendix Table 4's routing widths), where the separate pools give
 * two; with small pages and narrow E4M3 rows a separate run fills half of a
 * 128-byte memory line.  Pages are whole 128-byte lines: with 4-token pages an
 * odd chunk count is rounded up to the next even one (the last chunk of each
 * page is unused), so the pool is [n_kv][num_phys][C][page_size][CE] with
 * C = (r_v + r_q) / CE, plus one when page_size is 4 and that is odd.  Every
 * call of one cache must use the same layout.
 */
#ifndef BASISKV_H
#define BASISKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  BASISKV_OK = 0,
  BASISKV_ERR_NULL = 1,        /* a required pointer is NULL */
  BASISKV_ERR_SHAPE = 2,       /* sizes inconsistent or out of range */
  BASISKV_ERR_UNSUPPORTED = 3, /* valid, but outside what this library implements */
  BASISKV_ERR_WORKSPACE = 4,   /* workspace NULL or smaller than required */
  BASISKV_ERR_LAUNCH = 5       /* the HIP runtime rejected a kernel launch */
} basiskv_status;

enum { BASISKV_F32 = 0, BASISKV_BF16 = 1, BASISKV_BF16_FP8_E4M3 = 2 };
enum { BASISKV_LAYOUT_SEPARATE = 0, BASISKV_LAYOUT_ROUTING_FIRST = 1 };

/* Sizes of one layer's decode problem (host values). */
typedef struct {
  int32_t batch;             /* sequences, >= 1 */
  int32_t n_q_heads;         /* query heads, multiple of n_kv_heads */
  int32_t n_kv_heads;        /* physical KV heads */
  int32_t head_dim;          /* must be 128 */
  int32_t hidden;            /* output width D of W_O (multiple of 16) */
  int32_t r_v;               /* Value-latent width */
  int32_t r_b;               /* routing base width: leading latent dims, 0 <= r_b <= r_v */
  int32_t r_q;               /* Key-residual rank, >= 0.  r_b and r_q may not both be 0;
                                r_q = 0 routes from the latent alone, r_b = 0 from the
                                residual alone (appendix Table 9's single-source routers
                                B16, R16, R32, beside the combined B16R16) */
  int32_t page_size;         /* tokens per page: 4, 8, 16, 32 or 64 */
  int32_t max_pages_per_seq; /* columns of block_table, <= 32768 */
  int32_t num_phys_pages;    /* pages per pool and per KV head */
  int32_t dtype;             /* BASISKV_F32, BASISKV_BF16 or BASISKV_BF16_FP8_E4M3 */
  int32_t recent_tokens;     /* >= 0: recent window (appendix Table 9 caption: 64 recent
                                tokens beside the routed budget).  With W > 0 the pages
                                holding a sequence's last W valid tokens, from page
                                max(0, seq_len - W) / page_size on, are attended whatever
                                their score, and the top_k routed pages are chosen among the
                                pages before them; sel still holds the routed pages only.
                                0: no window. */
  int32_t page_layout;       /* BASISKV_LAYOUT_SEPARATE (three pools) or
                                BASISKV_LAYOUT_ROUTING_FIRST (see above) */
} basiskv_dims;

/* The paged cache (device pointers, caller-owned). */
typedef struct {
  void *z_pages;              /* Value latents  [n_kv][num_phys][r_v/CE][page_size][CE]
                                 (routing-first: [n_kv][num_phys][(r_v+r_q)/CE][page_size][CE]) */
  void *r_pages;              /* residual codes [n_kv][num_phys][r_q/CE][page_size][CE]
                                 (routing-first: unused, may be NULL) */
  void *k_pages;              /* exact Keys     [n_kv][num_phys][head_dim/CE][page_size][CE] */
  const int32_t *block_table; /* [batch][max_pages_per_seq] logical -> physical page */
  const int32_t *seq_lens;    /* [batch] valid tokens of each sequence */
  const float *rope_inv_freq; /* NULL: no positions.  Else rotary position embedding
                                 (the pages' Figure 6 predicts the pre-RoPE Key): float32
                                 [head_dim / 2] inverse frequencies w_i (w_i = base^(-2i /
                                 head_dim) for the standard embedding); every cached state
                                 is pre-RoPE, the queries are already rotated to their own
                                 position, and the predicted Key (routing) and the exact
                                 Key (attention) of the token at position t -- its index
                                 in the sequence -- are rotated to t before the dot
                                 product: rotate-half pairs (i, i + head_dim / 2) by the
                                 angle t * w_i (taken exactly).  Routing then forms each
                                 token's predicted Key on the matrix cores instead of
                                 using projected queries, so basiskv_score_pages (which
                                 takes projected queries) returns ERR_UNSUPPORTED; use
                                 basiskv_score_pages_rope, basiskv_route_pages or
                                 basiskv_decode_step.  Supported
                                 for bf16 activations (bf16 or E4M3 pages), groups of 4
                                 and 8 heads, routing widths (r_b, r_q) of (16, 16),
                                 (64, 32), (96, 48), latent widths 64 and 96 (ERR_UNSUPPORTED
                                 otherwise); not used by basiskv_dense_attend. */
} basiskv_cache;

/* Human-readable name of a status code (static storage). */
const char *basiskv_status_string(int32_t status);

/* Bytes of workspace that basiskv_route_pages, basiskv_sparse_attend and
 * basiskv_decode_step need for these dims and top_k; one buffer of this size
 * serves all three.  0 if dims are invalid.
 * The workspace is device memory owned by the caller.  It must be zero-filled
 * after allocation, and again before it serves calls of other dims: it holds
 * small integer counters with which the workgroups of the attention launch
 * elect the one that merges a (sequence, KV head) row's splits (every call
 * leaves them at zero again), and for basiskv_decode_step the epoch of its
 * last step and the marks with which that step's projection workgroups
 * told the scanning ones their queries were ready (both carried from call to
 * call; a step recognises only marks of its own epoch).  Calls that share one
 * workspace must not run concurrently. */
size_t basiskv_workspace_bytes(const basiskv_dims *dims, int32_t top_k);

/* (a0) Compress new tokens into the cache -- BasisKV abstract (Value kept
 * only as a low-rank latent; a Key-specific residual keeps what the latent
 * cannot predict) and appendix Table 4 (the three cached states).
 *   k, v      [batch][n_tokens][n_kv_heads][head_dim]  new Keys and Values
 *   start_pos [batch] (device int32): token i of sequence b is written at
 *             position start_pos[b] + i
 *   A [n_kv][head_dim][r_v]   Value encoder:   z = v A            -> z pool
 *   P [n_kv][r_b][head_dim]   latent -> Key predictor
 *   E [n_kv][head_dim][r_q]   residual encoder: r = (k - z_s[:r_b] P) E -> r pool
 *   the Key itself is stored in the k pool (copied; rounded to E4M3 with
 *   BASISKV_BF16_FP8_E4M3).  z_s is the latent as stored (rounded to the cache
 *   format).  GEMMs run on MFMA with float32 accumulation.
 * seq_lens are not read or changed.  Returns ERR_SHAPE for n_tokens < 1.
 * No workspace: each token's latent and residual are finished by one
 * wavefront (the factors are staged in LDS once per workgroup), so nothing
 * crosses workgroups.  Needs r_v and r_q multiples of 16 (MFMA output tiles). */
int32_t basiskv_compress_prefill(const basiskv_dims *dims, const void *k, const void *v,
                                 const int32_t *start_pos, int32_t n_tokens, const void *A,
                                 const void *P, const void *E, const basiskv_cache *cache,
                                 void *stream);

/* (a1) Routing projections of the queries (appendix Table 4: routing reads
 * r_b latent dims and r_q residual dims, so the query is carried into those
 * two spaces once per step).
 *   q [batch][n_q_heads][head_dim];  P [n_kv][r_b][head_dim];  Q [n_kv][r_q][head_dim]
 *   q_proj [batch][n_q_heads][r_b + r_q] float32 out:
 *          q_proj[b][h][:r_b] = P_g q_bh,  q_proj[b][h][r_b:] = Q_g q_bh. */
int32_t basiskv_project_queries(const basiskv_dims *dims, const void *q, const void *P,
                                const void *Q, float *q_proj, void *stream);

/* (a2) Page scores from the cached latents and residual codes (BasisKV
 * abstract: the latent predicts the routing part of the Key, the residual the
 * rest; Table 9 caption: routing is per page).  For every valid token t of
 * page p and head h of KV head g's group:
 *   logit = q_proj[b][h][:r_b] . z_t[:r_b] + q_proj[b][h][r_b:] . r_t,
 * page_scores[b][g][p] = max over the page's valid tokens and the group's
 * heads; pages at or past ceil(seq_len / page_size) get -inf.
 *   page_scores [batch][n_kv_heads][max_pages_per_seq] float32 out. */
int32_t basiskv_score_pages(const basiskv_dims *dims, const float *q_proj,
                            const basiskv_cache *cache, float *page_scores, void *stream);

/* (a2) Page scores with rotary positions (cache->rope_inv_freq set; the
 * pages' Figure 6 predicts the pre-RoPE Key): for every valid token t of
 * page p, its predicted Key k_t = z_t[:r_b] P_g + r_t Q_g is rotated to
 * position t, and
 *   logit = q_bh . RoPE_t(k_t),
 * page_scores[b][g][p] = max over the page's valid tokens and the group's
 * heads; pages at or past ceil(seq_len / page_size) get -inf.
 *   q [batch][n_q_heads][head_dim] (already rotated to its own position);
 *   P [n_kv][r_b][head_dim];  Q [n_kv][r_q][head_dim];
 *   page_scores [batch][n_kv_heads][max_pages_per_seq] float32 out.
 * ERR_NULL without a frequency table; ERR_UNSUPPORTED outside the supported
 * set listed at basiskv_cache.  No workspace. */
int32_t basiskv_score_pages_rope(const basiskv_dims *dims, const void *q, const void *P,
                                 const void *Q, const basiskv_cache *cache, float *page_scores,
                                 void *stream);

/* (a3) Top-k page selection per (sequence, KV head) (BasisKV abstract: only
 * the selected pages' Keys are fetched).  Exact: the top_k largest scores
 * among the sequence's ceil(seq_len / page_size) pages; equal scores go to
 * the lower page index; the list is in ascending page order and padded with
 * -1 when top_k exceeds the page count (all -1 for an empty sequence).  With
 * dims.recent_tokens = W > 0 the candidates are the pages before the recent
 * window, i.e. the first max(0, seq_len - W) / page_size pages.
 *   seq_lens [batch] device; sel [batch][n_kv_heads][top_k] int32 out. */
int32_t basiskv_select_pages(const basiskv_dims *dims, const float *page_scores,
                             const int32_t *seq_lens, int32_t top_k, int32_t *sel,
                             void *stream);

/* (a1)+(a2)+(a3) in one call: projection, scoring and selection launches;
 * q_proj lives in the workspace. */
int32_t basiskv_route_pages(const basiskv_dims *dims, const void *q, const void *P,
                            const void *Q, const basiskv_cache *cache, int32_t top_k,
                            float *page_scores, int32_t *sel, void *workspace,
                            size_t workspace_bytes, void *stream);

/* (a4) Exact attention over the selected pages, summed in latent space
 * (BasisKV abstract: exact QK scores with the original Keys of the selected
 * pages; Figure 1 and appendix Table 4: the weighted sum runs over the
 * cached Value latents, all r_v dims).  For each query head h of KV head g:
 *   s_t = scale * q_h . k_t over the valid tokens of the pages in sel[b][g],
 *   p = softmax(s) over those tokens, u[b][h] = sum_t p_t z_t.
 * Entries of sel that are -1 or outside the sequence are skipped; a head with
 * no valid token gets u = 0.  scale is usually 1/sqrt(head_dim).  With
 * dims.recent_tokens > 0 the recent window's pages are attended too; sel must
 * then hold pages before the window only (as basiskv_select_pages gives).
 *   q [batch][n_q_heads][head_dim]; sel [batch][n_kv_heads][top_k];
 *   u [batch][n_q_heads][r_v] float32 out.
 * The workspace (see basiskv_workspace_bytes) holds the per-split partial
 * results and the counters that elect the workgroup merging them. */
int32_t basiskv_sparse_attend(const basiskv_dims *dims, const void *q,
                              const basiskv_cache *cache, const int32_t *sel, int32_t top_k,
                              float scale, float *u, void *workspace, size_t workspace_bytes,
                              void *stream);

/* (a5) Output reconstruction y = u M.  Figure 1 of the BasisKV pages: after
 * the partitions exchange their latents, each one rebuilds the complete
 * output from them; the abstract: Value compression is tied to the output
 * projection, so the Value decoder is folded into it,
 *   M = blockdiag_h(Bf_{h/G}) W_O,   the plain fused matrix [n_q_heads * r_v][hidden]
 * (row k = h * r_v + i: latent dim i of query head h; column n: output feature).
 * MFMA GEMM with float32 accumulation; for bf16, u is split into two bf16
 * terms (hi + lo) so no precision is lost before the product.
 *   u [batch][n_q_heads * r_v] float32;
 *   M: the fused matrix in the library's MFMA-tiled layout, written once, at
 *      set-up, by basiskv_pack_output_matrix (from a caller's plain matrix)
 *      or basiskv_fuse_output_matrix (from Bf and W_O);
 *   y [batch][hidden] out, in dtype (bf16 for BASISKV_BF16_FP8_E4M3).
 * Needs hidden % 16 == 0 and K = n_q_heads * r_v a multiple of 32 (bf16
 * activations) or 16 (float32), ERR_UNSUPPORTED otherwise.  Any batch.
 * No workspace: every output column's sum over K is finished inside one
 * workgroup (its wavefronts' partial tiles are added in LDS). */
int32_t basiskv_reconstruct(const basiskv_dims *dims, const float *u, const void *M, void *y,
                            void *stream);

/* Set-up for (a5): the caller's plain fused matrix M_plain
 * [n_q_heads * r_v][hidden] (dtype: float32, or bf16 for BASISKV_BF16 and
 * BASISKV_BF16_FP8_E4M3; row k = h * r_v + i, column n = output feature, as
 * documented at basiskv_reconstruct) copied into the tiled layout that
 * basiskv_reconstruct and basiskv_decode_step read (see
 * basiskv_fuse_output_matrix for the layout).  Pure data movement: the tiled
 * matrix holds the same values bit for bit.  M_plain and M are device
 * buffers of n_q_heads * r_v * hidden elements that must not overlap
 * (ERR_SHAPE when they are the same pointer).  Same size requirements as
 * basiskv_reconstruct. */
int32_t basiskv_pack_output_matrix(const basiskv_dims *dims, const void *M_plain, void *M,
                                   void *stream);

/* A whole decode step of one layer in one call, with the same results as
 *   basiskv_compress_prefill(k_new, v_new, start_pos, n_tokens = 1),
 *   basiskv_route_pages, basiskv_sparse_attend, basiskv_reconstruct
 * in that order, bit for bit.  Five launches, stream-ordered, no host
 * synchronisation: the query projection; the scoring; the selection;
 * attention; reconstruction.  Where the scan is long (routing reads of 160 MiB
 * or more over the pool's capacity, batch * n_kv_heads * max_pages_per_seq *
 * page_size tokens) the scoring launch's first workgroups compress the new
 * tokens and score them while the rest scan the other tokens, and the
 * selection first folds each new token's score into its page's (page_scores
 * then holds the full scores); otherwise, and with rotary positions, the
 * compression shares the projection's launch.  Where the scoring launch can
 * take the projection in too (bf16 pages, groups of a multiple of 4 query
 * heads), it does so with such a long scan, and also with a shorter one
 * of 64 MiB or more over bf16 pages at least 32 routing dims wide, which then
 * takes the compression in as well (four launches): the projection's
 * workgroups come first in the grid, mark each block of projected rows done
 * with the step's epoch, and the scanning workgroups wait for those marks
 * before reading the projected queries.  The epoch is a word in the
 * workspace that the selection launch advances, so the call may be captured
 * in a graph and replayed.
 *   k_new, v_new [batch][n_kv_heads][head_dim]: the step's new token of every
 *     sequence, written at position start_pos[b] (device int32 [batch]);
 *     seq_lens must already count it.
 *   q, P, Q, A, E, M, top_k, scale, page_scores, sel, u, y: as in the calls
 *     above.  Needs r_v, r_q <= 128.
 *   workspace: see basiskv_workspace_bytes. */
int32_t basiskv_decode_step(const basiskv_dims *dims, const void *q, const void *k_new,
                            const void *v_new, const int32_t *start_pos, const void *A,
                            const void *P, const void *Q, const void *E, const void *M,
                            const basiskv_cache *cache, int32_t top_k, float scale,
                            float *page_scores, int32_t *sel, float *u, void *y,
                            void *workspace, size_t workspace_bytes, void *stream);

/* Size of the library's own scratch, the device memory that
 * basiskv_decode_step_static uses in place of a workspace. */
#define BASISKV_STATIC_SCRATCH_BYTES (8u << 20)
size_t basiskv_static_scratch_bytes(void);

/* basiskv_decode_step without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The same launches and results as
 * basiskv_decode_step, bit for bit; the workspace is a file-scope device
 * array of the library, BASISKV_STATIC_SCRATCH_BYTES (8 MiB) per GPU, held
 * from the first call on that GPU until the process ends; its device address
 * is looked up once per device (hipGetSymbolAddress) on the first call made
 * with that device current.  Nothing is allocated or freed.
 * Returns ERR_WORKSPACE when basiskv_workspace_bytes(dims, top_k) exceeds
 * BASISKV_STATIC_SCRATCH_BYTES (about batch 256 at the 8B shape with r_v 96),
 * and ERR_LAUNCH if the device address cannot be obtained; all other
 * arguments and checks as for basiskv_decode_step.  Every call on one GPU
 * shares that GPU's array and finds what the previous call left in it (the
 * step zeroes what must start at zero itself; when its dims differ from the
 * previous call's on that GPU it first zeroes, with a small fill kernel on
 * `stream`, the epoch and marks that steps carry from call to call): calls
 * that overlap on one GPU -- on different streams, or from different host
 * threads -- race and must not be made. */
int32_t basiskv_decode_step_static(const basiskv_dims *dims, const void *q, const void *k_new,
                                   const void *v_new, const int32_t *start_pos, const void *A,
                                   const void *P, const void *Q, const void *E, const void *M,
                                   const basiskv_cache *cache, int32_t top_k, float scale,
                                   float *page_scores, int32_t *sel, float *u, void *y,
                                   void *stream);

/* Dense decode attention over every page, the baseline the pages compare
 * the method against (sparse decoding latency, Table 3: full-context Key and
 * Value reads).  For each query head h of KV head g:
 *   s_t = scale * q_h . k_t over the sequence's valid tokens,
 *   p = softmax(s), o[b][h] = sum_t p_t v_t.
 *   q [batch][n_q_heads][head_dim]; k_pages, v_pages: pools laid out as the
 *   Key pool ([n_kv][num_phys][head_dim/CE][page_size][CE]); block_table
 *   [batch][max_pages_per_seq] and seq_lens [batch] device; o [batch]
 *   [n_q_heads][head_dim] float32 out (0 for an empty sequence).
 * dims.r_v, r_b, r_q and recent_tokens are not used.  The output projection
 * of the dense path is basiskv_reconstruct with dims.r_v = head_dim and the
 * matrix basiskv_fuse_output_matrix builds from an identity decoder.
 * workspace: basiskv_dense_workspace_bytes, zero-filled once, as for the
 * other calls.  BASISKV_BF16 or BASISKV_BF16_FP8_E4M3 (then both pools hold
 * E4M3 codes); ERR_UNSUPPORTED for float32. */
size_t basiskv_dense_workspace_bytes(const basiskv_dims *dims);
int32_t basiskv_dense_attend(const basiskv_dims *dims, const void *q, const void *k_pages,
                             const void *v_pages, const int32_t *block_table,
                             const int32_t *seq_lens, float scale, float *o, void *workspace,
                             size_t workspace_bytes, void *stream);

/* Set-up: fuse the Value decoder into the output projection,
 *   M[n][h * r_v + i] = sum_d Bf[h / G][i][d] * W_O[h * head_dim + d][n],
 * i.e. M = (blockdiag_h(Bf_{h/G}) W_O)^T, float32 accumulation, stored in dtype
 * (bf16 for BASISKV_BF16_FP8_E4M3) in MFMA tiles: element (n, k) at
 *   ((n / 16 * (K / KS) + k / KS) * 64 + (k % KS) / KL * 16 + n % 16) * KL + k % KL,
 * KL = 16 / element bytes (8 bf16, 4 float32), KS = 4 * KL, K = n_q_heads * r_v;
 * each MFMA step's operand (16 features x KS slots) is one contiguous 1 KB run.
 *   Bf [n_kv][r_v][head_dim];  W_O [n_q_heads * head_dim][hidden];
 *   M: hidden * n_q_heads * r_v elements out (same size as the plain matrix). */
int32_t basiskv_fuse_output_matrix(const basiskv_dims *dims, const void *Bf, const void *W_O,
                                   void *M, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* BASISKV_H */
