// C ABI of libbasiskv: host-side validation, workspace sizing and dispatch.
// Every entry point validates its arguments before enqueuing anything and
// returns a basiskv_status; nothing here allocates, frees or synchronises.
#include <mutex>
#include <string.h>

#include "common.hpp"

namespace bkv_host {
size_t compress_lds(const basiskv_dims &d);
bool score_supported(const basiskv_dims &d);
}

namespace {

constexpr int kMaxPages = 32768;
constexpr int kMaxGroup = 16;

bool pow2_page(int s) { return s == 4 || s == 8 || s == 16 || s == 32 || s == 64; }

// Sizes common to every call.
int32_t check_dims(const basiskv_dims *d) {
  if (!d) return BASISKV_ERR_NULL;
  if (d->dtype != BASISKV_F32 && d->dtype != BASISKV_BF16 && d->dtype != BASISKV_BF16_FP8_E4M3)
    return BASISKV_ERR_UNSUPPORTED;
  // r_b = 0 (a residual-only router) or r_q = 0 (a latent-only router) is
  // allowed, not both
  if (d->batch < 1 || d->n_q_heads < 1 || d->n_kv_heads < 1 || d->head_dim < 1 ||
      d->hidden < 1 || d->r_v < 1 || d->r_b < 0 || d->r_q < 0 || d->r_b + d->r_q < 1 ||
      d->page_size < 1 || d->max_pages_per_seq < 1 || d->num_phys_pages < 1)
    return BASISKV_ERR_SHAPE;
  if (d->n_q_heads % d->n_kv_heads != 0 || d->r_b > d->r_v) return BASISKV_ERR_SHAPE;
  if (d->recent_tokens < 0) return BASISKV_ERR_SHAPE;
  if (d->page_layout != BASISKV_LAYOUT_SEPARATE && d->page_layout != BASISKV_LAYOUT_ROUTING_FIRST)
    return BASISKV_ERR_UNSUPPORTED;
  if (d->head_dim != bkv::kHeadDim) return BASISKV_ERR_UNSUPPORTED;
  if (!pow2_page(d->page_size)) return BASISKV_ERR_UNSUPPORTED;
  const int ce = bkv_host::cache_chunk(*d);  // whole 16-byte chunks per cached row
  if (d->r_v % ce || d->r_b % ce || d->r_q % ce) return BASISKV_ERR_UNSUPPORTED;
  if (d->n_q_heads / d->n_kv_heads > kMaxGroup) return BASISKV_ERR_UNSUPPORTED;
  if (d->max_pages_per_seq > kMaxPages) return BASISKV_ERR_UNSUPPORTED;
  if ((int64_t)d->max_pages_per_seq * d->page_size > INT32_MAX / 2) return BASISKV_ERR_SHAPE;
  return BASISKV_OK;
}

// The fused output matrix is stored in MFMA tiles: 16 output features by 32
// (bf16) or 16 (float32) contraction slots.
bool output_tiles_fit(const basiskv_dims &d) {
  const int kstep = bkv_host::act_bf16(d) ? 32 : 16;
  return d.hidden % 16 == 0 && (d.n_q_heads * d.r_v) % kstep == 0;
}

// (with the routing-first layout the residual lives in the latent pool)
int32_t check_cache(const basiskv_dims &d, const basiskv_cache *c, bool need_k, bool need_z,
                    bool need_r) {
  if (!c || !c->block_table || !c->seq_lens) return BASISKV_ERR_NULL;
  if (d.r_q == 0) need_r = false;  // no residual codes to read or write
  if (bkv_host::routing_first(d)) {
    need_z = need_z || need_r;
    need_r = false;
  }
  if ((need_k && !c->k_pages) || (need_z && !c->z_pages) || (need_r && !c->r_pages))
    return BASISKV_ERR_NULL;
  return BASISKV_OK;
}

bool has_rope(const basiskv_cache *c) { return c && c->rope_inv_freq; }

// Routing of this cache is supported: projected queries, or (with RoPE) the
// rotated predicted Keys.
bool routing_supported(const basiskv_dims &d, const basiskv_cache *c) {
  return has_rope(c) ? bkv_host::score_rope_supported(d) : bkv_host::score_supported(d);
}

// The routing factors a call needs: P when r_b > 0, Q (routing) and E
// (compression) when r_q > 0.
bool missing_factor(const basiskv_dims &d, const void *P, const void *QorE) {
  return (d.r_b > 0 && !P) || (d.r_q > 0 && !QorE);
}

size_t align_up(size_t x) { return (x + 255) / 256 * 256; }

// Workspace layout:
//   [0, C)       per-(sequence, query subgroup) counters with which the attention
//                launch elects the workgroup that merges a row's splits;
//                zero after allocation, and every call leaves them zero
//   [C, C + U)   (bf16 decode step) u as the reconstruction's A operand
//   [C + U, +N)  (decode step) the new token's score per (sequence, KV head),
//                from the scoring launch to the selection launch
//   [.., +T)     (bf16 / E4M3 decode step, groups of a multiple of 4 heads)
//                the epoch word of the last step that projected its queries
//                inside the scoring launch (advanced by the step's selection
//                launch), then per (sequence, KV head, block of 16 projection
//                rows) the epoch that last projected it; zero after
//                allocation, which no step's epoch is
//   [C + U + N + T, ..)  scratch: the projected queries during routing, then the
//                attention splits' partial records (stream order keeps the
//                two uses apart)
size_t counter_bytes(const basiskv_dims &d) {  // one per (sequence, query subgroup)
  return align_up((size_t)d.batch * d.n_kv_heads * bkv_host::attend_group_split(d) *
                  sizeof(int32_t));
}

size_t utile_bytes(const basiskv_dims &d) {
  if (!bkv_host::act_bf16(d)) return 0;
  const size_t tiles = (size_t)(d.batch + 7) / 8;
  return align_up(tiles * ((size_t)d.n_q_heads * d.r_v / 32) * 1024);
}

size_t qproj_bytes(const basiskv_dims &d) {
  return align_up((size_t)d.batch * d.n_q_heads * (d.r_b + d.r_q) * sizeof(float));
}

size_t partial_bytes(const basiskv_dims &d, int32_t top_k) {
  const int ns = bkv_host::attend_splits(d, top_k);
  return align_up((size_t)d.batch * d.n_q_heads * ns * (d.r_v + 2) * sizeof(float));
}

size_t newtok_bytes(const basiskv_dims &d) {
  return align_up((size_t)d.batch * d.n_kv_heads * sizeof(float));
}

// (decode step with the projection inside the scoring launch) the done-tags
// of the projection's row blocks; sized wherever the scan may take the
// projection in (bf16 activations, groups of a multiple of 4 heads), so that
// the workspace does not depend on the page format
constexpr size_t kEpochBytes = 256;  // the epoch word, alone in its 256 bytes
size_t qtag_bytes(const basiskv_dims &d) {
  const int G = d.n_q_heads / d.n_kv_heads;
  return bkv_host::act_bf16(d) && G % 4 == 0
             ? kEpochBytes + align_up((size_t)d.batch * d.n_kv_heads *
                                      ((d.r_b + d.r_q + 15) / 16) * sizeof(uint32_t))
             : 0;
}

size_t scratch_offset(const basiskv_dims &d) {
  return counter_bytes(d) + utile_bytes(d) + newtok_bytes(d) + qtag_bytes(d);
}

int32_t *attend_counters(void *ws) { return static_cast<int32_t *>(ws); }
uint16_t *u_tiles(void *ws, const basiskv_dims &d) {
  return bkv_host::act_bf16(d)
             ? reinterpret_cast<uint16_t *>(static_cast<char *>(ws) + counter_bytes(d))
             : nullptr;
}
float *newtok_scores(void *ws, const basiskv_dims &d) {
  return reinterpret_cast<float *>(static_cast<char *>(ws) + counter_bytes(d) + utile_bytes(d));
}
uint32_t *epoch_word(void *ws, const basiskv_dims &d) {
  return reinterpret_cast<uint32_t *>(static_cast<char *>(ws) + counter_bytes(d) + utile_bytes(d) +
                                      newtok_bytes(d));
}
uint32_t *qtag_area(void *ws, const basiskv_dims &d) {
  return epoch_word(ws, d) + kEpochBytes / sizeof(uint32_t);
}
float *scratch_area(void *ws, const basiskv_dims &d) {
  return reinterpret_cast<float *>(static_cast<char *>(ws) + scratch_offset(d));
}

int32_t launched(hipError_t e) { return e == hipSuccess ? BASISKV_OK : BASISKV_ERR_LAUNCH; }

hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

// ---- the no-allocation decode step's scratch ----
// Device memory of the library itself (one copy per GPU, held until the
// process ends) standing in for the caller's workspace.  In host code the
// array's name is only a host-side stand-in: kernels get the device address
// that hipGetSymbolAddress returns for the current device.
constexpr size_t kStaticScratchBytes = (size_t)BASISKV_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices];  // per device, looked up on first use

// Device address of `scratch` on the current device (looked up once per device).
basiskv_dims g_scratch_dims[kMaxDevices];  // per device, the dims of the last step on it
bool g_scratch_used[kMaxDevices];

// Zeroes n 32-bit words (a fill kernel, not a memset: the step may be
// captured in a graph).
__global__ void zero_words_kernel(uint32_t *p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0;
}

// The scratch of the current device.  When the step's dims differ from the
// last step run on it, the words that a step carries over to the next (the
// projection's epoch and done-tags, at a place that depends on the dims) are
// zeroed first on the step's stream, so that nothing an earlier step of other
// dims left there can pass for this step's.
int32_t static_scratch(void **out, const basiskv_dims &d, hipStream_t s) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return BASISKV_ERR_LAUNCH;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return BASISKV_ERR_LAUNCH;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  if (!g_scratch_used[dev] || memcmp(&g_scratch_dims[dev], &d, sizeof d) != 0) {
    const size_t words = qtag_bytes(d) / sizeof(uint32_t);
    if (words > 0) {
      hipLaunchKernelGGL(zero_words_kernel, dim3(16), dim3(256), 0, s, epoch_word(*out, d), words);
      if (hipGetLastError() != hipSuccess) return BASISKV_ERR_LAUNCH;
    }
    g_scratch_dims[dev] = d;
    g_scratch_used[dev] = true;
  }
  return BASISKV_OK;
}

}  // namespace

extern "C" {

const char *basiskv_status_string(int32_t status) {
  switch (status) {
    case BASISKV_OK: return "ok";
    case BASISKV_ERR_NULL: return "null pointer argument";
    case BASISKV_ERR_SHAPE: return "inconsistent or out-of-range sizes";
    case BASISKV_ERR_UNSUPPORTED: return "unsupported configuration";
    case BASISKV_ERR_WORKSPACE: return "workspace missing or too small";
    case BASISKV_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

size_t basiskv_workspace_bytes(const basiskv_dims *d, int32_t top_k) {
  if (check_dims(d) != BASISKV_OK || top_k < 1) return 0;
  const size_t a = qproj_bytes(*d), b = partial_bytes(*d, top_k);
  return scratch_offset(*d) + (a > b ? a : b);
}

int32_t basiskv_compress_prefill(const basiskv_dims *d, const void *k, const void *v,
                                 const int32_t *start_pos, int32_t n_tokens, const void *A,
                                 const void *P, const void *E, const basiskv_cache *c,
                                 void *stream) {
  int32_t st = check_dims(d);
  if (st) return st;
  if (!k || !v || !start_pos || !A || missing_factor(*d, P, E)) return BASISKV_ERR_NULL;
  if ((st = check_cache(*d, c, true, true, true))) return st;
  if (n_tokens < 1) return BASISKV_ERR_SHAPE;
  if (d->r_v % 16 || d->r_q % 16) return BASISKV_ERR_UNSUPPORTED;  // 16-wide MFMA output tiles
  if ((int64_t)d->batch * n_tokens > INT32_MAX / 2) return BASISKV_ERR_SHAPE;
  if (bkv_host::compress_lds(*d) > 160 * 1024) return BASISKV_ERR_UNSUPPORTED;
  return launched(bkv_host::launch_compress(*d, k, v, start_pos, n_tokens, A, P, E, *c,
                                            as_stream(stream)));
}

int32_t basiskv_project_queries(const basiskv_dims *d, const void *q, const void *P,
                                const void *Q, float *q_proj, void *stream) {
  int32_t st = check_dims(d);
  if (st) return st;
  if (!q || missing_factor(*d, P, Q) || !q_proj) return BASISKV_ERR_NULL;
  return launched(bkv_host::launch_project(*d, q, P, Q, q_proj, as_stream(stream)));
}

int32_t basiskv_score_pages(const basiskv_dims *d, const float *q_proj, const basiskv_cache *c,
                            float *page_scores, void *stream) {
  int32_t st = check_dims(d);
  if (st) return st;
  if (!q_proj || !page_scores) return BASISKV_ERR_NULL;
  if ((st = check_cache(*d, c, false, true, true))) return st;
  // with RoPE the logits depend on each token's position: projected queries
  // cannot carry them (route_pages and decode_step take the raw queries)
  if (has_rope(c) || !bkv_host::score_supported(*d)) return BASISKV_ERR_UNSUPPORTED;
  bool unsupported = false;
  hipError_t e = bkv_host::launch_score(*d, q_proj, *c, page_scores, as_stream(stream),
                                        &unsupported);
  if (unsupported) return BASISKV_ERR_UNSUPPORTED;
  return launched(e);
}

int32_t basiskv_select_pages(const basiskv_dims *d, const float *page_scores,
                             const int32_t *seq_lens, int32_t top_k, int32_t *sel, void *stream) {
  int32_t st = check_dims(d);
  if (st) return st;
  if (!page_scores || !seq_lens || !sel) return BASISKV_ERR_NULL;
  if (top_k < 1) return BASISKV_ERR_SHAPE;
  // (the scores are only read: nothing is folded in without new-token scores)
  return launched(bkv_host::launch_select(*d, const_cast<float *>(page_scores), seq_lens, top_k,
                                          sel, as_stream(stream)));
}

int32_t basiskv_score_pages_rope(const basiskv_dims *d, const void *q, const void *P,
                                 const void *Q, const basiskv_cache *c, float *page_scores,
                                 void *stream) {
  int32_t st = check_dims(d);
  if (st) return st;
  if (!q || missing_factor(*d, P, Q) || !page_scores || !has_rope(c)) return BASISKV_ERR_NULL;
  if ((st = check_cache(*d, c, false, true, true))) return st;
  if (!bkv_host::score_rope_supported(*d)) return BASISKV_ERR_UNSUPPORTED;
  bool unsupported = false;
  hipError_t e = bkv_host::launch_score_rope(*d, q, P, Q, *c, page_scores, as_stream(stream),
                                             &unsupported);
  if (unsupported) return BASISKV_ERR_UNSUPPORTED;
  return launched(e);
}

int32_t basiskv_route_pages(const basiskv_dims *d, const void *q, const void *P, const void *Q,
                            const basiskv_cache *c, int32_t top_k, float *page_scores,
                            int32_t *sel, void *ws, size_t ws_bytes, void *stream) {
  int32_t st = check_dims(d);
  if (st) return st;
  if (!q || missing_factor(*d, P, Q) || !page_scores || !sel) return BASISKV_ERR_NULL;
  if ((st = check_cache(*d, c, false, true, true))) return st;
  if (top_k < 1) return BASISKV_ERR_SHAPE;
  if (!routing_supported(*d, c)) return BASISKV_ERR_UNSUPPORTED;
  if (!ws || ws_bytes < scratch_offset(*d) + qproj_bytes(*d)) return BASISKV_ERR_WORKSPACE;
  float *q_proj = scratch_area(ws, *d);
  hipStream_t s = as_stream(stream);
  bool unsupported = false;
  hipError_t e;
  if (has_rope(c)) {
    e = bkv_host::launch_score_rope(*d, q, P, Q, *c, page_scores, s, &unsupported);
  } else {
    e = bkv_host::launch_project(*d, q, P, Q, q_proj, s);
    if (e != hipSuccess) return BASISKV_ERR_LAUNCH;
    e = bkv_host::launch_score(*d, q_proj, *c, page_scores, s, &unsupported);
  }
  if (e != hipSuccess || unsupported) return BASISKV_ERR_LAUNCH;
  return launched(bkv_host::launch_select(*d, page_scores, c->seq_lens, top_k, sel, s));
}

int32_t basiskv_sparse_attend(const basiskv_dims *d, const void *q, const basiskv_cache *c,
                              const int32_t *sel, int32_t top_k, float scale, float *u, void *ws,
                              size_t ws_bytes, void *stream) {
  int32_t st = check_dims(d);
  if (st) return st;
  if (!q || !sel || !u) return BASISKV_ERR_NULL;
  if ((st = check_cache(*d, c, true, true, false))) return st;
  if (top_k < 1) return BASISKV_ERR_SHAPE;
  if (!bkv_host::attend_supported(*d, has_rope(c))) return BASISKV_ERR_UNSUPPORTED;
  if (!ws || ws_bytes < scratch_offset(*d) + partial_bytes(*d, top_k))
    return BASISKV_ERR_WORKSPACE;
  bool unsupported = false;
  hipError_t e = bkv_host::launch_attend(*d, q, *c, sel, top_k, scale, u, scratch_area(ws, *d),
                                         attend_counters(ws), nullptr, as_stream(stream),
                                         &unsupported);
  if (unsupported) return BASISKV_ERR_UNSUPPORTED;
  return launched(e);
}

int32_t basiskv_reconstruct(const basiskv_dims *d, const float *u, const void *M, void *y,
                            void *stream) {
  int32_t st = check_dims(d);
  if (st) return st;
  if (!u || !M || !y) return BASISKV_ERR_NULL;
  if (!output_tiles_fit(*d)) return BASISKV_ERR_UNSUPPORTED;
  return launched(bkv_host::launch_reconstruct(*d, u, nullptr, M, y, as_stream(stream)));
}

}  // extern "C"

namespace {

// Host-side checks of a decode step (no HIP call).
int32_t check_decode_step(const basiskv_dims *d, const void *q, const void *k_new,
                          const void *v_new, const int32_t *start_pos, const void *A,
                          const void *P, const void *Q, const void *E, const void *M,
                          const basiskv_cache *c, int32_t top_k, float *page_scores, int32_t *sel,
                          float *u, void *y, const void *ws, size_t ws_bytes) {
  int32_t st = check_dims(d);
  if (st) return st;
  if (!q || !k_new || !v_new || !start_pos || !A || missing_factor(*d, P, Q) ||
      missing_factor(*d, P, E) || !M || !page_scores || !sel || !u || !y)
    return BASISKV_ERR_NULL;
  if ((st = check_cache(*d, c, true, true, true))) return st;
  if (top_k < 1) return BASISKV_ERR_SHAPE;
  if (d->r_v > bkv::kHeadDim || d->r_q > bkv::kHeadDim) return BASISKV_ERR_UNSUPPORTED;
  if (!routing_supported(*d, c) || !bkv_host::attend_supported(*d, has_rope(c)))
    return BASISKV_ERR_UNSUPPORTED;
  if (!output_tiles_fit(*d)) return BASISKV_ERR_UNSUPPORTED;
  const size_t a = qproj_bytes(*d), b = partial_bytes(*d, top_k);
  if (!ws || ws_bytes < scratch_offset(*d) + (a > b ? a : b)) return BASISKV_ERR_WORKSPACE;
  return BASISKV_OK;
}

// Whether the decode step compresses its new tokens inside the scoring
// launch.  There the compression (a chain of dependent memory round trips,
// longer under the scan's load, in a register budget kept to the scan's)
// is hidden only behind a long scan.  Measured per step against compressing
// in the projection's launch: with routing reads of 200 MB and more
// (llama8b- and qwen32b-shaped layers at 32K context, bf16 or E4M3 pages)
// 0.5-2 us shorter; with 150 MB or less (4K context, the 4-token-page
// routers) 1-4 us longer while the projection kept a launch of its own, the
// compression outlasting the scan.
constexpr double kBesideScanMinBytes = 160.0 * (1 << 20);
constexpr double kBesideProjMinBytes = 64.0 * (1 << 20);

// Whether the step's scoring launch takes the query projection in (its scan
// then waits on the projection's marks): bf16 pages on the matrix-core logits.
// E4M3 pages keep the projection's own launch: with it inside, their scans
// measured 1-4.6 us longer (context sweep, 32K-96K, batch 8), none shorter.
bool projects_beside_scan(const basiskv_dims &d) {
  return bkv_host::score_projects(d) && !bkv_host::cache_fp8(d);
}
bool compress_beside_scan(const basiskv_dims &d) {
  const double bytes = (double)d.batch * d.n_kv_heads * d.max_pages_per_seq * d.page_size *
                       (d.r_b + d.r_q) * (bkv_host::cache_fp8(d) ? 1 : bkv_host::act_bf16(d) ? 2 : 4);
  if (bytes >= kBesideScanMinBytes) return true;
  // a shorter scan of 64 MiB or more takes both in where the query projection
  // can come too (the step then has no launch before the scan) over bf16
  // pages at least 32 routing dims wide.  Measured against the separate
  // launch: 4K-context llama8b-shaped layer 58.3 -> 55.5 us, the adopted
  // router 68.3 -> 66.6 us, R32 69.4 -> 67.0 us, batch-1 llama8b-shaped steps
  // at 64K and 96K context (101 and 151 MB) 2 us shorter; narrower scans (B16:
  // +0.8 us), E4M3 pages (no change) and scans under 64 MiB (batch 1 at 24K
  // and 32K context: 1.5-3 us longer, nearly every scanning workgroup waiting
  // on the projection) keep the launch.
  return bytes >= kBesideProjMinBytes && projects_beside_scan(d) && d.r_b + d.r_q >= 32;
}

// The launches of a decode step, after check_decode_step.
int32_t launch_decode_step(const basiskv_dims *d, const void *q, const void *k_new,
                           const void *v_new, const int32_t *start_pos, const void *A,
                           const void *P, const void *Q, const void *E, const void *M,
                           const basiskv_cache *c, int32_t top_k, float scale, float *page_scores,
                           int32_t *sel, float *u, void *y, void *ws, hipStream_t s) {
  float *scr = scratch_area(ws, *d);
  bool unsupported = false;
  const int n_counters = (int)(counter_bytes(*d) / sizeof(int32_t));
  const bool rope = has_rope(c);
  const bool beside = !rope && compress_beside_scan(*d);
  // with a long scan on the matrix-core logits, the query projection (a1)
  // runs inside the scoring launch too (it also clears the attention's merge
  // counters there)
  const bool project_beside = beside && projects_beside_scan(*d);
  // (a1) in one launch, which also clears the attention's merge counters;
  // with a long scan the new tokens' compression (a0) runs inside the scoring
  // launch (a2), beside the scan, and the selection (a3) folds their scores
  // in; otherwise (and with rotary positions) it shares the first launch.
  // Then (a4), (a5).
  if (!project_beside &&
      bkv_host::launch_step_prologue(*d, q, k_new, v_new, start_pos, A, P, Q, E, *c, scr,
                                     attend_counters(ws), n_counters, s, !beside) != hipSuccess)
    return BASISKV_ERR_LAUNCH;
  bkv_host::StepTokens tokens{k_new,     v_new, A, P, E, start_pos, newtok_scores(ws, *d), q, Q,
                              project_beside ? qtag_area(ws, *d) : nullptr,
                              project_beside ? epoch_word(ws, *d) : nullptr,
                              attend_counters(ws), n_counters};
  hipError_t e = rope ? bkv_host::launch_score_rope(*d, q, P, Q, *c, page_scores, s, &unsupported)
                      : bkv_host::launch_score(*d, scr, *c, page_scores, s, &unsupported,
                                               beside ? &tokens : nullptr);
  if (e != hipSuccess || unsupported) return BASISKV_ERR_LAUNCH;
  if (bkv_host::launch_select(*d, page_scores, c->seq_lens, top_k, sel, s,
                              beside ? start_pos : nullptr,
                              beside ? tokens.new_scores : nullptr,
                              project_beside ? epoch_word(ws, *d) : nullptr) != hipSuccess)
    return BASISKV_ERR_LAUNCH;
  uint16_t *ut = u_tiles(ws, *d);  // attention also leaves u as the reconstruction's operand
  e = bkv_host::launch_attend(*d, q, *c, sel, top_k, scale, u, scr, attend_counters(ws), ut, s,
                              &unsupported);
  if (e != hipSuccess || unsupported) return BASISKV_ERR_LAUNCH;
  return launched(bkv_host::launch_reconstruct(*d, u, ut, M, y, s));
}

}  // namespace

extern "C" {

int32_t basiskv_decode_step(const basiskv_dims *d, const void *q, const void *k_new,
                            const void *v_new, const int32_t *start_pos, const void *A,
                            const void *P, const void *Q, const void *E, const void *M,
                            const basiskv_cache *c, int32_t top_k, float scale,
                            float *page_scores, int32_t *sel, float *u, void *y, void *ws,
                            size_t ws_bytes, void *stream) {
  const int32_t st = check_decode_step(d, q, k_new, v_new, start_pos, A, P, Q, E, M, c, top_k,
                                       page_scores, sel, u, y, ws, ws_bytes);
  if (st) return st;
  return launch_decode_step(d, q, k_new, v_new, start_pos, A, P, Q, E, M, c, top_k, scale,
                            page_scores, sel, u, y, ws, as_stream(stream));
}

size_t basiskv_static_scratch_bytes(void) { return kStaticScratchBytes; }

int32_t basiskv_decode_step_static(const basiskv_dims *d, const void *q, const void *k_new,
                                   const void *v_new, const int32_t *start_pos, const void *A,
                                   const void *P, const void *Q, const void *E, const void *M,
                                   const basiskv_cache *c, int32_t top_k, float scale,
                                   float *page_scores, int32_t *sel, float *u, void *y,
                                   void *stream) {
  // every host check first, against the scratch's size (a stand-in pointer:
  // nothing is dereferenced or launched before the real address is known)
  const void *stand_in = &kStaticScratchBytes;
  int32_t st = check_decode_step(d, q, k_new, v_new, start_pos, A, P, Q, E, M, c, top_k,
                                 page_scores, sel, u, y, stand_in, kStaticScratchBytes);
  if (st) return st;
  void *ws = nullptr;
  if ((st = static_scratch(&ws, *d, as_stream(stream)))) return st;
  return launch_decode_step(d, q, k_new, v_new, start_pos, A, P, Q, E, M, c, top_k, scale,
                            page_scores, sel, u, y, ws, as_stream(stream));
}

// The dense baseline's sizes: the attention sums Values (head_dim wide) in the
// latent's place and attends every page, with no recent window.
static basiskv_dims dense_dims(const basiskv_dims &d) {
  basiskv_dims dd = d;
  dd.r_v = d.head_dim;
  dd.recent_tokens = 0;
  dd.page_layout = BASISKV_LAYOUT_SEPARATE;  // the Key and Value pools are plain
  return dd;
}

size_t basiskv_dense_workspace_bytes(const basiskv_dims *d) {
  if (check_dims(d) != BASISKV_OK) return 0;
  const basiskv_dims dd = dense_dims(*d);
  return scratch_offset(dd) + partial_bytes(dd, dd.max_pages_per_seq);
}

int32_t basiskv_dense_attend(const basiskv_dims *d, const void *q, const void *k_pages,
                             const void *v_pages, const int32_t *block_table,
                             const int32_t *seq_lens, float scale, float *o, void *ws,
                             size_t ws_bytes, void *stream) {
  int32_t st = check_dims(d);
  if (st) return st;
  if (!q || !k_pages || !v_pages || !block_table || !seq_lens || !o) return BASISKV_ERR_NULL;
  const basiskv_dims dd = dense_dims(*d);
  if (!bkv_host::attend_supported(dd, false)) return BASISKV_ERR_UNSUPPORTED;
  if (!ws || ws_bytes < scratch_offset(dd) + partial_bytes(dd, dd.max_pages_per_seq))
    return BASISKV_ERR_WORKSPACE;
  basiskv_cache c{};
  c.k_pages = const_cast<void *>(k_pages);
  c.z_pages = const_cast<void *>(v_pages);  // Values in the latent's place
  c.block_table = block_table;
  c.seq_lens = seq_lens;
  bool unsupported = false;
  hipError_t e = bkv_host::launch_attend(dd, q, c, nullptr, dd.max_pages_per_seq, scale, o,
                                         scratch_area(ws, dd), attend_counters(ws), nullptr,
                                         as_stream(stream), &unsupported);
  if (unsupported) return BASISKV_ERR_UNSUPPORTED;
  return launched(e);
}

int32_t basiskv_pack_output_matrix(const basiskv_dims *d, const void *M_plain, void *M,
                                   void *stream) {
  int32_t st = check_dims(d);
  if (st) return st;
  if (!M_plain || !M) return BASISKV_ERR_NULL;
  if (M_plain == M) return BASISKV_ERR_SHAPE;  // not in place
  if (!output_tiles_fit(*d)) return BASISKV_ERR_UNSUPPORTED;
  return launched(bkv_host::launch_pack_output(*d, M_plain, M, as_stream(stream)));
}

int32_t basiskv_fuse_output_matrix(const basiskv_dims *d, const void *Bf, const void *W_O, void *M,
                                   void *stream) {
  int32_t st = check_dims(d);
  if (st) return st;
  if (!Bf || !W_O || !M) return BASISKV_ERR_NULL;
  if (!output_tiles_fit(*d)) return BASISKV_ERR_UNSUPPORTED;
  return launched(bkv_host::launch_fuse(*d, Bf, W_O, M, as_stream(stream)));
}

}  // extern "C"
