// C ABI of libbasiskv: host-side validation, workspace sizing and dispatch.
// Every entry point validates its arguments before enqueuing anything and
// returns a basiskv_status; nothing here allocates, frees or synchronises.
#include <string.h>

#include "common.hpp"

namespace bkv_host {
size_t compress_lds(const basiskv_dims &d);
bool score_supported(const basiskv_dims &d);
bool attend_supported(const basiskv_dims &d);
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
  if (d->batch < 1 || d->n_q_heads < 1 || d->n_kv_heads < 1 || d->head_dim < 1 ||
      d->hidden < 1 || d->r_v < 1 || d->r_b < 1 || d->r_q < 1 || d->page_size < 1 ||
      d->max_pages_per_seq < 1 || d->num_phys_pages < 1)
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
  if (bkv_host::routing_first(d)) {
    need_z = need_z || need_r;
    need_r = false;
  }
  if ((need_k && !c->k_pages) || (need_z && !c->z_pages) || (need_r && !c->r_pages))
    return BASISKV_ERR_NULL;
  return BASISKV_OK;
}

size_t align_up(size_t x) { return (x + 255) / 256 * 256; }

// Workspace layout:
//   [0, C)       per-(sequence, query subgroup) counters with which the attention
//                launch elects the workgroup that merges a row's splits;
//                zero after allocation, and every call leaves them zero
//   [C, C + U)   (bf16 decode step) u as the reconstruction's A operand
//   [C + U, ..)  scratch: the projected queries during routing, then the
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

size_t scratch_offset(const basiskv_dims &d) { return counter_bytes(d) + utile_bytes(d); }

int32_t *attend_counters(void *ws) { return static_cast<int32_t *>(ws); }
uint16_t *u_tiles(void *ws, const basiskv_dims &d) {
  return bkv_host::act_bf16(d)
             ? reinterpret_cast<uint16_t *>(static_cast<char *>(ws) + counter_bytes(d))
             : nullptr;
}
float *scratch(void *ws, const basiskv_dims &d) {
  return reinterpret_cast<float *>(static_cast<char *>(ws) + scratch_offset(d));
}

int32_t launched(hipError_t e) { return e == hipSuccess ? BASISKV_OK : BASISKV_ERR_LAUNCH; }

hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

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
  if (!k || !v || !start_pos || !A || !P || !E) return BASISKV_ERR_NULL;
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
  if (!q || !P || !Q || !q_proj) return BASISKV_ERR_NULL;
  return launched(bkv_host::launch_project(*d, q, P, Q, q_proj, as_stream(stream)));
}

int32_t basiskv_score_pages(const basiskv_dims *d, const float *q_proj, const basiskv_cache *c,
                            float *page_scores, void *stream) {
  int32_t st = check_dims(d);
  if (st) return st;
  if (!q_proj || !page_scores) return BASISKV_ERR_NULL;
  if ((st = check_cache(*d, c, false, true, true))) return st;
  if (!bkv_host::score_supported(*d)) return BASISKV_ERR_UNSUPPORTED;
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
  return launched(bkv_host::launch_select(*d, page_scores, seq_lens, top_k, sel, as_stream(stream)));
}

int32_t basiskv_route_pages(const basiskv_dims *d, const void *q, const void *P, const void *Q,
                            const basiskv_cache *c, int32_t top_k, float *page_scores,
                            int32_t *sel, void *ws, size_t ws_bytes, void *stream) {
  int32_t st = check_dims(d);
  if (st) return st;
  if (!q || !P || !Q || !page_scores || !sel) return BASISKV_ERR_NULL;
  if ((st = check_cache(*d, c, false, true, true))) return st;
  if (top_k < 1) return BASISKV_ERR_SHAPE;
  if (!ws || ws_bytes < scratch_offset(*d) + qproj_bytes(*d)) return BASISKV_ERR_WORKSPACE;
  if (!bkv_host::score_supported(*d)) return BASISKV_ERR_UNSUPPORTED;
  float *q_proj = scratch(ws, *d);
  hipStream_t s = as_stream(stream);
  bool unsupported = false;
  hipError_t e = bkv_host::launch_project(*d, q, P, Q, q_proj, s);
  if (e != hipSuccess) return BASISKV_ERR_LAUNCH;
  e = bkv_host::launch_score(*d, q_proj, *c, page_scores, s, &unsupported);
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
  if (!bkv_host::attend_supported(*d)) return BASISKV_ERR_UNSUPPORTED;
  if (!ws || ws_bytes < scratch_offset(*d) + partial_bytes(*d, top_k))
    return BASISKV_ERR_WORKSPACE;
  bool unsupported = false;
  hipError_t e = bkv_host::launch_attend(*d, q, *c, sel, top_k, scale, u, scratch(ws, *d),
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
  if (d->batch > (bkv_host::act_bf16(*d) ? 32 : 64)) return BASISKV_ERR_UNSUPPORTED;
  if (!output_tiles_fit(*d)) return BASISKV_ERR_UNSUPPORTED;
  return launched(bkv_host::launch_reconstruct(*d, u, nullptr, M, y, as_stream(stream)));
}

int32_t basiskv_decode_step(const basiskv_dims *d, const void *q, const void *k_new,
                            const void *v_new, const int32_t *start_pos, const void *A,
                            const void *P, const void *Q, const void *E, const void *M,
                            const basiskv_cache *c, int32_t top_k, float scale,
                            float *page_scores, int32_t *sel, float *u, void *y, void *ws,
                            size_t ws_bytes, void *stream) {
  int32_t st = check_dims(d);
  if (st) return st;
  if (!q || !k_new || !v_new || !start_pos || !A || !P || !Q || !E || !M || !page_scores ||
      !sel || !u || !y)
    return BASISKV_ERR_NULL;
  if ((st = check_cache(*d, c, true, true, true))) return st;
  if (top_k < 1) return BASISKV_ERR_SHAPE;
  if (d->r_v > bkv::kHeadDim || d->r_q > bkv::kHeadDim) return BASISKV_ERR_UNSUPPORTED;
  if (!bkv_host::score_supported(*d) || !bkv_host::attend_supported(*d))
    return BASISKV_ERR_UNSUPPORTED;
  if (d->batch > (bkv_host::act_bf16(*d) ? 32 : 64)) return BASISKV_ERR_UNSUPPORTED;
  if (!output_tiles_fit(*d)) return BASISKV_ERR_UNSUPPORTED;
  const size_t a = qproj_bytes(*d), b = partial_bytes(*d, top_k);
  if (!ws || ws_bytes < scratch_offset(*d) + (a > b ? a : b)) return BASISKV_ERR_WORKSPACE;
  hipStream_t s = as_stream(stream);
  float *scr = scratch(ws, *d);
  bool unsupported = false;
  // (a0) + (a1) in one launch, then (a2), (a3), (a4), (a5)
  if (bkv_host::launch_step_prologue(*d, q, k_new, v_new, start_pos, A, P, Q, E, *c, scr, s) !=
      hipSuccess)
    return BASISKV_ERR_LAUNCH;
  hipError_t e = bkv_host::launch_score(*d, scr, *c, page_scores, s, &unsupported);
  if (e != hipSuccess || unsupported) return BASISKV_ERR_LAUNCH;
  if (bkv_host::launch_select(*d, page_scores, c->seq_lens, top_k, sel, s) != hipSuccess)
    return BASISKV_ERR_LAUNCH;
  uint16_t *ut = u_tiles(ws, *d);  // attention also leaves u as the reconstruction's operand
  e = bkv_host::launch_attend(*d, q, *c, sel, top_k, scale, u, scr, attend_counters(ws), ut, s,
                              &unsupported);
  if (e != hipSuccess || unsupported) return BASISKV_ERR_LAUNCH;
  return launched(bkv_host::launch_reconstruct(*d, u, ut, M, y, s));
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
  if (!bkv_host::attend_supported(dd)) return BASISKV_ERR_UNSUPPORTED;
  if (!ws || ws_bytes < scratch_offset(dd) + partial_bytes(dd, dd.max_pages_per_seq))
    return BASISKV_ERR_WORKSPACE;
  basiskv_cache c{};
  c.k_pages = const_cast<void *>(k_pages);
  c.z_pages = const_cast<void *>(v_pages);  // Values in the latent's place
  c.block_table = block_table;
  c.seq_lens = seq_lens;
  bool unsupported = false;
  hipError_t e = bkv_host::launch_attend(dd, q, c, nullptr, dd.max_pages_per_seq, scale, o,
                                         scratch(ws, dd), attend_counters(ws), nullptr,
                                         as_stream(stream), &unsupported);
  if (unsupported) return BASISKV_ERR_UNSUPPORTED;
  return launched(e);
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
