// Routing kernels: query projection (a1), page scoring (a2), top-k page
// selection (a3).  BasisKV (arXiv 2611.02583): the abstract's latent-based Key
// routing with a Key-specific residual; appendix Table 4's routing read widths
// (r_b latent dims + r_q residual dims per context token); Table 9's caption
// (routing by page, with a page budget).
#include "decode_bodies.hpp"
#include "topk.hpp"

namespace bkv {

// ---------------------------------------------------------------------------
// (a1) query projection launch; the body is in decode_bodies.hpp.
// grid (ceil((r_b + r_q) / 8), n_kv, batch), 128 threads.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(128) void project_queries_kernel(
    const T *__restrict__ q, const T *__restrict__ P, const T *__restrict__ Q,
    float *__restrict__ q_proj, int n_q, int n_kv, int rb, int rq) {
  project_body<T, 128>(q, P, Q, q_proj, n_q, n_kv, rb, rq, blockIdx.x, blockIdx.y, blockIdx.z);
}

// ---------------------------------------------------------------------------
// (a3) exact top-k per (sequence, KV head); topk_row is in topk.hpp.
// ---------------------------------------------------------------------------
// Standalone selection: grid (n_kv, batch), 64 * NWV threads.  With a recent
// window of `recent` tokens the candidates are the pages before the window.
// With new_scores (a decode step whose scoring left each sequence's new token,
// at new_pos[b], to the compression workgroups) that token's score is first
// folded into its page's score, max(page, token), which is also written back.
template <int KPT, int NWV>
__global__ __launch_bounds__(64 * NWV) void topk_select_kernel(
    float *__restrict__ scores, const int32_t *__restrict__ seq_lens,
    int32_t *__restrict__ sel, int n_kv, int max_pages, int page_size, int cap, int k,
    int recent, const int32_t *__restrict__ new_pos, const float *__restrict__ new_scores,
    uint32_t *__restrict__ epoch) {
  const int g = blockIdx.x, b = blockIdx.y;
  // (decode step with the projection inside the scoring launch) the scan is
  // over: the next step's scoring launch takes the next epoch
  if (epoch && g == 0 && b == 0 && threadIdx.x == 0)
    store_coherent_u32(epoch, load_coherent_u32(epoch) + 1);
  // the whole row is requested before the sequence length arrives
  float *row = scores + ((int64_t)b * n_kv + g) * max_pages;
  const int base = (threadIdx.x >> 6) * 64 * KPT + (threadIdx.x & 63);
  float v[KPT];
#pragma unroll
  for (int j = 0; j < KPT; ++j) v[j] = base + 64 * j < max_pages ? row[base + 64 * j] : 0.f;
  if (new_scores) {
    const int pos = new_pos[b];
    const float ns = new_scores[(int64_t)b * n_kv + g];
    const int np = pos >= 0 && pos < cap ? pos / page_size : -1;
    if (np >= 0 && ns != -INFINITY) {  // (-inf: the token does not count)
#pragma unroll
      for (int j = 0; j < KPT; ++j)
        if (base + 64 * j == np) {
          v[j] = fmaxf(v[j], ns);
          row[np] = v[j];
        }
    }
  }
  const int L = clamp_len(seq_lens[b], cap);
  const int NP = recent > 0 ? max(0, L - recent) / page_size : (L + page_size - 1) / page_size;
  int32_t *out = sel + ((int64_t)b * n_kv + g) * k;
  if (k >= NP) {
    for (int i = threadIdx.x; i < k; i += blockDim.x) out[i] = i < NP ? i : -1;
    return;
  }
  topk_row<KPT, NWV>(v, KPT, NP, k, [&](int pos, int j) { out[pos] = base + 64 * j; });
}

// ---------------------------------------------------------------------------
// (a2) page scores.
//
// One lane per token: a wavefront scores one 64-token step (64 / page_size
// pages), each lane issuing NZ + NR 16-byte loads (its token's chunks of the
// latent and residual pages).  With the chunk-major page layout those loads
// are page_size * 16 contiguous bytes per chunk, i.e. fully coalesced.  The
// logits of bf16 and E4M3 pages for groups of 4 and 8 heads run on the matrix
// cores (MF below: G x (r_b + r_q) multiply-adds per token were the launch's
// limit for 8-head groups); float32 pages and groups of 1 or 2 heads use FMAs
// whose wave-uniform query operand comes through the scalar cache.  Page
// maxima are butterfly reductions over the page's lanes.  A workgroup is four such
// steps: many short workgroups keep more loads in flight than a few long
// ones walking several steps each.  With STREAM the page loads are marked
// non-temporal: the launch streams the pages once, and on MI355X such loads
// read faster when every instruction reads whole 128-byte lines (pages of 8
// or more tokens) and a lane has many of them in flight (8 or more chunks);
// with 64-byte runs the other half of each line is fetched again, and with
// few loads per lane their longer latency is not hidden.
// ---------------------------------------------------------------------------

// The decode step's new tokens compressed inside the scoring launch (n_append
// > 0): the first app_padded workgroups of the grid each compress the new
// token of one (sequence, KV head) -- with the low-register body, so that the
// launch keeps the scan's register budget -- and then score that token with
// the scan's own arithmetic into new_scores; the scan leaves the token at
// start_pos[b] out of its page's score, and the selection launch takes the
// maximum of the two.  Max is exact, so the page scores are those of scoring
// after the compression, while the compression's chain of round trips runs
// beside the scan instead of before it.
//
// The query projection inside the scoring launch as well (n_proj > 0, the
// matrix-core logits only): the grid's first proj_padded workgroups each
// project 16 rows of [P_g; Q_g] for one (sequence, KV head) with the
// arithmetic of the separate projection (the same values, bit for bit, at the
// same place) and then mark the row block done with the step's epoch
// (project_body's TAG form).  Every other workgroup requests the done-tags of
// the row blocks its queries come from where it would have requested the
// projected queries; once its page loads are issued it checks them, waits
// (sleeps, re-reading the stale tags) until all carry this step's epoch, and
// only then reads the values.  The projection workgroups come first in the
// grid and wait for nothing, so they run and finish whatever the others do;
// the wait is bounded all the same (kTagWaitRounds).  The first of them also
// zeroes the attention's merge counters, as the projection's own launch does.
// The step's epoch is one more than the device word epoch, which the step's
// selection launch then advances: no two launches of a stream share an
// epoch, graph replays included, and a zero-filled workspace starts both at
// zero.
struct DeferArgs {
  const void *k_new, *v_new, *A, *P, *E;  // new tokens and factors (activation type)
  const int32_t *start_pos;               // the new token's position per sequence
  void *zpool, *rpool, *kpool;            // the pools it is written to
  float *new_scores;                      // [batch * n_kv] the new token's score (-inf: none)
  AppendArgs ap;
  int n_append, app_padded;  // batch * n_kv workgroups, padded to a multiple of the XCD count
  const void *q, *Q;         // raw queries and residual factor (activation type)
  uint32_t *qtags;           // done-tags per (sequence, KV head, row block) (null: projected before)
  float *q_proj_out;         // where the projection writes: the launch's q_proj
  const uint32_t *epoch;     // the last step's tag: this launch's is one more
  int n_proj, proj_padded, proj_x;  // projection workgroups (padded as above); row blocks per KV head
  int32_t *counters;         // the attention's merge counters
  int n_counters;
};
constexpr int kTagWaitRounds = 1 << 16;  // rounds of a 1 us sleep and a read (over 0.1 s)

struct ScoreArgs {
  int n_q, n_kv, max_pages, num_phys, page_size, log2_page, cap;
  int pages_per_wg, chunks_per_bg, total, padded;
  PoolGeom geom;  // chunk positions of the latent and residual pages
  DeferArgs df;   // df.n_append = 0: scoring only
};

typedef short route_s4 __attribute__((ext_vector_type(4)));
typedef float route_f4 __attribute__((ext_vector_type(4)));

// MF: the logits on the matrix cores (bf16 and E4M3 pages, groups of 4 or 8
// heads).  v_mfma_f32_4x4x4bf16_1k runs 16 independent 4x4x4 products; in
// each, lane 4 j + i supplies 4 dims of head i's projected query (A) and 4
// dims of its own token (B), and receives its token's logits for the 4 heads
// of the quad -- the one-token-per-lane layout is kept.  The float32
// projected queries enter as two bf16 terms, hi = bf16(q) and lo = bf16(q -
// hi) (about 16 significant bits); every product is exact and the sums are
// float32.  The query operands are staged in LDS once per workgroup.
// Wavefronts per SIMD asked of the compiler: the projection-inside form of a
// narrow 4-head scan (up to 6 chunk loads per lane) carries more scalar state
// than fits eight wavefronts' share of the scalar registers, and is held to the
// eight its plain form runs (its few extra scalars then live in vector-register
// lanes); no request otherwise.
template <int G, int NZ, int NR, bool PROJ>
constexpr int route_waves_per_eu() {
  return PROJ && G == 4 && NZ + NR <= 6 ? 8 : 1;
}
template <typename T, int G, int NZ, int NR, bool STREAM, bool MF, bool PROJ = false>
__global__ __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(route_waves_per_eu<G, NZ, NR, PROJ>())))
void route_scan_kernel(
    const float *__restrict__ q_proj, const T *zpool, const T *rpool,  // (written by compression)
    const int32_t *__restrict__ block_table, const int32_t *__restrict__ seq_lens,
    float *__restrict__ scores, ScoreArgs a) {
  constexpr int CE = Elem<T>::CE;
  constexpr int W = (NZ + NR) * CE;  // r_b + r_q
  constexpr int QG = MF ? G / 4 : 1;  // head quads
  constexpr int NST = W / 4;          // 4-dim steps
  static_assert(!MF || (G % 4 == 0 && sizeof(T) <= 2), "matrix-core logits: bf16/E4M3, G % 4 == 0");
  // [quad][step][head in quad]: {hi 4 x bf16, lo 4 x bf16}
  __shared__ __align__(16) uint4 qf[MF ? QG * NST * 4 : 1];
  using TA = typename std::conditional<sizeof(T) == 1, uint16_t, T>::type;  // activations
  // projection workgroups first, then compression workgroups (proj_padded and
  // app_padded of them, multiples of the XCD count, so the scan's workgroups
  // keep their XCD placement)
  int bid = blockIdx.x;
  static_assert(!PROJ || MF, "the projection inside the launch goes with the matrix-core logits");
  if (PROJ && bid < a.df.proj_padded) {  // (workgroup-uniform)
    if (bid < a.df.n_proj) {
      if (bid == 0)
        for (int i = threadIdx.x; i < a.df.n_counters; i += blockDim.x) a.df.counters[i] = 0;
      const int xblk = bid % a.df.proj_x, rest = bid / a.df.proj_x;
      const uint32_t tag = load_coherent_u32(a.df.epoch) + 1;
      project_body<TA, 256, true>(static_cast<const TA *>(a.df.q), static_cast<const TA *>(a.df.P),
                                  static_cast<const TA *>(a.df.Q), a.df.q_proj_out,
                                  a.n_q, a.n_kv, W - NR * CE, NR * CE, xblk, rest % a.n_kv,
                                  rest / a.n_kv, a.df.qtags + bid, tag);
    }
    return;
  }
  if constexpr (PROJ) bid -= a.df.proj_padded;
  const bool compress = bid < a.df.app_padded;  // (workgroup-uniform)
  if (compress && bid >= a.df.n_append) return;
  int bg, chunk = 0;
  if (compress) {
    bg = bid;  // b * n_kv + g
  } else {
    bid -= a.df.app_padded;
    const int per_xcd = a.padded / kXcds;
    const int work = (bid % kXcds) * per_xcd + bid / kXcds;
    if (work >= a.total) return;
    bg = work / a.chunks_per_bg;
    chunk = work - bg * a.chunks_per_bg;
  }
  const int b = bg / a.n_kv, g = bg - b * a.n_kv;
  if (compress) {
    append_body<TA, T, true>(
        static_cast<const TA *>(a.df.k_new), static_cast<const TA *>(a.df.v_new), a.df.start_pos,
        static_cast<const TA *>(a.df.A), static_cast<const TA *>(a.df.P),
        static_cast<const TA *>(a.df.E), static_cast<T *>(a.df.zpool),
        static_cast<T *>(a.df.rpool), static_cast<T *>(a.df.kpool), block_table, a.df.ap, g, b);
    __syncthreads();  // the token's codes are stored, and visible to this workgroup
  }

  const int p_begin = chunk * a.pages_per_wg;
  const int p_end = min(a.max_pages, p_begin + a.pages_per_wg);
  const int ppi = kWave >> a.log2_page;  // pages per wave step
  const int n_steps = (p_end - p_begin + ppi - 1) / ppi;

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;
  const int slot = lane & (a.page_size - 1);
  const float *qp = q_proj + ((int64_t)b * a.n_q + (int64_t)g * G) * W;
  const int32_t *bt = block_table + (int64_t)b * a.max_pages;
  float *out = scores + (int64_t)bg * a.max_pages;
  const int64_t zhead = (int64_t)g * a.num_phys;
  const int64_t page_z_bytes = (int64_t)a.geom.z_page_chunks * a.page_size * 16;
  const int64_t page_r_bytes = (int64_t)a.geom.r_page_chunks * a.page_size * 16;

  // The lane's block-table entry (every entry of the row is in bounds), the
  // sequence length and the projected queries are requested together; the
  // page loads are issued as soon as they arrive, and the queries are staged
  // in LDS while the pages are in flight.  A step then costs two dependent
  // round trips, not the three of staging the queries first.  (Measured:
  // qwen32b-shaped scoring 48.2 -> 46.8 us, llama8b-shaped 59.6 -> 59.1 us;
  // converting the queries before issuing the page loads saves the 8-head
  // kernel 8 registers, five instead of four wavefronts per SIMD, but measured
  // 48.0 us.)
  const int step = wave;
  int p = p_begin + step * ppi + (lane >> a.log2_page);
  bool in_range = step < n_steps && p < p_end;
  int slot_t = slot;  // the lane's token slot in its page
  const int newpos = a.df.n_append > 0 ? a.df.start_pos[b] : -1;
  if (compress) {  // one token: the new one, in thread 0
    const bool pos_ok = newpos >= 0 && newpos < a.cap;
    p = pos_ok ? newpos >> a.log2_page : 0;
    slot_t = newpos & (a.page_size - 1);
    in_range = pos_ok && threadIdx.x == 0;
  }
  const int phys = in_range ? bt[p] : -1;
  const int L = clamp_len(seq_lens[b], a.cap);
  const int NP = (L + a.page_size - 1) >> a.log2_page;
  constexpr int QN = MF ? QG * NST * 4 : 1;  // staged query entries
  constexpr int QI = (QN + 255) / 256;       // per thread (256 threads)
  float4 qv_in[QI];
  uint32_t qt[PROJ ? QI : 1];  // done-tags of the entries' row blocks (projection in this launch)
  constexpr bool tagged = PROJ;
  const uint32_t *tags = tagged ? a.df.qtags + (int64_t)bg * a.df.proj_x : nullptr;
  auto q_index = [&](int i) {  // staged entry i: 4 dims of one head's projected query
    const int hq = i & 3, st = (i >> 2) % NST, qd = i / (NST * 4);
    return (qd * 4 + hq) * W + st * 4;
  };
  auto q_block = [&](int i) { return ((i >> 2) % NST) / 4; };  // its row block (16 rows)
  uint32_t expect = 0;  // this launch's epoch
  if constexpr (tagged) expect = load_coherent_u32(a.df.epoch) + 1;
  if constexpr (MF) {
#pragma unroll
    for (int u = 0; u < QI; ++u) {
      const int i = u * 256 + threadIdx.x;
      if constexpr (tagged)
        qt[u] = i < QN ? load_coherent_u32(tags + q_block(i)) : 0u;
      else
        qv_in[u] = i < QN ? *reinterpret_cast<const float4 *>(qp + q_index(i))
                          : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  const int tok = p * a.page_size + slot_t;
  // (the scan leaves the new token to the compression workgroups)
  const bool valid = in_range && p < NP && tok < L && phys >= 0 && phys < a.num_phys &&
                     (compress || tok != newpos);
  // matrix-core path: every lane joins the matrix instructions; one without a
  // valid token scores zeros and is masked
  uint4 cz[NZ > 0 ? NZ : 1], cr[NR > 0 ? NR : 1];  // (a width may be 0)
  if constexpr (MF) {
#pragma unroll
    for (int c = 0; c < NZ; ++c) cz[c] = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int c = 0; c < NR; ++c) cr[c] = make_uint4(0u, 0u, 0u, 0u);
    if (valid) {
      const int64_t zoff = (zhead + phys) * page_z_bytes + (int64_t)slot_t * 16;
      const int64_t roff =
          (zhead + phys) * page_r_bytes + ((int64_t)a.geom.r_first * a.page_size + slot_t) * 16;
#pragma unroll
      for (int c = 0; c < NZ; ++c)
        cz[c] = load_page_chunk<STREAM>(zpool, zoff + (int64_t)c * a.page_size * 16);
#pragma unroll
      for (int c = 0; c < NR; ++c)
        cr[c] = load_page_chunk<STREAM>(rpool, roff + (int64_t)c * a.page_size * 16);
    }
    if constexpr (tagged) {  // this step's projected queries: their row blocks done, then the values
      auto stale = [&]() {
        bool any = false;
#pragma unroll
        for (int u = 0; u < QI; ++u) any |= u * 256 + (int)threadIdx.x < QN && qt[u] != expect;
        return any;
      };
      if (__syncthreads_or(stale())) {
        for (int round = 0; round < kTagWaitRounds; ++round) {
          __builtin_amdgcn_s_sleep(40);
#pragma unroll
          for (int u = 0; u < QI; ++u) {
            const int i = u * 256 + threadIdx.x;
            if (i < QN && qt[u] != expect) qt[u] = load_coherent_u32(tags + q_block(i));
          }
          if (!__syncthreads_or(stale())) break;
        }
      }
#pragma unroll
      for (int u = 0; u < QI; ++u) {
        const int i = u * 256 + threadIdx.x;
        const float *src = qp + (i < QN ? q_index(i) : 0);
        qv_in[u] = make_float4(load_coherent(src), load_coherent(src + 1), load_coherent(src + 2),
                               load_coherent(src + 3));
      }
    }
    // the queries (arrived with the block-table entry) into LDS while the
    // pages are in flight
#pragma unroll
    for (int u = 0; u < QI; ++u) {
      const int i = u * 256 + threadIdx.x;
      const float4 v = qv_in[u];
      const uint32_t h01 = f32x2_to_bf16x2(v.x, v.y), h23 = f32x2_to_bf16x2(v.z, v.w);
      const uint32_t l01 = f32x2_to_bf16x2(v.x - __uint_as_float(h01 << 16),
                                           v.y - __uint_as_float(h01 & 0xffff0000u));
      const uint32_t l23 = f32x2_to_bf16x2(v.z - __uint_as_float(h23 << 16),
                                           v.w - __uint_as_float(h23 & 0xffff0000u));
      if (i < QN) qf[i] = make_uint4(h01, h23, l01, l23);
    }
    __syncthreads();
  }

  if (compress ? wave == 0 : step < n_steps) {
    float best = -INFINITY;
    if constexpr (MF) {
      route_f4 sc[QG];
#pragma unroll
      for (int qd = 0; qd < QG; ++qd) sc[qd] = route_f4{0.f, 0.f, 0.f, 0.f};
      const int hq = lane & 3;
      // 8 bf16 dims (one uint4) starting at 4-dim step st0
      auto mma8 = [&](const uint4 &k8, int st0) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const route_s4 kv = __builtin_bit_cast(
              route_s4, hh ? make_uint2(k8.z, k8.w) : make_uint2(k8.x, k8.y));
#pragma unroll
          for (int qd = 0; qd < QG; ++qd) {
            const uint4 qv = qf[(qd * NST + st0 + hh) * 4 + hq];
            sc[qd] = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(
                __builtin_bit_cast(route_s4, make_uint2(qv.x, qv.y)), kv, sc[qd], 0, 0, 0);
            sc[qd] = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(
                __builtin_bit_cast(route_s4, make_uint2(qv.z, qv.w)), kv, sc[qd], 0, 0, 0);
          }
        }
      };
      auto mma_chunk = [&](const uint4 &ch, int dim0) {
        if constexpr (sizeof(T) == 1) {  // 16 E4M3 codes: widened to bf16 (exact)
          mma8(fp8x8_to_bf16x8(ch.x, ch.y), dim0 / 4);
          mma8(fp8x8_to_bf16x8(ch.z, ch.w), dim0 / 4 + 2);
        } else {
          mma8(ch, dim0 / 4);
        }
      };
#pragma unroll
      for (int c = 0; c < NZ; ++c) mma_chunk(cz[c], c * CE);
#pragma unroll
      for (int c = 0; c < NR; ++c) mma_chunk(cr[c], NZ * CE + c * CE);
      if (valid) {
#pragma unroll
        for (int h = 0; h < G; ++h) best = fmaxf(best, sc[h / 4][h % 4]);
      }
    } else if (valid) {
      const int64_t zoff = (zhead + phys) * page_z_bytes + (int64_t)slot_t * 16;
      const int64_t roff =
          (zhead + phys) * page_r_bytes + ((int64_t)a.geom.r_first * a.page_size + slot_t) * 16;
#pragma unroll
      for (int c = 0; c < NZ; ++c) {
        const int64_t o = zoff + (int64_t)c * a.page_size * 16;
        cz[c] = load_page_chunk<STREAM>(zpool, o);
      }
#pragma unroll
      for (int c = 0; c < NR; ++c) {
        const int64_t o = roff + (int64_t)c * a.page_size * 16;
        cr[c] = load_page_chunk<STREAM>(rpool, o);
      }
      float acc[G];
#pragma unroll
      for (int h = 0; h < G; ++h) acc[h] = 0.f;
#pragma unroll
      for (int c = 0; c < NZ; ++c) {
        float x[CE];
        unpack_chunk<T>(cz[c], x);
#pragma unroll
        for (int e = 0; e < CE; ++e)
#pragma unroll
          for (int h = 0; h < G; ++h) acc[h] = fmaf(qp[h * W + c * CE + e], x[e], acc[h]);
      }
#pragma unroll
      for (int c = 0; c < NR; ++c) {
        float x[CE];
        unpack_chunk<T>(cr[c], x);
#pragma unroll
        for (int e = 0; e < CE; ++e)
#pragma unroll
          for (int h = 0; h < G; ++h)
            acc[h] = fmaf(qp[h * W + NZ * CE + c * CE + e], x[e], acc[h]);
      }
#pragma unroll
      for (int h = 0; h < G; ++h) best = fmaxf(best, acc[h]);
    }
    if (compress) {  // thread 0's token alone
      if (threadIdx.x == 0) a.df.new_scores[bg] = best;  // (-inf when it does not count)
      return;
    }
    best = group_max(best, a.page_size);
    if (in_range && slot == 0) out[p] = (p < NP) ? best : -INFINITY;
  }
}

// ---------------------------------------------------------------------------
// (a2) page scores with rotary position embedding.  The cached codes are
// pre-RoPE, so the projected-query shortcut does not apply: the predicted Key
// of every token is formed, k_hat = [z[:r_b], r] [P; Q] (dims x 128), rotated
// to the token's position and dotted with the group's queries.
//
// A wavefront takes 64-token steps (a page-aligned run of pages), each as
// four 16-token tiles.  For a tile, one v_mfma_f32_16x16x32_bf16 per 32 codes
// and 16 Key dims forms the predicted Keys transposed: A = [P; Q]^T (lane l:
// dim l % 16 of the Key tile, codes 8 (l / 16) .. + 7 of the k step), B = the
// tokens' codes (lane l: token l % 16, the same 8 codes -- one 8-element run
// of a page chunk, widened from E4M3 when the cache is FP8).  The result puts
// dims 16 nt + 4 (l / 16) + 0..3 of token l % 16 in lane l for Key tile nt, so
// the rotate-half pair (d, d + 64) -- tiles nt and nt + 4 -- is lane-local and
// a lane holds 32 dims of one token.  Each lane rotates its 16 pairs in float32
// and splits the rotated values into bf16 hi + lo terms (about 16 significant
// bits); the dot products with the group's bf16 queries then run on the same
// matrix instruction (A = the queries, heads as rows; B = the rotated Key; k
// slots map to the lane's dims in the same order on both sides), hi and lo
// accumulating into one float32 tile that holds the tile's logits.
//
// Angles: the token at tile position i sits at t = t0 + i (t0 uniform over
// the wavefront).  Every tile, lane l takes one exact sine and cosine of
// t0 w_l (turns reduced in double precision), shared through LDS; each lane
// combines them with the fixed rotation by i w_d of its own dims (taken once,
// exactly) -- four products per pair.
//
// [P; Q]^T is staged in LDS once per workgroup and, for 32 codes, held in
// registers by every wave.  A workgroup covers pages_per_wg pages, i.e.
// several steps per wave, so the staging is shared by many tokens, and each
// wave loads the codes of its next step while it computes the current one.
// grid: (batch x n_kv x chunks), XCD-major; 256 threads; q: the raw
// (rotated) queries.
// ---------------------------------------------------------------------------
// wavefronts per SIMD: two for routing widths up to 96 codes, one for the
// wider ones (whole register file)
#ifndef BKV_ROPE_WAVES_PER_EU
#define BKV_ROPE_WAVES_PER_EU 2
#endif
template <typename C, int G, int NZ, int NR>
__global__ __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu((NZ + NR) * (16 / sizeof(C)) <= 96 ? BKV_ROPE_WAVES_PER_EU : 1)))
void route_rope_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ P, const uint16_t *__restrict__ Q,
    const float *__restrict__ inv_freq, const C *__restrict__ zpool, const C *__restrict__ rpool,
    const int32_t *__restrict__ block_table, const int32_t *__restrict__ seq_lens,
    float *__restrict__ scores, ScoreArgs a) {
  constexpr int CE = Elem<C>::CE;        // cache elements per 16-byte chunk
  constexpr int RB = NZ * CE, RQ = NR * CE, W = RB + RQ;
  constexpr int KS = (W + 31) / 32;      // 32-code k steps
  constexpr int KP = KS * 32;
  constexpr int FS = KP + 8;             // LDS row stride of [P;Q]^T (16-byte pad)
  // factor fragments held in registers for one k step (32 codes); wider
  // routing reads them from LDS each tile, which leaves room for two
  // wavefronts per SIMD up to 96 codes (measured 168 -> 142 us at 96)
  constexpr bool kRegB = KS <= 1;
  typedef __bf16 rb16x8 __attribute__((ext_vector_type(8)));
  typedef float rf4 __attribute__((ext_vector_type(4)));
  __shared__ __align__(16) uint16_t ft[kHeadDim * FS];   // [dim][code]
  __shared__ float qs[G][kHeadDim];
  __shared__ float tok_score[4][kWave];
  __shared__ __align__(16) float ang[4][2][kHeadDim / 2];  // per wave: cos, sin of t0 w_d
  static_assert(G <= 16, "heads are the rows of one matrix tile");

  const int work = xcd_work_index(a.padded);
  if (work >= a.total) return;
  const int bg = work / a.chunks_per_bg;
  const int chunk = work - bg * a.chunks_per_bg;
  const int b = bg / a.n_kv, g = bg - b * a.n_kv;
  const int L = clamp_len(seq_lens[b], a.cap);
  const int NP = (L + a.page_size - 1) >> a.log2_page;
  const int p_begin = chunk * a.pages_per_wg;
  const int p_end = min(a.max_pages, p_begin + a.pages_per_wg);
  const int ppi = kWave >> a.log2_page;  // pages per 64-token step
  const int n_steps = (p_end - p_begin + ppi - 1) / ppi;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  const int slot = lane & (a.page_size - 1);
  const int64_t zhead = (int64_t)g * a.num_phys;
  const int64_t page_z_bytes = (int64_t)a.geom.z_page_chunks * a.page_size * 16;
  const int64_t page_r_bytes = (int64_t)a.geom.r_page_chunks * a.page_size * 16;
  float *out = scores + (int64_t)bg * a.max_pages;

  // ---- stage [P_g; Q_g]^T (bf16, zero past W) and the queries ----
  for (int o = threadIdx.x; o < kHeadDim * KP; o += blockDim.x) {
    const int k = o / kHeadDim, n = o % kHeadDim;  // consecutive threads: consecutive dims
    uint16_t v = 0;
    if (k < RB) v = P[((int64_t)g * RB + k) * kHeadDim + n];
    else if (k < W) v = Q[((int64_t)g * RQ + (k - RB)) * kHeadDim + n];
    ft[n * FS + k] = v;
  }
  for (int o = threadIdx.x; o < G * kHeadDim; o += blockDim.x)
    qs[o / kHeadDim][o % kHeadDim] = bf16_to_f32(q[((int64_t)b * a.n_q + (int64_t)g * G) * kHeadDim + o]);
  __syncthreads();
  if (wave >= n_steps) return;  // (no barrier below)

  const int li = lane & 15, lg = lane >> 4;
  // k slot j of dot step s <-> Key dim 16 (2 s + j / 4) + 4 lg + j % 4 (the
  // lane's rotated values of Key tiles 2 s and 2 s + 1); the query operand:
  // head li's values at those dims (zero rows past the group)
  uint4 qop[4];
#pragma unroll
  for (int st = 0; st < 4; ++st) {
    float x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      x[j] = li < G ? qs[li < G ? li : 0][16 * (2 * st + j / 4) + 4 * lg + j % 4] : 0.f;
    qop[st] = make_uint4(f32x2_to_bf16x2(x[0], x[1]), f32x2_to_bf16x2(x[2], x[3]),
                         f32x2_to_bf16x2(x[4], x[5]), f32x2_to_bf16x2(x[6], x[7]));
  }
  // this lane's pairs (d, d + 64), d = 16 nt + 4 lg + r: the rotation by li w_d
  // (its token's offset in a tile); and frequency l in turns per position
  float cl[4][4], sl[4][4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt)
#pragma unroll
    for (int r = 0; r < 4; ++r) rope_sincos(li, inv_freq[16 * nt + 4 * lg + r], sl[nt][r], cl[nt][r]);
  const double wt = (double)inv_freq[lane] * 0.15915494309189535;  // 1 / (2 pi); lane < 64 pairs
  uint4 bf[kRegB ? 8 : 1][kRegB ? KS : 1];
  if constexpr (kRegB) {
#pragma unroll
    for (int nt = 0; nt < 8; ++nt)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        bf[nt][ks] = *reinterpret_cast<const uint4 *>(&ft[(nt * 16 + li) * FS + ks * 32 + lg * 8]);
  }

  // The codes of step st for the four tiles.  Every lane loads (tokens past
  // the sequence read page 0 of the pool); tmask gets bit mt when the lane's
  // token of tile mt is valid, and the codes of the others are zeroed at use,
  // so no load waits on a branch.  Returns whether the lane's own token of the
  // step is valid.
  auto load_step = [&](int st, uint4 (&af)[4][KS], uint32_t &tmask) -> bool {
    const int p = p_begin + st * ppi + (lane >> a.log2_page);
    int phys = -1;
    if (p < p_end && p < NP) phys = block_table[(int64_t)b * a.max_pages + p];
    const bool valid = p < p_end && p < NP && p * a.page_size + slot < L && phys >= 0 &&
                       phys < a.num_phys;
    tmask = 0;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const int tok = mt * 16 + li;
      const int tv = __shfl((int)valid, tok);
      const int ph0 = __shfl(phys, tok);
      const int ph = tv ? ph0 : 0;
      tmask |= (uint32_t)(tv != 0) << mt;
      const int tslot = tok & (a.page_size - 1);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int run = (ks * 4 + lg) * 8;            // this lane's 8-code run
        const int code0 = run < W ? run : 0;          // (runs past W: zeroed at use)
        const bool in_z = code0 < RB;
        const int cc = in_z ? code0 / CE : (code0 - RB) / CE;  // chunk of its pool
        const int64_t off = in_z
            ? (zhead + ph) * page_z_bytes + ((int64_t)cc * a.page_size + tslot) * 16
            : (zhead + ph) * page_r_bytes + ((int64_t)(a.geom.r_first + cc) * a.page_size + tslot) * 16;
        const char *base = reinterpret_cast<const char *>(in_z ? (const void *)zpool : (const void *)rpool);
        if constexpr (sizeof(C) == 1) {
          const uint2 w = *reinterpret_cast<const uint2 *>(base + off + ((code0 % CE) / 8) * 8);
          af[mt][ks] = make_uint4(w.x, w.y, 0u, 0u);  // widened at use
        } else {
          af[mt][ks] = *reinterpret_cast<const uint4 *>(base + off);
        }
      }
    }
    return valid;
  };

  auto compute_step = [&](int st, const uint4 (&af)[4][KS], uint32_t tmask, bool valid) {
    const int p0 = p_begin + st * ppi;
    const int pos0 = p0 * a.page_size;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      // the tile's base angles t0 w_l, exact, one frequency per lane
      {
        float sn, cs;
        rope_sincos_turns((double)(pos0 + mt * 16), wt, sn, cs);
        ang[wave][0][lane] = cs;
        ang[wave][1][lane] = sn;
      }
      rb16x8 av[KS];
      const bool tv = (tmask >> mt) & 1u;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        uint4 v = af[mt][ks];
        if constexpr (sizeof(C) == 1) v = fp8x8_to_bf16x8(v.x, v.y);
        if (!tv || (ks * 4 + lg) * 8 >= W) v = make_uint4(0u, 0u, 0u, 0u);
        av[ks] = __builtin_bit_cast(rb16x8, v);
      }
      // predicted Keys of the tile, transposed: dims 16 nt + 4 lg + r of token li
      rf4 kh[8];
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) {
        kh[nt] = rf4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          uint4 bv;
          if constexpr (kRegB) bv = bf[nt][ks];
          else bv = *reinterpret_cast<const uint4 *>(&ft[(nt * 16 + li) * FS + ks * 32 + lg * 8]);
          kh[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(rb16x8, bv), av[ks],
                                                           kh[nt], 0, 0, 0);
        }
      }
      wave_lds_sync();
      // rotate each pair to the token's position: angle t0 w_d + li w_d
      float kr[8][4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const float4 c0 = *reinterpret_cast<const float4 *>(&ang[wave][0][16 * nt + 4 * lg]);
        const float4 s0 = *reinterpret_cast<const float4 *>(&ang[wave][1][16 * nt + 4 * lg]);
        const float ct[4] = {c0.x, c0.y, c0.z, c0.w}, stt[4] = {s0.x, s0.y, s0.z, s0.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float cs = ct[r] * cl[nt][r] - stt[r] * sl[nt][r];
          const float sn = stt[r] * cl[nt][r] + ct[r] * sl[nt][r];
          const float x = kh[nt][r], y = kh[nt + 4][r];
          kr[nt][r] = x * cs - y * sn;
          kr[nt + 4][r] = x * sn + y * cs;
        }
      }
      // logits of the tile: heads 4 lg + r of token li, hi and lo terms
      rf4 lgh = rf4{0.f, 0.f, 0.f, 0.f}, lgl = lgh;  // hi and lo terms: two independent chains
#pragma unroll
      for (int ds = 0; ds < 4; ++ds) {
        float x[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = kr[2 * ds + j / 4][j % 4];
        uint32_t h[4], l[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          h[i] = f32x2_to_bf16x2(x[2 * i], x[2 * i + 1]);
          l[i] = f32x2_to_bf16x2(x[2 * i] - __uint_as_float(h[i] << 16),
                                 x[2 * i + 1] - __uint_as_float(h[i] & 0xffff0000u));
        }
        const rb16x8 qv = __builtin_bit_cast(rb16x8, qop[ds]);
        lgh = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            qv, __builtin_bit_cast(rb16x8, make_uint4(h[0], h[1], h[2], h[3])), lgh, 0, 0, 0);
        lgl = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            qv, __builtin_bit_cast(rb16x8, make_uint4(l[0], l[1], l[2], l[3])), lgl, 0, 0, 0);
      }
      const rf4 lg4 = lgh + lgl;
      // maximum over the group's heads (rows 4 lg + r < G)
      float best = -INFINITY;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (4 * lg + r < G) best = fmaxf(best, lg4[r]);
      if constexpr (G > 4) best = fmaxf(best, __shfl_xor(best, 16));
      if (lg == 0) tok_score[wave][mt * 16 + li] = best;
    }
    wave_lds_sync();
    float best = valid ? tok_score[wave][lane] : -INFINITY;
    best = group_max(best, a.page_size);
    const int p = p0 + (lane >> a.log2_page);
    if (p < p_end && slot == 0) out[p] = (p < NP) ? best : -INFINITY;
  };

  // Steps wave, wave + 4, ... of the workgroup's range; steps wholly past the
  // sequence write -inf without loads.  Two code buffers: the next step's
  // loads are issued before the current step's compute.
  const int first_dead = (NP - p_begin + ppi - 1) / ppi;  // first step with no valid page
  const int n_live = max(0, min(n_steps, first_dead));
  int dead = wave;  // this wave's first step at or past n_live
  if (dead < n_live) dead += ((n_live - 1 - dead) / 4 + 1) * 4;
  for (int st = dead; st < n_steps; st += 4) {
    const int p = p_begin + st * ppi + (lane >> a.log2_page);
    if (p < p_end && slot == 0) out[p] = -INFINITY;
  }
  if (wave >= n_live) return;
  uint4 fa[4][KS], fb[4][KS];
  uint32_t ma = 0, mb = 0;
  bool va = load_step(wave, fa, ma), vb = false;
  for (int st = wave;; st += 8) {
    const bool more1 = st + 4 < n_live;
    if (more1) vb = load_step(st + 4, fb, mb);
    compute_step(st, fa, ma, va);
    if (!more1) break;
    const bool more2 = st + 8 < n_live;
    if (more2) va = load_step(st + 8, fa, ma);
    compute_step(st + 4, fb, mb, vb);
    if (!more2) break;
  }
}

template <typename T>
hipError_t project_t(const basiskv_dims &d, const void *q, const void *P, const void *Q,
                     float *q_proj, hipStream_t s) {
  const int row_blocks = (d.r_b + d.r_q + 7) / 8;  // 8 rows per 128-thread workgroup
  hipLaunchKernelGGL(project_queries_kernel<T>, dim3(row_blocks, d.n_kv_heads, d.batch),
                     dim3(128), 0, s,
                     (const T *)q, (const T *)P, (const T *)Q, q_proj, d.n_q_heads, d.n_kv_heads,
                     d.r_b, d.r_q);
  return hipGetLastError();
}

#ifndef BKV_STREAM_MIN_CHUNKS
#define BKV_STREAM_MIN_CHUNKS 8
#endif
constexpr int kStreamMinChunks = BKV_STREAM_MIN_CHUNKS;  // chunk loads per lane the non-temporal form needs

struct ScoreVariant {
  int dtype, G, rb, rq;
  const void *fn, *fn_nt;  // ordinary loads; non-temporal loads (null: not built)
  // matrix-core logits with the projection inside (null: not built): ordinary
  // and non-temporal loads
  const void *fn_proj, *fn_nt_proj;
};

#ifndef BKV_ROUTE_MFMA_MIN_G
#define BKV_ROUTE_MFMA_MIN_G 4
#endif
// groups this wide (of 2-byte or 1-byte pages) take the matrix-core logits
template <typename T, int G>
constexpr bool route_mfma() {
  return sizeof(T) <= 2 && G % 4 == 0 && G >= BKV_ROUTE_MFMA_MIN_G;
}

// the decode step's scan with the query projection inside: built where the
// scan takes the matrix-core logits, with the loads the plain scan uses
template <typename T, int G, int NZ, int NR, bool STREAM>
const void *score_proj_kernel() {
  if constexpr (route_mfma<T, G>() && (!STREAM || NZ + NR >= kStreamMinChunks))
    return reinterpret_cast<const void *>(&route_scan_kernel<T, G, NZ, NR, STREAM, true, true>);
  else
    return nullptr;
}

#define BKV_SCORE(T, DT, G, RB, RQ)                                                                  \
  {DT, G, RB, RQ,                                                                                     \
   reinterpret_cast<const void *>(&route_scan_kernel<T, G, (RB) / Elem<T>::CE, (RQ) / Elem<T>::CE,   \
                                                     false, route_mfma<T, G>()>),                     \
   ((RB) + (RQ)) / Elem<T>::CE >= kStreamMinChunks                                                    \
       ? reinterpret_cast<const void *>(                                                              \
             &route_scan_kernel<T, G, (RB) / Elem<T>::CE, (RQ) / Elem<T>::CE,                         \
                                (((RB) + (RQ)) / Elem<T>::CE >= kStreamMinChunks),                    \
                                route_mfma<T, G>()>)                                                  \
       : nullptr,                                                                                     \
   score_proj_kernel<T, G, (RB) / Elem<T>::CE, (RQ) / Elem<T>::CE, false>(),                         \
   score_proj_kernel<T, G, (RB) / Elem<T>::CE, (RQ) / Elem<T>::CE, true>()}

#define BKV_SCORE_G(T, DT, RB, RQ) \
  BKV_SCORE(T, DT, 1, RB, RQ), BKV_SCORE(T, DT, 2, RB, RQ), BKV_SCORE(T, DT, 4, RB, RQ), \
      BKV_SCORE(T, DT, 8, RB, RQ)

// (the kernel's element type is the cache's: E4M3 codes for BASISKV_BF16_FP8_E4M3)
static const ScoreVariant kScoreVariants[] = {
    BKV_SCORE_G(uint16_t, BASISKV_BF16, 64, 32), BKV_SCORE_G(uint16_t, BASISKV_BF16, 96, 48),
    BKV_SCORE_G(uint16_t, BASISKV_BF16, 16, 16), BKV_SCORE_G(uint16_t, BASISKV_BF16, 32, 32),
    BKV_SCORE_G(uint16_t, BASISKV_BF16, 32, 16),
    BKV_SCORE_G(uint16_t, BASISKV_BF16, 128, 32), BKV_SCORE_G(float, BASISKV_F32, 64, 32),
    BKV_SCORE_G(float, BASISKV_F32, 16, 16), BKV_SCORE_G(float, BASISKV_F32, 32, 16),
    BKV_SCORE_G(uint8_t, BASISKV_BF16_FP8_E4M3, 64, 32),
    BKV_SCORE_G(uint8_t, BASISKV_BF16_FP8_E4M3, 96, 48),
    BKV_SCORE_G(uint8_t, BASISKV_BF16_FP8_E4M3, 16, 16),
    BKV_SCORE_G(uint8_t, BASISKV_BF16_FP8_E4M3, 32, 16),
    // single-source routers (appendix Table 9: B16, R16, R32)
    BKV_SCORE_G(uint16_t, BASISKV_BF16, 16, 0), BKV_SCORE_G(uint16_t, BASISKV_BF16, 0, 16),
    BKV_SCORE_G(uint16_t, BASISKV_BF16, 0, 32), BKV_SCORE_G(float, BASISKV_F32, 16, 0),
    BKV_SCORE_G(float, BASISKV_F32, 0, 16), BKV_SCORE_G(float, BASISKV_F32, 0, 32),
    BKV_SCORE_G(uint8_t, BASISKV_BF16_FP8_E4M3, 16, 0),
    BKV_SCORE_G(uint8_t, BASISKV_BF16_FP8_E4M3, 0, 16),
    BKV_SCORE_G(uint8_t, BASISKV_BF16_FP8_E4M3, 0, 32),
};

struct ScoreRopeVariant {
  int dtype, G, rb, rq;
  const void *fn;
};
#define BKV_SCORE_ROPE(C, DT, G, RB, RQ) \
  {DT, G, RB, RQ,                         \
   reinterpret_cast<const void *>(&route_rope_kernel<C, G, (RB) / Elem<C>::CE, (RQ) / Elem<C>::CE>)}
static const ScoreRopeVariant kScoreRopeVariants[] = {
    BKV_SCORE_ROPE(uint16_t, BASISKV_BF16, 4, 16, 16), BKV_SCORE_ROPE(uint16_t, BASISKV_BF16, 8, 16, 16),
    BKV_SCORE_ROPE(uint16_t, BASISKV_BF16, 4, 64, 32), BKV_SCORE_ROPE(uint16_t, BASISKV_BF16, 8, 64, 32),
    BKV_SCORE_ROPE(uint16_t, BASISKV_BF16, 4, 96, 48), BKV_SCORE_ROPE(uint16_t, BASISKV_BF16, 8, 96, 48),
    BKV_SCORE_ROPE(uint8_t, BASISKV_BF16_FP8_E4M3, 4, 16, 16),
    BKV_SCORE_ROPE(uint8_t, BASISKV_BF16_FP8_E4M3, 8, 16, 16),
    BKV_SCORE_ROPE(uint8_t, BASISKV_BF16_FP8_E4M3, 4, 64, 32),
    BKV_SCORE_ROPE(uint8_t, BASISKV_BF16_FP8_E4M3, 8, 64, 32),
    BKV_SCORE_ROPE(uint8_t, BASISKV_BF16_FP8_E4M3, 4, 96, 48),
    BKV_SCORE_ROPE(uint8_t, BASISKV_BF16_FP8_E4M3, 8, 96, 48),
};

}  // namespace bkv

namespace bkv_host {
using namespace bkv;

hipError_t launch_project(const basiskv_dims &d, const void *q, const void *P, const void *Q,
                          float *q_proj, hipStream_t s) {
  return act_bf16(d) ? project_t<uint16_t>(d, q, P, Q, q_proj, s)
                     : project_t<float>(d, q, P, Q, q_proj, s);
}

static int ilog2(int x) {
  int l = 0;
  while ((1 << l) < x) ++l;
  return l;
}

static const void *find_score(const basiskv_dims &d) {
  const int G = d.n_q_heads / d.n_kv_heads;
  for (const auto &v : kScoreVariants)
    if (v.dtype == d.dtype && v.G == G && v.rb == d.r_b && v.rq == d.r_q)
      return v.fn_nt && d.page_size >= 8 ? v.fn_nt : v.fn;  // whole 128-byte lines per load
  return nullptr;
}

bool score_supported(const basiskv_dims &d) { return find_score(d) != nullptr; }

static const void *find_score_proj(const basiskv_dims &d) {
  const int G = d.n_q_heads / d.n_kv_heads;
  for (const auto &v : kScoreVariants)
    if (v.dtype == d.dtype && v.G == G && v.rb == d.r_b && v.rq == d.r_q)
      return v.fn_nt && d.page_size >= 8 ? v.fn_nt_proj : v.fn_proj;  // as find_score
  return nullptr;
}

static const void *find_score_rope(const basiskv_dims &d) {
  const int G = d.n_q_heads / d.n_kv_heads;
  for (const auto &v : kScoreRopeVariants)
    if (v.dtype == d.dtype && v.G == G && v.rb == d.r_b && v.rq == d.r_q) return v.fn;
  return nullptr;
}

bool score_rope_supported(const basiskv_dims &d) { return find_score_rope(d) != nullptr; }

// Page scores with RoPE from the raw queries and the routing factors.
#ifndef BKV_ROPE_WORKGROUPS
#define BKV_ROPE_WORKGROUPS 512
#endif
constexpr int kRopeWorkgroups = BKV_ROPE_WORKGROUPS;
constexpr int kRopeMaxStepsPerWave = 32;

hipError_t launch_score_rope(const basiskv_dims &d, const void *q, const void *P, const void *Q,
                             const basiskv_cache &c, float *scores, hipStream_t s,
                             bool *unsupported) {
  const void *fn = find_score_rope(d);
  if (!fn) {
    *unsupported = true;
    return hipSuccess;
  }
  *unsupported = false;
  ScoreArgs a{};
  a.n_q = d.n_q_heads;
  a.n_kv = d.n_kv_heads;
  a.max_pages = d.max_pages_per_seq;
  a.num_phys = d.num_phys_pages;
  a.page_size = d.page_size;
  a.log2_page = ilog2(d.page_size);
  a.geom = pool_geom(d);
  a.cap = d.max_pages_per_seq * d.page_size;
  // steps of 64 tokens per wave: enough workgroups to fill the chip
  // (kRopeWorkgroups), as few as that allows, so the factor staging of a
  // workgroup serves many tokens
  const int ppi = 64 / d.page_size;
  const int64_t steps = (int64_t)d.batch * d.n_kv_heads * ((d.max_pages_per_seq + ppi - 1) / ppi);
  const int spw = (int)std::max<int64_t>(1, std::min<int64_t>(kRopeMaxStepsPerWave,
                                                               steps / (4 * kRopeWorkgroups)));
  a.pages_per_wg = ppi * 4 * spw;
  a.chunks_per_bg = (d.max_pages_per_seq + a.pages_per_wg - 1) / a.pages_per_wg;
  a.total = d.batch * d.n_kv_heads * a.chunks_per_bg;
  a.padded = (a.total + kXcds - 1) / kXcds * kXcds;
  void *rpool = residual_pool(d, c);
  const float *w = c.rope_inv_freq;
  void *args[] = {(void *)&q,         (void *)&P,           (void *)&Q,
                  (void *)&w,         (void *)&c.z_pages,   (void *)&rpool,
                  (void *)&c.block_table, (void *)&c.seq_lens, (void *)&scores, (void *)&a};
  return hipLaunchKernel(fn, dim3(a.padded), dim3(256), args, 0, s);
}

hipError_t launch_score(const basiskv_dims &d, const float *q_proj, const basiskv_cache &c,
                        float *scores, hipStream_t s, bool *unsupported, const StepTokens *step) {
  const void *fn = step && step->qtags ? find_score_proj(d) : find_score(d);
  if (!fn) {
    *unsupported = true;
    return hipSuccess;
  }
  *unsupported = false;
  ScoreArgs a{};
  if (step && step->qtags) {  // the query projection in this launch too
    a.df.q = step->q;
    a.df.Q = step->Q;
    a.df.P = step->P;
    a.df.qtags = step->qtags;
    a.df.q_proj_out = const_cast<float *>(q_proj);  // (the caller's scratch)
    a.df.epoch = step->epoch;
    a.df.proj_x = (d.r_b + d.r_q + 15) / 16;  // 16 rows per 256-thread workgroup
    a.df.n_proj = a.df.proj_x * d.n_kv_heads * d.batch;
    a.df.proj_padded = (a.df.n_proj + kXcds - 1) / kXcds * kXcds;
    a.df.counters = step->counters;
    a.df.n_counters = step->n_counters;
  }
  if (step) {  // the step's new tokens compressed and scored in this launch
    a.df.k_new = step->k_new;
    a.df.v_new = step->v_new;
    a.df.A = step->A;
    a.df.P = step->P;
    a.df.E = step->E;
    a.df.start_pos = step->start_pos;
    a.df.zpool = c.z_pages;
    a.df.rpool = residual_pool(d, c);
    a.df.kpool = c.k_pages;
    a.df.new_scores = step->new_scores;
    a.df.ap = step_append_args(d);
    a.df.n_append = d.batch * d.n_kv_heads;
    a.df.app_padded = (a.df.n_append + kXcds - 1) / kXcds * kXcds;
  }
  a.n_q = d.n_q_heads;
  a.n_kv = d.n_kv_heads;
  a.max_pages = d.max_pages_per_seq;
  a.num_phys = d.num_phys_pages;
  a.page_size = d.page_size;
  a.log2_page = ilog2(d.page_size);
  a.geom = pool_geom(d);
  a.cap = d.max_pages_per_seq * d.page_size;
  // 4 wavefronts per workgroup, one step of 64 tokens each
  const int ppi = 64 / d.page_size;
  a.pages_per_wg = ppi * 4;
  a.chunks_per_bg = (d.max_pages_per_seq + a.pages_per_wg - 1) / a.pages_per_wg;
  a.total = d.batch * d.n_kv_heads * a.chunks_per_bg;
  a.padded = (a.total + kXcds - 1) / kXcds * kXcds;
  void *rpool = residual_pool(d, c);
  void *args[] = {(void *)&q_proj, (void *)&c.z_pages, (void *)&rpool,
                  (void *)&c.block_table, (void *)&c.seq_lens, (void *)&scores, (void *)&a};
  return hipLaunchKernel(fn, dim3(a.df.proj_padded + a.df.app_padded + a.padded), dim3(256), args,
                         0, s);
}

bool score_projects(const basiskv_dims &d) { return find_score_proj(d) != nullptr; }

#ifndef BKV_SELECT_SMALL_WAVES
#define BKV_SELECT_SMALL_WAVES 4
#endif
constexpr int kSelectSmallWaves = BKV_SELECT_SMALL_WAVES;  // wavefronts per row up to 1024 pages

hipError_t launch_select(const basiskv_dims &d, float *scores, const int32_t *seq_lens,
                         int32_t top_k, int32_t *sel, hipStream_t s, const int32_t *new_pos,
                         const float *new_scores, uint32_t *epoch) {
  const int mp = d.max_pages_per_seq, cap = d.max_pages_per_seq * d.page_size;
  const dim3 grid(d.n_kv_heads, d.batch);
  if (mp <= 1024)
    hipLaunchKernelGGL((topk_select_kernel<16 / kSelectSmallWaves, kSelectSmallWaves>), grid,
                       dim3(64 * kSelectSmallWaves), 0, s, scores, seq_lens, sel, d.n_kv_heads, mp,
                       d.page_size, cap, top_k, d.recent_tokens, new_pos, new_scores, epoch);
  else if (mp <= 4096)
    hipLaunchKernelGGL((topk_select_kernel<16, 4>), grid, dim3(256), 0, s, scores, seq_lens, sel,
                       d.n_kv_heads, mp, d.page_size, cap, top_k, d.recent_tokens, new_pos, new_scores, epoch);
  else if (mp <= 8192)
    hipLaunchKernelGGL((topk_select_kernel<8, 16>), grid, dim3(1024), 0, s, scores, seq_lens, sel,
                       d.n_kv_heads, mp, d.page_size, cap, top_k, d.recent_tokens, new_pos, new_scores, epoch);
  else if (mp <= 16384)
    hipLaunchKernelGGL((topk_select_kernel<16, 16>), grid, dim3(1024), 0, s, scores, seq_lens, sel,
                       d.n_kv_heads, mp, d.page_size, cap, top_k, d.recent_tokens, new_pos, new_scores, epoch);
  else
    hipLaunchKernelGGL((topk_select_kernel<32, 16>), grid, dim3(1024), 0, s, scores, seq_lens, sel,
                       d.n_kv_heads, mp, d.page_size, cap, top_k, d.recent_tokens, new_pos, new_scores, epoch);
  return hipGetLastError();
}

}  // namespace bkv_host
