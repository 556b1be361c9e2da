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
// grid (ceil(G * (r_b + r_q) / 128), n_kv, batch), 128 threads.
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
template <int KPT, int NWV>
__global__ __launch_bounds__(64 * NWV) void topk_select_kernel(
    const float *__restrict__ scores, const int32_t *__restrict__ seq_lens,
    int32_t *__restrict__ sel, int n_kv, int max_pages, int page_size, int cap, int k,
    int recent) {
  const int g = blockIdx.x, b = blockIdx.y;
  // the whole row is requested before the sequence length arrives
  const float *row = scores + ((int64_t)b * n_kv + g) * max_pages;
  const int base = (threadIdx.x >> 6) * 64 * KPT + (threadIdx.x & 63);
  float v[KPT];
#pragma unroll
  for (int j = 0; j < KPT; ++j) v[j] = base + 64 * j < max_pages ? row[base + 64 * j] : 0.f;
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

struct ScoreArgs {
  int n_q, n_kv, max_pages, num_phys, page_size, log2_page, cap;
  int pages_per_wg, chunks_per_bg, total, padded;
  PoolGeom geom;  // chunk positions of the latent and residual pages
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
template <typename T, int G, int NZ, int NR, bool STREAM, bool MF>
__global__ __launch_bounds__(256) void route_scan_kernel(
    const float *__restrict__ q_proj, const T *__restrict__ zpool, const T *__restrict__ rpool,
    const int32_t *__restrict__ block_table, const int32_t *__restrict__ seq_lens,
    float *__restrict__ scores, ScoreArgs a) {
  constexpr int CE = Elem<T>::CE;
  constexpr int W = (NZ + NR) * CE;  // r_b + r_q
  constexpr int QG = MF ? G / 4 : 1;  // head quads
  constexpr int NST = W / 4;          // 4-dim steps
  static_assert(!MF || (G % 4 == 0 && sizeof(T) <= 2), "matrix-core logits: bf16/E4M3, G % 4 == 0");
  // [quad][step][head in quad]: {hi 4 x bf16, lo 4 x bf16}
  __shared__ __align__(16) uint4 qf[MF ? QG * NST * 4 : 1];
  const int work = xcd_work_index(a.padded);
  if (work >= a.total) return;
  const int bg = work / a.chunks_per_bg;
  const int chunk = work - bg * a.chunks_per_bg;
  const int b = bg / a.n_kv, g = bg - b * a.n_kv;

  const int L = clamp_len(seq_lens[b], a.cap);
  const int NP = (L + a.page_size - 1) >> a.log2_page;
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

  if constexpr (MF) {
    for (int i = threadIdx.x; i < QG * NST * 4; i += blockDim.x) {
      const int hq = i & 3, st = (i >> 2) % NST, qd = i / (NST * 4);
      const float4 v = *reinterpret_cast<const float4 *>(qp + (qd * 4 + hq) * W + st * 4);
      const uint32_t h01 = f32x2_to_bf16x2(v.x, v.y), h23 = f32x2_to_bf16x2(v.z, v.w);
      const uint32_t l01 = f32x2_to_bf16x2(v.x - __uint_as_float(h01 << 16),
                                           v.y - __uint_as_float(h01 & 0xffff0000u));
      const uint32_t l23 = f32x2_to_bf16x2(v.z - __uint_as_float(h23 << 16),
                                           v.w - __uint_as_float(h23 & 0xffff0000u));
      qf[i] = make_uint4(h01, h23, l01, l23);
    }
    __syncthreads();
  }

  if (const int step = wave; step < n_steps) {
    const int p = p_begin + step * ppi + (lane >> a.log2_page);
    const bool in_range = p < p_end;
    const int tok = p * a.page_size + slot;
    int phys = -1;
    if (in_range && p < NP) phys = bt[p];
    const bool valid = in_range && p < NP && tok < L && phys >= 0 && phys < a.num_phys;
    float best = -INFINITY;
    if constexpr (MF) {
      // every lane joins the matrix instructions; one without a valid token
      // scores zeros and is masked
      uint4 cz[NZ], cr[NR];
#pragma unroll
      for (int c = 0; c < NZ; ++c) cz[c] = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
      for (int c = 0; c < NR; ++c) cr[c] = make_uint4(0u, 0u, 0u, 0u);
      if (valid) {
        const int64_t zoff = (zhead + phys) * page_z_bytes + (int64_t)slot * 16;
        const int64_t roff =
            (zhead + phys) * page_r_bytes + ((int64_t)a.geom.r_first * a.page_size + slot) * 16;
#pragma unroll
        for (int c = 0; c < NZ; ++c)
          cz[c] = load_page_chunk<STREAM>(zpool, zoff + (int64_t)c * a.page_size * 16);
#pragma unroll
        for (int c = 0; c < NR; ++c)
          cr[c] = load_page_chunk<STREAM>(rpool, roff + (int64_t)c * a.page_size * 16);
      }
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
      const int64_t zoff = (zhead + phys) * page_z_bytes + (int64_t)slot * 16;
      const int64_t roff =
          (zhead + phys) * page_r_bytes + ((int64_t)a.geom.r_first * a.page_size + slot) * 16;
      uint4 cz[NZ], cr[NR];
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
    best = group_max(best, a.page_size);
    if (in_range && slot == 0) out[p] = (p < NP) ? best : -INFINITY;
  }
}

template <typename T>
hipError_t project_t(const basiskv_dims &d, const void *q, const void *P, const void *Q,
                     float *q_proj, hipStream_t s) {
  const int G = d.n_q_heads / d.n_kv_heads;
  const int outs = G * (d.r_b + d.r_q);
  hipLaunchKernelGGL(project_queries_kernel<T>, dim3((outs + 127) / 128, d.n_kv_heads, d.batch),
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
};

#ifndef BKV_ROUTE_MFMA_MIN_G
#define BKV_ROUTE_MFMA_MIN_G 4
#endif
// groups this wide (of 2-byte or 1-byte pages) take the matrix-core logits
template <typename T, int G>
constexpr bool route_mfma() {
  return sizeof(T) <= 2 && G % 4 == 0 && G >= BKV_ROUTE_MFMA_MIN_G;
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
       : nullptr}

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

hipError_t launch_score(const basiskv_dims &d, const float *q_proj, const basiskv_cache &c,
                        float *scores, hipStream_t s, bool *unsupported) {
  const void *fn = find_score(d);
  if (!fn) {
    *unsupported = true;
    return hipSuccess;
  }
  *unsupported = false;
  ScoreArgs a;
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
  return hipLaunchKernel(fn, dim3(a.padded), dim3(256), args, 0, s);
}

#ifndef BKV_SELECT_SMALL_WAVES
#define BKV_SELECT_SMALL_WAVES 4
#endif
constexpr int kSelectSmallWaves = BKV_SELECT_SMALL_WAVES;  // wavefronts per row up to 1024 pages

hipError_t launch_select(const basiskv_dims &d, const float *scores, const int32_t *seq_lens,
                         int32_t top_k, int32_t *sel, hipStream_t s) {
  const int mp = d.max_pages_per_seq, cap = d.max_pages_per_seq * d.page_size;
  const dim3 grid(d.n_kv_heads, d.batch);
  if (mp <= 1024)
    hipLaunchKernelGGL((topk_select_kernel<16 / kSelectSmallWaves, kSelectSmallWaves>), grid,
                       dim3(64 * kSelectSmallWaves), 0, s, scores, seq_lens, sel, d.n_kv_heads, mp,
                       d.page_size, cap, top_k, d.recent_tokens);
  else if (mp <= 4096)
    hipLaunchKernelGGL((topk_select_kernel<16, 4>), grid, dim3(256), 0, s, scores, seq_lens, sel,
                       d.n_kv_heads, mp, d.page_size, cap, top_k, d.recent_tokens);
  else if (mp <= 8192)
    hipLaunchKernelGGL((topk_select_kernel<8, 16>), grid, dim3(1024), 0, s, scores, seq_lens, sel,
                       d.n_kv_heads, mp, d.page_size, cap, top_k, d.recent_tokens);
  else if (mp <= 16384)
    hipLaunchKernelGGL((topk_select_kernel<16, 16>), grid, dim3(1024), 0, s, scores, seq_lens, sel,
                       d.n_kv_heads, mp, d.page_size, cap, top_k, d.recent_tokens);
  else
    hipLaunchKernelGGL((topk_select_kernel<32, 16>), grid, dim3(1024), 0, s, scores, seq_lens, sel,
                       d.n_kv_heads, mp, d.page_size, cap, top_k, d.recent_tokens);
  return hipGetLastError();
}

}  // namespace bkv_host
