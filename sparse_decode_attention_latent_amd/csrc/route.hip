// Routing kernels: query projection (a1), page scoring (a2), top-k page
// selection (a3).  BasisKV (arXiv 2611.02583): the abstract's latent-based Key
// routing with a Key-specific residual; appendix Table 4's routing read widths
// (r_b latent dims + r_q residual dims per context token); Table 9's caption
// (routing by page, with a page budget).
#include "common.hpp"

namespace bkv {

// ---------------------------------------------------------------------------
// (a1) q_proj[b][h] = [P_g q_bh, Q_g q_bh]   (float32, exact widening of inputs)
// grid (ceil(G * (r_b + r_q) / 128), n_kv, batch), 128 threads: one output per
// thread; its whole factor row (head_dim elements) is requested before the
// queries are staged, so the two loads overlap.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(128) void project_queries_kernel(
    const T *__restrict__ q, const T *__restrict__ P, const T *__restrict__ Q,
    float *__restrict__ q_proj, int n_q, int n_kv, int rb, int rq) {
  constexpr int CE = Elem<T>::CE;
  constexpr int NC = kHeadDim / CE;
  __shared__ __align__(16) float qs[16][kHeadDim];
  const int g = blockIdx.y, b = blockIdx.z;
  const int G = n_q / n_kv;
  const int w = rb + rq;
  const int o = blockIdx.x * blockDim.x + threadIdx.x;
  const bool active = o < G * w;
  const int h = active ? o / w : 0, j = active ? o % w : 0;
  const T *row = j < rb ? P + ((int64_t)g * rb + j) * kHeadDim
                        : Q + ((int64_t)g * rq + (j - rb)) * kHeadDim;
  uint4 c[NC];
  if (active) {  // the factor row is in flight while the queries are staged
#pragma unroll
    for (int i = 0; i < NC; ++i) c[i] = reinterpret_cast<const uint4 *>(row)[i];
  }
  {  // the group's queries: G * head_dim elements, 128 threads, one batch of loads
    const T *qg = q + ((int64_t)b * n_q + g * G) * kHeadDim;
    T qv[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int i = u * 128 + threadIdx.x;
      if (i < G * kHeadDim) qv[u] = qg[i];
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int i = u * 128 + threadIdx.x;
      if (i < G * kHeadDim) qs[i / kHeadDim][i % kHeadDim] = to_f32(qv[u]);
    }
  }
  __syncthreads();
  if (!active) return;
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    float x[CE];
    unpack_chunk<T>(c[i], x);
#pragma unroll
    for (int e = 0; e < CE; ++e) acc = fmaf(x[e], qs[h][i * CE + e], acc);
  }
  q_proj[((int64_t)b * n_q + g * G + h) * w + j] = acc;
}

// ---------------------------------------------------------------------------
// (a2) page scores.
//
// One lane per token: a wavefront covers 64 tokens (64 / page_size pages) per
// step, each lane issuing NZ + NR 16-byte loads (its token's chunks of the
// latent and residual pages).  With the chunk-major page layout those loads
// are page_size * 16 contiguous bytes per chunk, i.e. fully coalesced.  The
// projected queries are wave-uniform and are read through the scalar cache,
// so every FMA takes one scalar and one vector operand.  Page maxima are
// butterfly reductions over the page's lanes.
// ---------------------------------------------------------------------------
#ifndef BKV_ROUTE_STEPS
#define BKV_ROUTE_STEPS 4
#endif
constexpr int kRouteSteps = BKV_ROUTE_STEPS;

struct ScoreArgs {
  int n_q, n_kv, max_pages, num_phys, page_size, log2_page, zc_total, cap;
  int pages_per_wg, chunks_per_bg, total, padded;
};

template <typename T, int G, int NZ, int NR>
__global__ __launch_bounds__(256) void route_scan_kernel(
    const float *__restrict__ q_proj, const T *__restrict__ zpool, const T *__restrict__ rpool,
    const int32_t *__restrict__ block_table, const int32_t *__restrict__ seq_lens,
    float *__restrict__ scores, ScoreArgs a) {
  constexpr int CE = Elem<T>::CE;
  constexpr int W = (NZ + NR) * CE;  // r_b + r_q
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
  const int64_t page_z_bytes = (int64_t)a.zc_total * a.page_size * 16;
  const int64_t page_r_bytes = (int64_t)NR * a.page_size * 16;

  for (int step = wave; step < n_steps; step += 4) {
    const int p = p_begin + step * ppi + (lane >> a.log2_page);
    const bool in_range = p < p_end;
    const int tok = p * a.page_size + slot;
    int phys = -1;
    if (in_range && p < NP) phys = bt[p];
    const bool valid = in_range && p < NP && tok < L && phys >= 0 && phys < a.num_phys;
    float best = -INFINITY;
    if (valid) {
      const int64_t zoff = (zhead + phys) * page_z_bytes + (int64_t)slot * 16;
      const int64_t roff = (zhead + phys) * page_r_bytes + (int64_t)slot * 16;
      uint4 cz[NZ], cr[NR];
#pragma unroll
      for (int c = 0; c < NZ; ++c) cz[c] = load_chunk(zpool, zoff + (int64_t)c * a.page_size * 16);
#pragma unroll
      for (int c = 0; c < NR; ++c) cr[c] = load_chunk(rpool, roff + (int64_t)c * a.page_size * 16);
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

// ---------------------------------------------------------------------------
// (a3) exact top-k per (sequence, KV head).  Scores become order-preserving
// 32-bit keys in LDS.  The k-th largest key tau is built two bits at a time
// from the top: of the candidates tau | d << shift, the largest that at least
// k keys reach is kept (counts by wavefront ballots, one barrier per round,
// no atomics).  The compaction then takes, in index order, every key above
// tau and the lowest-index keys equal to it.
// grid (n_kv, batch), 256 threads, dynamic LDS = max_pages * 4 bytes.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t order_key(float f) {
  if (f != f) return 0u;                      // NaN ranks lowest
  uint32_t u = __float_as_uint(f == 0.f ? 0.f : f);  // -0 == +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix sum over the 256 threads of the block (unsigned, so two
// 16-bit counts may share one word); returns the total via *total.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t *scratch,
                                                         uint32_t *total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t t = __shfl_up(incl, off);
    if (lane >= off) incl += t;
  }
  if (lane == 63) scratch[wave] = incl;
  __syncthreads();
  uint32_t base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t s = scratch[w];
    if (w < wave) base += s;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return base + incl - v;
}

__global__ __launch_bounds__(256) void topk_select_kernel(
    const float *__restrict__ scores, const int32_t *__restrict__ seq_lens,
    int32_t *__restrict__ sel, int n_kv, int max_pages, int page_size, int cap, int k) {
  extern __shared__ uint32_t keys[];
  __shared__ int counts[2][4][3];
  __shared__ uint32_t scan_scratch[4];
  const int g = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x;
  const int L = clamp_len(seq_lens[b], cap);
  const int NP = (L + page_size - 1) / page_size;
  int32_t *out = sel + ((int64_t)b * n_kv + g) * k;
  if (k >= NP) {
    for (int i = tid; i < k; i += 256) out[i] = i < NP ? i : -1;
    return;
  }
  const float *row = scores + ((int64_t)b * n_kv + g) * max_pages;
  for (int i0 = 0; i0 < NP; i0 += 256 * 16) {  // 16 loads per thread in flight
    float v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int i = i0 + u * 256 + tid;
      v[u] = i < NP ? row[i] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int i = i0 + u * 256 + tid;
      if (i < NP) keys[i] = order_key(v[u]);
    }
  }
  __syncthreads();

  // two bits per round: counts of keys reaching the three candidates
  // tau | d << shift (d = 1, 2, 3), one ballot per candidate and 64 keys
  const int lane = tid & 63, wave = tid >> 6;
  uint32_t tau = 0;
  int buf = 0;
  for (int shift = 30; shift >= 0; shift -= 2, buf ^= 1) {
    const uint32_t c1 = tau | (1u << shift), c2 = tau | (2u << shift), c3 = tau | (3u << shift);
    int n1 = 0, n2 = 0, n3 = 0;
    for (int i0 = wave * 64; i0 < NP; i0 += 256) {  // wavefront-uniform trip count
      const int i = i0 + lane;
      const uint32_t key = i < NP ? keys[i] : 0u;  // 0 reaches no candidate (all >= 1)
      n1 += __popcll(__ballot(key >= c1));
      n2 += __popcll(__ballot(key >= c2));
      n3 += __popcll(__ballot(key >= c3));
    }
    if (lane == 0) {
      counts[buf][wave][0] = n1;
      counts[buf][wave][1] = n2;
      counts[buf][wave][2] = n3;
    }
    __syncthreads();
    int t1 = 0, t2 = 0, t3 = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      t1 += counts[buf][w][0];
      t2 += counts[buf][w][1];
      t3 += counts[buf][w][2];
    }
    const uint32_t dg = t3 >= k ? 3u : t2 >= k ? 2u : t1 >= k ? 1u : 0u;
    tau |= dg << shift;
  }
  // tau is the k-th largest key: at least k keys reach it, fewer than k exceed it

  const int per = (NP + 255) / 256;
  const int i0 = min(NP, tid * per), i1 = min(NP, i0 + per);
  uint32_t n_gt = 0, n_eq = 0;
  for (int i = i0; i < i1; ++i) {
    const uint32_t key = keys[i];
    n_gt += key > tau;
    n_eq += key == tau;
  }
  // one scan of both counts: each total is < 65536 (NP <= 32768 < k + NP), so
  // the low half never carries into the high half
  uint32_t total;
  const uint32_t packed = block_exclusive_scan(n_gt | (n_eq << 16), scan_scratch, &total);
  const int need = k - (int)(total & 0xffffu);  // keys equal to tau still to take
  const int eq_before = (int)(packed >> 16);
  const int take_eq = max(0, min((int)n_eq, need - eq_before));
  int pos = (int)(packed & 0xffffu) + min(eq_before, need);
  int taken = 0;
  for (int i = i0; i < i1; ++i) {
    const uint32_t key = keys[i];
    if (key > tau || (key == tau && taken < take_eq)) {
      taken += key == tau;
      out[pos++] = i;
    }
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

struct ScoreVariant {
  int dtype, G, rb, rq;
  const void *fn;
};

#define BKV_SCORE(T, DT, G, RB, RQ)                                                        \
  {DT, G, RB, RQ,                                                                           \
   reinterpret_cast<const void *>(                                                          \
       &route_scan_kernel<T, G, (RB) / Elem<T>::CE, (RQ) / Elem<T>::CE>)}

#define BKV_SCORE_G(T, DT, RB, RQ) \
  BKV_SCORE(T, DT, 1, RB, RQ), BKV_SCORE(T, DT, 2, RB, RQ), BKV_SCORE(T, DT, 4, RB, RQ), \
      BKV_SCORE(T, DT, 8, RB, RQ)

static const ScoreVariant kScoreVariants[] = {
    BKV_SCORE_G(uint16_t, BASISKV_BF16, 64, 32), BKV_SCORE_G(uint16_t, BASISKV_BF16, 96, 48),
    BKV_SCORE_G(uint16_t, BASISKV_BF16, 16, 16), BKV_SCORE_G(uint16_t, BASISKV_BF16, 32, 32),
    BKV_SCORE_G(uint16_t, BASISKV_BF16, 32, 16),
    BKV_SCORE_G(uint16_t, BASISKV_BF16, 128, 32), BKV_SCORE_G(float, BASISKV_F32, 64, 32),
    BKV_SCORE_G(float, BASISKV_F32, 16, 16), BKV_SCORE_G(float, BASISKV_F32, 32, 16),
};

}  // namespace bkv

namespace bkv_host {
using namespace bkv;

hipError_t launch_project(const basiskv_dims &d, const void *q, const void *P, const void *Q,
                          float *q_proj, hipStream_t s) {
  return d.dtype == BASISKV_BF16 ? project_t<uint16_t>(d, q, P, Q, q_proj, s)
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
    if (v.dtype == d.dtype && v.G == G && v.rb == d.r_b && v.rq == d.r_q) return v.fn;
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
  const int ce = d.dtype == BASISKV_BF16 ? 8 : 4;
  ScoreArgs a;
  a.n_q = d.n_q_heads;
  a.n_kv = d.n_kv_heads;
  a.max_pages = d.max_pages_per_seq;
  a.num_phys = d.num_phys_pages;
  a.page_size = d.page_size;
  a.log2_page = ilog2(d.page_size);
  a.zc_total = d.r_v / ce;
  a.cap = d.max_pages_per_seq * d.page_size;
  // 4 wavefronts per workgroup, each streaming kRouteSteps steps of 64 tokens.
  const int ppi = 64 / d.page_size;
  a.pages_per_wg = ppi * 4 * kRouteSteps;
  a.chunks_per_bg = (d.max_pages_per_seq + a.pages_per_wg - 1) / a.pages_per_wg;
  a.total = d.batch * d.n_kv_heads * a.chunks_per_bg;
  a.padded = (a.total + kXcds - 1) / kXcds * kXcds;
  void *args[] = {(void *)&q_proj, (void *)&c.z_pages, (void *)&c.r_pages,
                  (void *)&c.block_table, (void *)&c.seq_lens, (void *)&scores, (void *)&a};
  return hipLaunchKernel(fn, dim3(a.padded), dim3(256), args, 0, s);
}

hipError_t launch_select(const basiskv_dims &d, const float *scores, const int32_t *seq_lens,
                         int32_t top_k, int32_t *sel, hipStream_t s) {
  const size_t lds = (size_t)d.max_pages_per_seq * sizeof(uint32_t);
  if (lds > 48 * 1024) {
    // more than the default dynamic LDS: raise the kernel's limit (gfx950 has 160 KB per CU)
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&topk_select_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(topk_select_kernel, dim3(d.n_kv_heads, d.batch), dim3(256), lds, s, scores,
                     seq_lens, sel, d.n_kv_heads, d.max_pages_per_seq, d.page_size,
                     d.max_pages_per_seq * d.page_size, top_k);
  return hipGetLastError();
}

}  // namespace bkv_host
