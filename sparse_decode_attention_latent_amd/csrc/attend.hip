// (a4) Exact attention over the selected pages with a latent-space weighted
// sum.  BasisKV (arXiv 2611.02583): abstract (exact QK scores from the
// original Keys of the selected pages only), Figure 1 (the attention output
// is carried as a Value latent), appendix Table 4 (selected attention reads
// r_v latent dims and head_dim Key dims per selected token).
//
// Split-K over the selected pages, flash-decoding style: each workgroup takes
// a run of one (sequence, KV head)'s selected pages, keeps a running max /
// sum / latent accumulator per query head, and writes one partial; a second
// kernel merges the partials in a fixed order (deterministic, no atomics).
#include "common.hpp"

namespace bkv {

struct AttendArgs {
  int n_q, n_kv, max_pages, num_phys, page_size, log2_page, cap, top_k;
  int pages_per_split, n_split, total, padded;
  float scale_log2;  // scale * log2(e): exponentials are taken base 2
};

// Partial record per (b, h, split): [m, l, u[0..r_v)] with m in base-2 logit
// units (scale * log2 e already applied), l = sum 2^(s - m), u = sum 2^(s - m) z.
template <typename T, int G, int NVC>
__global__ __launch_bounds__(256) void attend_split_kernel(
    const T *__restrict__ q, const T *__restrict__ kpool, const T *__restrict__ zpool,
    const int32_t *__restrict__ block_table, const int32_t *__restrict__ seq_lens,
    const int32_t *__restrict__ sel, float *__restrict__ part, AttendArgs a) {
  constexpr int CE = Elem<T>::CE;
  constexpr int NKC = kHeadDim / CE;  // Key chunks per token
  constexpr int RV = NVC * CE;        // latent width
  constexpr int TG = kWave / NVC;     // token groups in the latent phase
  constexpr int NJ = (kWave + TG - 1) / TG;
  constexpr int NW = 4;               // wavefronts per workgroup

  __shared__ float p_lds[NW][kWave][G];
  __shared__ int64_t zoff_lds[NW][kWave];
  __shared__ float m_lds[NW][G];
  __shared__ float l_lds[NW][G];
  __shared__ float u_lds[NW][G][RV];

  const int work = xcd_work_index(a.padded);
  if (work >= a.total) return;  // uniform per workgroup
  const int bg = work / a.n_split;
  const int split = work - bg * a.n_split;
  const int b = bg / a.n_kv, g = bg - b * a.n_kv;
  const int L = clamp_len(seq_lens[b], a.cap);
  const int NP = (L + a.page_size - 1) >> a.log2_page;

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;
  const int slot = lane & (a.page_size - 1);
  const int ppi = kWave >> a.log2_page;  // pages per 64-token block
  const int e_begin = split * a.pages_per_split;
  const int e_end = min(a.top_k, e_begin + a.pages_per_split);
  const int n_blocks = (e_end - e_begin + ppi - 1) / ppi;
  const int n_iter = (n_blocks + NW - 1) / NW;  // same trip count for every wavefront

  const int32_t *sel_bg = sel + (int64_t)bg * a.top_k;
  const int32_t *bt = block_table + (int64_t)b * a.max_pages;
  const uint32_t *q32 = reinterpret_cast<const uint32_t *>(q);
  const int64_t qrow0 = ((int64_t)b * a.n_q + (int64_t)g * G) * kHeadDim;  // element index
  const int64_t head_page0 = (int64_t)g * a.num_phys;
  const int64_t kpage_bytes = (int64_t)NKC * a.page_size * 16;
  const int64_t zpage_bytes = (int64_t)NVC * a.page_size * 16;

  // latent-phase lane roles: chunk c of tokens t = j * TG + tg
  const int vc = lane % NVC;
  const int tg = lane / NVC;

  float m_run[G], l_lane[G], acc[G][CE];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m_run[h] = -INFINITY;
    l_lane[h] = 0.f;
#pragma unroll
    for (int e = 0; e < CE; ++e) acc[h][e] = 0.f;
  }

  for (int it = 0; it < n_iter; ++it) {
    const int blk = it * NW + wave;
    const int e = e_begin + blk * ppi + (lane >> a.log2_page);
    int page = -1;
    if (blk < n_blocks && e < e_end) page = sel_bg[e];
    int phys = -1;
    if (page >= 0 && page < NP) phys = bt[page];
    const int tok = page * a.page_size + slot;
    const bool valid = page >= 0 && page < NP && tok < L && phys >= 0 && phys < a.num_phys;

    // ---- exact scores, one token per lane ----
    float s[G];
#pragma unroll
    for (int h = 0; h < G; ++h) s[h] = -INFINITY;
    int64_t zoff = -1;
    if (valid) {
      const int64_t koff = (head_page0 + phys) * kpage_bytes + (int64_t)slot * 16;
      zoff = (head_page0 + phys) * zpage_bytes + (int64_t)slot * 16;
      uint4 kc[NKC];
#pragma unroll
      for (int c = 0; c < NKC; ++c) kc[c] = load_chunk(kpool, koff + (int64_t)c * a.page_size * 16);
      float dot[G];
#pragma unroll
      for (int h = 0; h < G; ++h) dot[h] = 0.f;
#pragma unroll
      for (int c = 0; c < NKC; ++c) {
        float x[CE];
        unpack_chunk<T>(kc[c], x);
#pragma unroll
        for (int ee = 0; ee < CE; ++ee) {
          const int d = c * CE + ee;
#pragma unroll
          for (int h = 0; h < G; ++h) {
            float qv;
            if constexpr (CE == 8) {
              const uint32_t w = q32[(qrow0 + (int64_t)h * kHeadDim + d) >> 1];
              qv = (d & 1) ? __uint_as_float(w & 0xffff0000u) : __uint_as_float(w << 16);
            } else {
              qv = reinterpret_cast<const float *>(q)[qrow0 + (int64_t)h * kHeadDim + d];
            }
            dot[h] = fmaf(qv, x[ee], dot[h]);
          }
        }
      }
#pragma unroll
      for (int h = 0; h < G; ++h) s[h] = dot[h] * a.scale_log2;
    }

    // ---- online softmax update (wave-uniform running max per head) ----
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float bm = wave_max(s[h]);
      const float m_new = fmaxf(m_run[h], bm);
      float pr = 0.f, alpha = 1.f;
      if (m_new != -INFINITY) {
        alpha = exp2f(m_run[h] - m_new);  // 0 when m_run is -inf
        pr = valid ? exp2f(s[h] - m_new) : 0.f;
      }
      m_run[h] = m_new;
      l_lane[h] = l_lane[h] * alpha + pr;
#pragma unroll
      for (int ee = 0; ee < CE; ++ee) acc[h][ee] *= alpha;
      p_lds[wave][lane][h] = pr;
    }
    zoff_lds[wave][lane] = zoff;
    __syncthreads();

    // ---- latent weighted sum: lane (tg, vc) takes chunk vc of tokens j*TG + tg ----
    if (tg < TG) {
      uint4 zc[NJ];
      int64_t zo[NJ];
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int t = j * TG + tg;
        zo[j] = (t < kWave) ? zoff_lds[wave][t] : -1;
        if (zo[j] >= 0) zc[j] = load_chunk(zpool, zo[j] + (int64_t)vc * a.page_size * 16);
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int t = j * TG + tg;
        if (zo[j] >= 0) {
          float x[CE];
          unpack_chunk<T>(zc[j], x);
#pragma unroll
          for (int h = 0; h < G; ++h) {
            const float pr = p_lds[wave][t][h];
#pragma unroll
            for (int ee = 0; ee < CE; ++ee) acc[h][ee] = fmaf(pr, x[ee], acc[h][ee]);
          }
        }
      }
    }
    __syncthreads();
  }

  // ---- merge: token groups of each wavefront, then the wavefronts ----
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float lw = wave_sum(l_lane[h]);
    if (lane == 0) {
      m_lds[wave][h] = m_run[h];
      l_lds[wave][h] = lw;
    }
  }
  for (int i = lane; i < G * RV; i += kWave) u_lds[wave][i / RV][i % RV] = 0.f;
  __syncthreads();
  for (int t = 0; t < TG; ++t) {
    if (tg == t) {
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int ee = 0; ee < CE; ++ee) u_lds[wave][h][vc * CE + ee] += acc[h][ee];
    }
    __syncthreads();
  }
  const int rec = RV + 2;
  for (int i = threadIdx.x; i < G * RV; i += blockDim.x) {
    const int h = i / RV, d = i % RV;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, m_lds[w][h]);
    float lsum = 0.f, usum = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float f = exp2f(m_lds[w][h] - M);
        lsum = fmaf(l_lds[w][h], f, lsum);
        usum = fmaf(u_lds[w][h][d], f, usum);
      }
    }
    float *rp = part + (((int64_t)b * a.n_q + (int64_t)g * G + h) * a.n_split + split) * rec;
    rp[2 + d] = usum;
    if (d == 0) {
      rp[0] = M;
      rp[1] = lsum;
    }
  }
}

// Merge of the split partials: u = sum_s u_s 2^(m_s - M) / sum_s l_s 2^(m_s - M).
// grid (n_q, batch), 128 threads; a head with no valid token gets u = 0.
__global__ __launch_bounds__(128) void attend_combine_kernel(const float *__restrict__ part,
                                                             float *__restrict__ u, int n_q,
                                                             int rv, int n_split) {
  const int h = blockIdx.x, b = blockIdx.y;
  const int rec = rv + 2;
  const float *base = part + ((int64_t)b * n_q + h) * n_split * rec;
  float M = -INFINITY;
  for (int s = 0; s < n_split; ++s) M = fmaxf(M, base[s * rec]);
  for (int d = threadIdx.x; d < rv; d += blockDim.x) {
    float lsum = 0.f, usum = 0.f;
    if (M != -INFINITY) {
      for (int s = 0; s < n_split; ++s) {
        const float f = exp2f(base[s * rec] - M);
        lsum = fmaf(base[s * rec + 1], f, lsum);
        usum = fmaf(base[s * rec + 2 + d], f, usum);
      }
    }
    u[((int64_t)b * n_q + h) * rv + d] = lsum > 0.f ? usum / lsum : 0.f;
  }
}

struct AttendVariant {
  int dtype, G, rv;
  const void *fn;
};

#define BKV_ATT(T, DT, G, RV) \
  {DT, G, RV, reinterpret_cast<const void *>(&attend_split_kernel<T, G, (RV) / Elem<T>::CE>)}
#define BKV_ATT_G(T, DT, RV) \
  BKV_ATT(T, DT, 1, RV), BKV_ATT(T, DT, 2, RV), BKV_ATT(T, DT, 4, RV), BKV_ATT(T, DT, 8, RV)

static const AttendVariant kAttendVariants[] = {
    BKV_ATT_G(uint16_t, BASISKV_BF16, 64), BKV_ATT_G(uint16_t, BASISKV_BF16, 96),
    BKV_ATT_G(uint16_t, BASISKV_BF16, 32), BKV_ATT_G(uint16_t, BASISKV_BF16, 128),
    BKV_ATT_G(float, BASISKV_F32, 64),     BKV_ATT_G(float, BASISKV_F32, 32),
};

}  // namespace bkv

namespace bkv_host {
using namespace bkv;

static int ilog2i(int x) {
  int l = 0;
  while ((1 << l) < x) ++l;
  return l;
}

// Pages per split: 4 wavefronts x one 64-token block each.
static int pages_per_split(const basiskv_dims &d) { return 4 * (64 / d.page_size); }

int attend_splits(const basiskv_dims &d, int32_t top_k) {
  const int pps = pages_per_split(d);
  return (top_k + pps - 1) / pps;
}

static const void *find_attend(const basiskv_dims &d) {
  const int G = d.n_q_heads / d.n_kv_heads;
  for (const auto &v : kAttendVariants)
    if (v.dtype == d.dtype && v.G == G && v.rv == d.r_v) return v.fn;
  return nullptr;
}

bool attend_supported(const basiskv_dims &d) { return find_attend(d) != nullptr; }

hipError_t launch_attend(const basiskv_dims &d, const void *q, const basiskv_cache &c,
                         const int32_t *sel, int32_t top_k, float scale, float *u, float *part,
                         hipStream_t s, bool *unsupported) {
  const void *fn = find_attend(d);
  if (!fn) {
    *unsupported = true;
    return hipSuccess;
  }
  *unsupported = false;
  AttendArgs a;
  a.n_q = d.n_q_heads;
  a.n_kv = d.n_kv_heads;
  a.max_pages = d.max_pages_per_seq;
  a.num_phys = d.num_phys_pages;
  a.page_size = d.page_size;
  a.log2_page = ilog2i(d.page_size);
  a.cap = d.max_pages_per_seq * d.page_size;
  a.top_k = top_k;
  a.pages_per_split = pages_per_split(d);
  a.n_split = attend_splits(d, top_k);
  a.total = d.batch * d.n_kv_heads * a.n_split;
  a.padded = (a.total + kXcds - 1) / kXcds * kXcds;
  a.scale_log2 = scale * kLog2e;
  void *args[] = {(void *)&q,          (void *)&c.k_pages, (void *)&c.z_pages,
                  (void *)&c.block_table, (void *)&c.seq_lens, (void *)&sel,
                  (void *)&part,       (void *)&a};
  hipError_t e = hipLaunchKernel(fn, dim3(a.padded), dim3(256), args, 0, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attend_combine_kernel, dim3(d.n_q_heads, d.batch), dim3(128), 0, s, part, u,
                     d.n_q_heads, d.r_v, a.n_split);
  return hipGetLastError();
}

}  // namespace bkv_host
