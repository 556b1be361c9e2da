// (a4) Exact attention over the selected pages with a latent-space weighted
// sum.  BasisKV (arXiv 2611.02583): abstract (exact QK scores from the
// original Keys of the selected pages only), Figure 1 (the attention output
// is carried as a Value latent), appendix Table 4 (selected attention reads
// r_v latent dims and head_dim Key dims per selected token).
//
// Split-K over the selected pages, flash-decoding style.  Each workgroup
// takes a run of one (sequence, KV head)'s selected pages; each of its
// wavefronts walks 64-token blocks of that run with one token per lane:
//   * the lane gathers its token's Key (head_dim * 2 or 4 bytes as 16-byte
//     chunks: with the chunk-major page layout a wavefront reads page_size *
//     16 contiguous bytes per chunk) and, in the same breath, the latent
//     chunks it owns in the weighted-sum phase, so both gathers are in flight
//     together;
//   * exact scores against the group's queries, held as float32 in LDS and
//     read by broadcast;
//   * an online softmax with a wavefront-uniform running max per head;
//   * the weighted latent sum: the block's probabilities go through a
//     wavefront-private LDS row, and lane (tg, vc) accumulates chunk vc of the
//     tokens tg, tg + TG, ... for every head of the group.
// The wavefronts and the workgroup's splits are merged in a fixed order
// (deterministic: no floating-point atomics).  A single split writes u
// directly; otherwise every split writes a partial record and the last split
// of the (sequence, KV head) to finish -- elected with an integer counter --
// merges the records in split order.
#include "common.hpp"

namespace bkv {

constexpr int kAttendWaves = 4;
#ifndef BKV_ATTEND_WAVES_PER_EU
#define BKV_ATTEND_WAVES_PER_EU 2
#endif
constexpr int kMaxSplits = 64;  // partial records per (sequence, head)
#ifndef BKV_ATTEND_BLOCKS
#define BKV_ATTEND_BLOCKS 2
#endif
constexpr int kAttendBlocks = BKV_ATTEND_BLOCKS;  // 64-token blocks per wavefront

struct AttendArgs {
  int n_q, n_kv, max_pages, num_phys, page_size, log2_page, cap, top_k;
  int pages_per_split, n_split, total, padded;
  float scale_log2;  // scale * log2(e): exponentials are taken base 2
  int32_t *counters;  // [batch * n_kv], zero between calls (see the merge)
  uint16_t *u_tiles;  // optional: u also written as the reconstruction's A operand (bf16)
};

// Ordering point for LDS traffic between the lanes of one wavefront.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Partial record per (b, h, split): [m, l, u[0..r_v)] with m in base-2 logit
// units (scale * log2 e already applied), l = sum 2^(s - m), u = sum 2^(s - m) z.
//
// Each wavefront owns kAttendBlocks 64-token blocks of the split; their
// selection entries and block-table rows are requested before the queries are
// staged, so the chain selection -> block table -> Key gather costs its
// latency once per wavefront rather than once per block.  With a wide query
// group (G * latent chunks > 48) the latent chunks are gathered after the
// scores instead of beside the Key, keeping the live registers within two
// wavefronts per SIMD.
template <typename T, int G, int NVC>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(BKV_ATTEND_WAVES_PER_EU)))
void attend_split_kernel(
    const T *__restrict__ q, const T *__restrict__ kpool, const T *__restrict__ zpool,
    const int32_t *__restrict__ block_table, const int32_t *__restrict__ seq_lens,
    const int32_t *__restrict__ sel, float *__restrict__ part, float *__restrict__ u_out,
    AttendArgs a) {
  constexpr int CE = Elem<T>::CE;
  constexpr int NKC = kHeadDim / CE;  // Key chunks per token
  constexpr int RV = NVC * CE;        // latent width
  constexpr int TG = kWave / NVC;     // token groups in the latent phase
  constexpr int NJ = (kWave + TG - 1) / TG;
  constexpr int NW = kAttendWaves;
  constexpr int NB = kAttendBlocks;
  constexpr bool kZLate = G * NVC > 48 || sizeof(T) == 4;

  __shared__ __align__(16) float q_lds[G][kHeadDim];
  __shared__ float p_lds[NW][G][kWave];
  __shared__ float m_lds[NW][G];
  __shared__ float l_lds[NW][G];
  __shared__ float u_lds[NW][G][RV];

  const int work = xcd_work_index(a.padded);
  if (work >= a.total) return;  // uniform per workgroup
  const int bg = work / a.n_split;
  const int split = work - bg * a.n_split;
  const int b = bg / a.n_kv, g = bg - b * a.n_kv;

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;
  const int slot = lane & (a.page_size - 1);
  const int ppi = kWave >> a.log2_page;  // pages per 64-token block
  const int e_begin = split * a.pages_per_split;
  const int e_end = min(a.top_k, e_begin + a.pages_per_split);
  const int n_blocks = (e_end - e_begin + ppi - 1) / ppi;
  const int32_t *sel_bg = sel + (int64_t)bg * a.top_k;
  const int32_t *bt = block_table + (int64_t)b * a.max_pages;

  // ---- this wavefront's blocks of round r: selection entries, then physical pages ----
  const int L = clamp_len(seq_lens[b], a.cap);
  const int NP = (L + a.page_size - 1) >> a.log2_page;
  const int n_rounds = (n_blocks + NW * NB - 1) / (NW * NB);
  int page[NB], phys[NB];
  auto fetch_pages = [&](int r) {
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int blk = (r * NB + i) * NW + wave;
      const int e = e_begin + blk * ppi + (lane >> a.log2_page);
      page[i] = (blk < n_blocks && e < e_end) ? sel_bg[e] : -1;
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      phys[i] = -1;
      if (page[i] >= 0 && page[i] < NP) phys[i] = bt[page[i]];
    }
  };
  fetch_pages(0);

  // The group's queries: bf16 kept as packed pairs (the scores use the
  // two-term bf16 dot instruction, products exact, float32 sums), float32 as is.
  {
    constexpr int QW = G * kHeadDim * (int)sizeof(T) / 4;  // 32-bit words
    constexpr int QL = (QW + 255) / 256;
    const uint32_t *qg = reinterpret_cast<const uint32_t *>(
        q + ((int64_t)b * a.n_q + (int64_t)g * G) * kHeadDim);
    uint32_t *qw = reinterpret_cast<uint32_t *>(&q_lds[0][0]);
    uint32_t qv[QL];
#pragma unroll
    for (int u = 0; u < QL; ++u) {
      const int i = u * 256 + threadIdx.x;
      if (i < QW) qv[u] = qg[i];
    }
#pragma unroll
    for (int u = 0; u < QL; ++u) {
      const int i = u * 256 + threadIdx.x;
      if (i < QW) qw[i] = qv[u];
    }
  }
  __syncthreads();

  const int64_t head_page0 = (int64_t)g * a.num_phys;
  const int64_t kpage_bytes = (int64_t)NKC * a.page_size * 16;
  const int64_t zpage_bytes = (int64_t)NVC * a.page_size * 16;
  const int64_t chunk_stride = (int64_t)a.page_size * 16;

  // latent-phase lane roles: chunk vc of tokens t = j * TG + tg
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

  for (int r = 0; r < n_rounds; ++r) {
  if (r > 0) fetch_pages(r);
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    if ((r * NB + i) * NW + wave >= n_blocks) break;  // wavefront-uniform
    const int tok = page[i] * a.page_size + slot;
    const bool valid = page[i] >= 0 && page[i] < NP && tok < L && phys[i] >= 0 &&
                       phys[i] < a.num_phys;

    // ---- gathers: this lane's Key, and the latent chunks it sums ----
    uint4 kc[NKC];
    if (valid) {
      const int64_t koff = (head_page0 + phys[i]) * kpage_bytes + (int64_t)slot * 16;
#pragma unroll
      for (int c = 0; c < NKC; ++c) kc[c] = load_chunk(kpool, koff + c * chunk_stride);
    }
    uint4 zc[NJ];
    bool zv[NJ];
    auto gather_latents = [&]() {
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int t = j * TG + tg;
        const bool role = tg < TG && t < kWave;
        const int src = role ? t : 0;
        const int phys_t = __shfl(phys[i], src);
        const int valid_t = __shfl((int)valid, src);
        zv[j] = role && valid_t;
        if (zv[j])
          zc[j] = load_chunk(zpool, (head_page0 + phys_t) * zpage_bytes + vc * chunk_stride +
                                        (int64_t)(src & (a.page_size - 1)) * 16);
      }
    };
    if (!kZLate) gather_latents();

    // ---- exact scores, one token per lane ----
    float s[G];
#pragma unroll
    for (int h = 0; h < G; ++h) s[h] = -INFINITY;
    if (valid) {
      float dot[G];
#pragma unroll
      for (int h = 0; h < G; ++h) dot[h] = 0.f;
#pragma unroll
      for (int c = 0; c < NKC; ++c) {
        if constexpr (sizeof(T) == 2) {
          const uint32_t *qw = reinterpret_cast<const uint32_t *>(&q_lds[0][0]);
#pragma unroll
          for (int h = 0; h < G; ++h) {
            const uint4 q4 = *reinterpret_cast<const uint4 *>(qw + h * (kHeadDim / 2) + c * 4);
            dot[h] = dot2_bf16(kc[c].x, q4.x, dot[h]);
            dot[h] = dot2_bf16(kc[c].y, q4.y, dot[h]);
            dot[h] = dot2_bf16(kc[c].z, q4.z, dot[h]);
            dot[h] = dot2_bf16(kc[c].w, q4.w, dot[h]);
          }
        } else {
          float x[CE];
          unpack_chunk<T>(kc[c], x);
#pragma unroll
          for (int h = 0; h < G; ++h) {
            const float4 q4 = *reinterpret_cast<const float4 *>(&q_lds[h][c * CE]);
            dot[h] = fmaf(q4.x, x[0], dot[h]);
            dot[h] = fmaf(q4.y, x[1], dot[h]);
            dot[h] = fmaf(q4.z, x[2], dot[h]);
            dot[h] = fmaf(q4.w, x[3], dot[h]);
          }
        }
        if (G >= 8) __builtin_amdgcn_sched_barrier(0);  // bound the hoisted query reads
      }
#pragma unroll
      for (int h = 0; h < G; ++h) s[h] = dot[h] * a.scale_log2;
    }
    if (kZLate) gather_latents();

    // ---- online softmax update (wavefront-uniform running max per head) ----
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
      p_lds[wave][h][lane] = pr;
    }
    wave_lds_sync();

    // ---- latent weighted sum ----
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      if (zv[j]) {
        const int t = j * TG + tg;
        float x[CE];
        unpack_chunk<T>(zc[j], x);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float pr = p_lds[wave][h][t];
#pragma unroll
          for (int ee = 0; ee < CE; ++ee) acc[h][ee] = fmaf(pr, x[ee], acc[h][ee]);
        }
      }
      if (G >= 8) __builtin_amdgcn_sched_barrier(0);  // bound the hoisted probability reads
    }
    wave_lds_sync();
    // keep the next block's gathers from being hoisted into this one (registers)
    __builtin_amdgcn_sched_barrier(0);
  }
  }

  // ---- merge inside the wavefront: token groups in a fixed order ----
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float lw = wave_sum(l_lane[h]);
    if (lane == 0) {
      m_lds[wave][h] = m_run[h];
      l_lds[wave][h] = lw;
    }
  }
  for (int i = lane; i < G * RV; i += kWave) u_lds[wave][i / RV][i % RV] = 0.f;
  wave_lds_sync();
  for (int t = 0; t < TG; ++t) {
    if (tg == t) {
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int ee = 0; ee < CE; ++ee) u_lds[wave][h][vc * CE + ee] += acc[h][ee];
    }
    wave_lds_sync();
  }
  __syncthreads();

  // ---- merge the wavefronts; write u (one split) or this split's record ----
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
    const int64_t row = (int64_t)b * a.n_q + (int64_t)g * G + h;
    if (a.n_split == 1) {
      const float uv = lsum > 0.f ? usum / lsum : 0.f;
      u_out[row * RV + d] = uv;
      if (a.u_tiles) store_u_tiles(a.u_tiles, b, (g * G + h) * RV + d, a.n_q * RV, uv);
    } else {
      float *rp = part + (row * a.n_split + split) * rec;
      store_coherent(rp + 2 + d, usum);
      if (d == 0) {
        store_coherent(rp, M);
        store_coherent(rp + 1, lsum);
      }
    }
  }
  if (a.n_split == 1) return;

  // ---- the last split of the (sequence, KV head) to finish merges them all ----
  //   u = sum_s u_s 2^(m_s - M) / sum_s l_s 2^(m_s - M),  M = max_s m_s,
  // in split order; a head with no valid token gets u = 0.
  if (!last_to_arrive(a.counters + bg, a.n_split)) return;
  constexpr int U = 8;  // records read per batch of loads
  for (int i = threadIdx.x; i < G * RV; i += blockDim.x) {
    const int h = i / RV, d = i % RV;
    const int64_t row = (int64_t)b * a.n_q + (int64_t)g * G + h;
    const float *base = part + row * a.n_split * rec;
    float M = -INFINITY;
    for (int s0 = 0; s0 < a.n_split; s0 += U) {
      float m[U];
#pragma unroll
      for (int k = 0; k < U; ++k)
        m[k] = s0 + k < a.n_split ? load_coherent(base + (s0 + k) * rec) : -INFINITY;
#pragma unroll
      for (int k = 0; k < U; ++k) M = fmaxf(M, m[k]);
    }
    float lsum = 0.f, usum = 0.f;
    if (M != -INFINITY) {
      for (int s0 = 0; s0 < a.n_split; s0 += U) {
        float m[U], l[U], uu[U];
#pragma unroll
        for (int k = 0; k < U; ++k) {
          const bool ok = s0 + k < a.n_split;
          const float *r = base + (s0 + k) * rec;
          m[k] = ok ? load_coherent(r) : -INFINITY;
          l[k] = ok ? load_coherent(r + 1) : 0.f;
          uu[k] = ok ? load_coherent(r + 2 + d) : 0.f;
        }
#pragma unroll
        for (int k = 0; k < U; ++k) {
          const float f = exp2f(m[k] - M);
          lsum = fmaf(l[k], f, lsum);
          usum = fmaf(uu[k], f, usum);
        }
      }
    }
    const float uv = lsum > 0.f ? usum / lsum : 0.f;
    u_out[row * RV + d] = uv;
    if (a.u_tiles) store_u_tiles(a.u_tiles, b, (g * G + h) * RV + d, a.n_q * RV, uv);
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

// Pages per split.  Every wavefront takes up to kAttendBlocks 64-token blocks
// per round; a split is one round when there is work enough for about two
// workgroups per compute unit at that size, otherwise one block per
// wavefront (more, smaller workgroups).  A split grows by whole rounds when
// that would leave more than kMaxSplits splits (the kernel loops over them).
static int pages_per_split(const basiskv_dims &d, int32_t top_k) {
  const int ppi = 64 / d.page_size;
  const int64_t blocks = (int64_t)d.batch * d.n_kv_heads * (((int64_t)top_k + ppi - 1) / ppi);
  const int per_wave = blocks >= (int64_t)kAttendWaves * kAttendBlocks * 512 ? kAttendBlocks : 1;
  const int per_round = kAttendWaves * per_wave * ppi;
  int rounds = 1;
  const int64_t need = ((int64_t)top_k + kMaxSplits - 1) / kMaxSplits;
  if (need > per_round) {
    const int full = kAttendWaves * kAttendBlocks * ppi;  // several rounds: full rounds
    rounds = (int)((need + full - 1) / full);
    return full * rounds;
  }
  return per_round;
}

int attend_splits(const basiskv_dims &d, int32_t top_k) {
  const int pps = pages_per_split(d, top_k);
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
                         int32_t *counters, uint16_t *u_tiles, hipStream_t s, bool *unsupported) {
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
  a.pages_per_split = pages_per_split(d, top_k);
  a.n_split = attend_splits(d, top_k);
  a.total = d.batch * d.n_kv_heads * a.n_split;
  a.padded = (a.total + kXcds - 1) / kXcds * kXcds;
  a.scale_log2 = scale * kLog2e;
  a.counters = counters;
  a.u_tiles = u_tiles;
  void *args[] = {(void *)&q,           (void *)&c.k_pages,  (void *)&c.z_pages,
                  (void *)&c.block_table, (void *)&c.seq_lens, (void *)&sel,
                  (void *)&part,        (void *)&u,          (void *)&a};
  return hipLaunchKernel(fn, dim3(a.padded), dim3(256), args, 0, s);
}

}  // namespace bkv_host
