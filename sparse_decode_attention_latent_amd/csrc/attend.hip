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
// RoPE kernels hold one wavefront per SIMD (1024 on the chip) and are also
// built with three blocks per wavefront: rows of a little over one block per
// SIMD (the adopted router: 2176 blocks) then take three block times instead
// of a second round of two-block wavefronts (four).  The launch picks the
// block count (pages_per_split).
constexpr int kAttendRopeBlocks = 3;

struct AttendArgs {
  int n_q, n_kv, max_pages, num_phys, page_size, log2_page, cap, top_k;
  int recent;     // recent-window tokens (0: none)
  int all_pages;  // dense attention: entry e is page e (no selection)
  int n_entries;  // entries per row: top_k routed, then the recent window's pages
  int gs;  // query subgroups per KV head (the kernel's group is n_q / n_kv / gs heads)
  int pages_per_split, n_split, total, padded;
  float scale_log2;  // scale * log2(e): exponentials are taken base 2
  int32_t *counters;  // [batch * n_kv * gs], zero between calls (see the merge)
  uint16_t *u_tiles;  // optional: u also written as the reconstruction's A operand (bf16)
  PoolGeom geom;      // latent chunk positions within a page of the latent pool
  const float *rope;  // RoPE inverse frequencies [head_dim / 2] (ROPE kernels only)
};

// Partial record per (b, h, split): [m, l, u[0..r_v)] with m in base-2 logit
// units (scale * log2 e already applied), l = sum 2^(s - m), u = sum 2^(s - m) z.
//
// Each wavefront owns up to NB 64-token blocks of the split per round (NB is
// 1, or kAttendBlocks when the split is that long); their
// selection entries and block-table rows are requested before the queries are
// staged, so the chain selection -> block table -> Key gather costs its
// latency once per wavefront rather than once per block.
//
// bf16: the scores of a query group of 2 to 8 heads run on the 4x4x4 bf16
// matrix instruction (16 independent 4x4 products per wavefront: lane l
// supplies 4 Key dims of its own token and receives its token's scores for
// four heads, so the one-token-per-lane layout carries through), and the
// next block's Key and latent chunks are requested as soon as the current
// block has consumed the registers they land in, so the gathers of block
// i + 1 are in flight while block i is scored and summed.
// float32: the scores are float32 FMAs against the queries held in LDS, and
// each block is gathered when it starts (latents after the scores: their
// registers would not fit beside the Key).
// Wavefronts per SIMD the register budget is sized for: two, except for the
// widest bf16 groups, whose streamed Key (64) and latent (4 per token group)
// registers and accumulators (8 per head) come to 170 or more of the 256,
// leaving too few for the rest, and for float32 (a 128-register Key): these
// take one wavefront per SIMD and its whole register file.  (E4M3 pages:
// the Key takes 32 registers, the accumulators 16 per head.)
// (RoPE kernels, whose rotation keeps the Key and its angles live, take one
// wavefront per SIMD too.)
template <typename C, int G, int NVC, bool ROPE = false>
constexpr int attend_waves_per_eu() {
  constexpr int nj = (kWave + kWave / NVC - 1) / (kWave / NVC);
  constexpr int ce = Elem<C>::CE;
  return ROPE || sizeof(C) == 4 || (kHeadDim / ce) * 4 + 4 * nj + ce * G >= 170
             ? 1 : BKV_ATTEND_WAVES_PER_EU;
}

typedef short attend_s4 __attribute__((ext_vector_type(4)));
typedef float attend_f4 __attribute__((ext_vector_type(4)));

// T: query elements (float32 or bf16); C: cache elements (float32, bf16, or
// E4M3 codes beside bf16 queries, whose Key chunks are widened to bf16 -- exact
// -- for the same matrix instruction).  STREAM: page gathers marked non-temporal
// (used where every load instruction reads whole 128-byte lines and no other
// workgroup reads the same pages: pages of 8 or more tokens, one query
// subgroup per KV head).
// ROPE: the cached Keys are pre-RoPE; each is rotated to its token's position
// (rotate-half pairs d, d + head_dim / 2, which a lane holds in chunks c and
// c + NKC / 2) before the float32 scores.
template <typename T, typename C, int G, int NVC, int NB, bool STREAM, bool ROPE = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(attend_waves_per_eu<C, G, NVC, ROPE>())))
void attend_split_kernel(
    const T *__restrict__ q, const C *__restrict__ kpool, const C *__restrict__ zpool,
    const int32_t *__restrict__ block_table, const int32_t *__restrict__ seq_lens,
    const int32_t *__restrict__ sel, float *__restrict__ part, float *__restrict__ u_out,
    AttendArgs a) {
  constexpr int CE = Elem<C>::CE;     // cache elements per 16-byte chunk
  constexpr int NKC = kHeadDim / CE;  // Key chunks per token
  constexpr int RV = NVC * CE;        // latent width
  constexpr int TG = kWave / NVC;     // token groups in the latent phase
  constexpr int NJ = (kWave + TG - 1) / TG;
  constexpr int NW = kAttendWaves;
  constexpr bool kBf = sizeof(T) == 2;
  constexpr bool kFp8 = sizeof(C) == 1;
  static_assert(sizeof(C) == sizeof(T) || (kBf && kFp8), "E4M3 pages go with bf16 queries");
  constexpr bool kMfma = kBf && !ROPE;   // scores on the matrix cores
  constexpr bool kStream = kBf && !ROPE; // next block's gathers overlap this block
  constexpr int QG = (G + 3) / 4;        // head quads (matrix-instruction row sets)
  constexpr int NQC = kHeadDim / 8;      // 8-dim bf16 query chunks

  // queries: matrix operands [quad][8-dim chunk][head in quad][8 dims] (bf16),
  // else [head][dims] (float32)
  __shared__ __align__(16) uint4 qa_lds[kMfma ? QG * NQC * 4 : 1];
  __shared__ __align__(16) float q_lds[kMfma ? 1 : G][kMfma ? 4 : kHeadDim];
  __shared__ double w_lds[ROPE ? kHeadDim / 2 : 1];  // RoPE frequencies, turns per position
  __shared__ float p_lds[NW][G][kWave];
  __shared__ float m_lds[NW][G];
  __shared__ float l_lds[NW][G];
  // token-group sums of HC heads at a time (the merge walks the group in passes)
  constexpr int HC = (32768 / (NW * TG * RV * 4)) < 1 ? 1
                     : (32768 / (NW * TG * RV * 4)) > G ? G : (32768 / (NW * TG * RV * 4));
  static_assert(G % HC == 0, "head passes must tile the group");
  __shared__ __align__(16) float u_part[NW][TG][HC][RV];

  const int work = xcd_work_index(a.padded);
  if (work >= a.total) return;  // uniform per workgroup
  // work item = (sequence, query subgroup, split); subgroup gv holds query
  // heads gv G .. gv G + G - 1 and reads KV head g = gv / gs
  const int bv = work / a.n_split;
  const int split = work - bv * a.n_split;
  const int nv = a.n_kv * a.gs;
  const int b = bv / nv, gv = bv - b * nv;
  const int g = gv / a.gs;
  const int bg = b * a.n_kv + g;

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;
  const int slot = lane & (a.page_size - 1);
  const int ppi = kWave >> a.log2_page;  // pages per 64-token block
  const int e_begin = split * a.pages_per_split;
  const int e_end = min(a.n_entries, e_begin + a.pages_per_split);
  const int n_blocks = (e_end - e_begin + ppi - 1) / ppi;
  const int32_t *sel_bg = a.all_pages ? sel : sel + (int64_t)bg * a.top_k;
  const int32_t *bt = block_table + (int64_t)b * a.max_pages;

  // ---- this wavefront's blocks of round r: selection entries, then physical pages ----
  const int L = clamp_len(seq_lens[b], a.cap);
  const int NP = (L + a.page_size - 1) >> a.log2_page;
  // entries past top_k are the recent window's pages, from first_recent on
  const int first_recent = max(0, L - a.recent) >> a.log2_page;
  const int n_rounds = (n_blocks + NW * NB - 1) / (NW * NB);
  int page[NB], phys[NB];
  auto fetch_pages = [&](int r) {
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int blk = (r * NB + i) * NW + wave;
      const int e = e_begin + blk * ppi + (lane >> a.log2_page);
      const int pr = first_recent + (e - a.top_k);
      int pg = -1;
      if (blk < n_blocks && e < e_end) {
        if (a.all_pages) pg = e < NP ? e : -1;
        else pg = e < a.top_k ? sel_bg[e] : (pr < NP ? pr : -1);
      }
      page[i] = pg;
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      phys[i] = -1;
      if (page[i] >= 0 && page[i] < NP) phys[i] = bt[page[i]];
    }
  };
  fetch_pages(0);

  // ---- the group's queries into LDS ----
  {
    const T *qg = q + ((int64_t)b * a.n_q + (int64_t)gv * G) * kHeadDim;
    if constexpr (kMfma) {
      // entry (quad, chunk c, head hq): dims 8c .. 8c + 7 of head 4 quad + hq (zero past G)
      for (int i = threadIdx.x; i < QG * NQC * 4; i += blockDim.x) {
        const int hq = i & 3, c = (i >> 2) % NQC, qd = i / (NQC * 4);
        const int h = qd * 4 + hq;
        qa_lds[i] = h < G ? *reinterpret_cast<const uint4 *>(qg + h * kHeadDim + c * 8)
                          : make_uint4(0u, 0u, 0u, 0u);
      }
    } else if constexpr (ROPE) {  // float32 queries, and the rotation's frequencies
      for (int i = threadIdx.x; i < G * kHeadDim; i += blockDim.x)
        q_lds[i / kHeadDim][i % kHeadDim] = to_f32(qg[i]);
      for (int i = threadIdx.x; i < kHeadDim / 2; i += blockDim.x)
        w_lds[i] = (double)a.rope[i] * 0.15915494309189535;  // 1 / (2 pi)
    } else {
      constexpr int QW = G * kHeadDim * (int)sizeof(T) / 4;  // 32-bit words
      constexpr int QL = (QW + 255) / 256;
      const uint32_t *qw_g = reinterpret_cast<const uint32_t *>(qg);
      uint32_t *qw = reinterpret_cast<uint32_t *>(&q_lds[0][0]);
      uint32_t qv[QL];
#pragma unroll
      for (int u = 0; u < QL; ++u) {
        const int i = u * 256 + threadIdx.x;
        if (i < QW) qv[u] = qw_g[i];
      }
#pragma unroll
      for (int u = 0; u < QL; ++u) {
        const int i = u * 256 + threadIdx.x;
        if (i < QW) qw[i] = qv[u];
      }
    }
  }
  __syncthreads();

  const int64_t head_page0 = (int64_t)g * a.num_phys;
  const int64_t kpage_bytes = (int64_t)NKC * a.page_size * 16;
  const int64_t zpage_bytes = (int64_t)a.geom.z_page_chunks * a.page_size * 16;
  const int64_t chunk_stride = (int64_t)a.page_size * 16;

  // latent-phase lane roles: chunk vc of tokens t = j * TG + tg
  const int vc = lane % NVC;
  const int tg = lane / NVC;

  auto lane_valid = [&](int i) {
    const int tok = page[i] * a.page_size + slot;
    return page[i] >= 0 && page[i] < NP && tok < L && phys[i] >= 0 && phys[i] < a.num_phys;
  };
  // block (r, i) is wavefront-uniformly present or absent
  auto block_live = [&](int r, int i) { return (r * NB + i) * NW + wave < n_blocks; };

  // byte offset of this lane's Key in block i
  auto k_off = [&](int i) {
    return (head_page0 + phys[i]) * kpage_bytes + (int64_t)slot * 16;
  };
  // latent chunk j of block i: token t = j * TG + tg, whose page lives in lane t;
  // returns whether this lane loads it, and from where
  auto z_src = [&](int i, bool v, int j, int64_t &off) {
    const int t = j * TG + tg;
    const bool role = tg < TG && t < kWave;
    const int src = role ? t : 0;
    const int phys_t = __shfl(phys[i], src);
    const int valid_t = __shfl((int)v, src);
    off = (head_page0 + phys_t) * zpage_bytes + z_chunk_slot(a.geom, vc) * chunk_stride +
          (int64_t)(src & (a.page_size - 1)) * 16;
    return role && valid_t != 0;
  };

  // gather registers: streamed (bf16) they carry block i + 1's chunks while
  // block i finishes; a lane with no valid token scores whatever they hold
  // and masks the result
  uint4 kc[NKC], zc[NJ];
  bool zv[NJ];
  if constexpr (kStream) {
#pragma unroll
    for (int c = 0; c < NKC; ++c) kc[c] = make_uint4(0u, 0u, 0u, 0u);
  }

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
  if constexpr (kStream) {  // the round's first block; later ones are requested by their predecessor
    const bool v0 = lane_valid(0);
    const int64_t ko = k_off(0);
#pragma unroll
    for (int c = 0; c < NKC; ++c)
      if (v0) kc[c] = load_page_chunk<STREAM>(kpool, ko + c * chunk_stride);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      int64_t zo;
      zv[j] = z_src(0, v0, j, zo);
      if (zv[j]) zc[j] = load_page_chunk<STREAM>(zpool, zo);
    }
  }
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    if (!block_live(r, i)) break;  // wavefront-uniform
    const bool valid = lane_valid(i);
    const bool nxt = kStream && i + 1 < NB && block_live(r, i + 1);  // wavefront-uniform
    const int inx = i + 1 < NB ? i + 1 : i;
    const bool vn = nxt && lane_valid(inx);
    const int64_t ko_next = k_off(inx);
    if constexpr (!kStream) {
      const int64_t ko = k_off(i);
#pragma unroll
      for (int c = 0; c < NKC; ++c)
        if (valid) kc[c] = load_page_chunk<STREAM>(kpool, ko + c * chunk_stride);
    }

    // ---- exact scores, one token per lane ----
    float s[G];
    if constexpr (kMfma) {
      attend_f4 sc[QG][2];
#pragma unroll
      for (int qd = 0; qd < QG; ++qd) sc[qd][0] = sc[qd][1] = attend_f4{0.f, 0.f, 0.f, 0.f};
      const int hq = lane & 3;
#pragma unroll
      for (int c = 0; c < NKC; ++c) {
        // this Key chunk as 8-dim bf16 chunks (E4M3: two, widened exactly)
        constexpr int SUB = kFp8 ? 2 : 1;
        uint4 kb[SUB];
        if constexpr (kFp8) {
          kb[0] = fp8x8_to_bf16x8(kc[c].x, kc[c].y);
          kb[SUB - 1] = fp8x8_to_bf16x8(kc[c].z, kc[c].w);
          if (nxt && vn) kc[c] = load_page_chunk<STREAM>(kpool, ko_next + c * chunk_stride);  // registers free again
        } else {
          kb[0] = kc[c];
        }
#pragma unroll
        for (int sb = 0; sb < SUB; ++sb) {
          const attend_s4 klo = __builtin_bit_cast(attend_s4, make_uint2(kb[sb].x, kb[sb].y));
          const attend_s4 khi = __builtin_bit_cast(attend_s4, make_uint2(kb[sb].z, kb[sb].w));
#pragma unroll
          for (int qd = 0; qd < QG; ++qd) {
            const uint4 qv = qa_lds[(qd * NQC + c * SUB + sb) * 4 + hq];
            const attend_s4 qlo = __builtin_bit_cast(attend_s4, make_uint2(qv.x, qv.y));
            const attend_s4 qhi = __builtin_bit_cast(attend_s4, make_uint2(qv.z, qv.w));
            sc[qd][0] = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(qlo, klo, sc[qd][0], 0, 0, 0);
            sc[qd][1] = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(qhi, khi, sc[qd][1], 0, 0, 0);
          }
        }
        if constexpr (!kFp8)
          if (nxt && vn) kc[c] = load_page_chunk<STREAM>(kpool, ko_next + c * chunk_stride);  // registers free again
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float dot = sc[h / 4][0][h % 4] + sc[h / 4][1][h % 4];
        s[h] = valid ? dot * a.scale_log2 : -INFINITY;
      }
    } else if constexpr (ROPE) {
#pragma unroll
      for (int h = 0; h < G; ++h) s[h] = -INFINITY;
      if (valid) {
        const double pos = (double)(page[i] * a.page_size + slot);  // the token's position
        constexpr int HALF = NKC / 2;
        float dot[G];
#pragma unroll
        for (int h = 0; h < G; ++h) dot[h] = 0.f;
#pragma unroll
        for (int c = 0; c < HALF; ++c) {
          float x[CE], y[CE];
          unpack_chunk<C>(kc[c], x);
          unpack_chunk<C>(kc[c + HALF], y);
#pragma unroll
          for (int e = 0; e < CE; ++e) {
            const int d = c * CE + e;
            float sn, cs;
            rope_sincos_turns(pos, w_lds[d], sn, cs);
            const float xr = x[e] * cs - y[e] * sn;
            const float yr = x[e] * sn + y[e] * cs;
#pragma unroll
            for (int h = 0; h < G; ++h)
              dot[h] = fmaf(q_lds[h][d], xr, fmaf(q_lds[h][d + kHeadDim / 2], yr, dot[h]));
          }
        }
#pragma unroll
        for (int h = 0; h < G; ++h) s[h] = dot[h] * a.scale_log2;
      }
    } else {
#pragma unroll
      for (int h = 0; h < G; ++h) s[h] = -INFINITY;
      float dot[G];
#pragma unroll
      for (int h = 0; h < G; ++h) dot[h] = 0.f;
      // (float32: only lanes with a valid token, which have gathered this block)
#pragma unroll
      for (int c = 0; c < NKC; ++c) {
        if constexpr (kBf) {
          const uint32_t *qw = reinterpret_cast<const uint32_t *>(&q_lds[0][0]);
#pragma unroll
          for (int h = 0; h < G; ++h) {
            const uint4 q4 = *reinterpret_cast<const uint4 *>(qw + h * (kHeadDim / 2) + c * 4);
            dot[h] = dot2_bf16(kc[c].x, q4.x, dot[h]);
            dot[h] = dot2_bf16(kc[c].y, q4.y, dot[h]);
            dot[h] = dot2_bf16(kc[c].z, q4.z, dot[h]);
            dot[h] = dot2_bf16(kc[c].w, q4.w, dot[h]);
          }
          if (nxt && vn) kc[c] = load_page_chunk<STREAM>(kpool, ko_next + c * chunk_stride);
        } else if (valid) {
          float x[CE];
          unpack_chunk<C>(kc[c], x);
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
      if (valid) {
#pragma unroll
        for (int h = 0; h < G; ++h) s[h] = dot[h] * a.scale_log2;
      }
    }
    if constexpr (!kStream) {
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        int64_t zo;
        zv[j] = z_src(i, valid, j, zo);
        if (zv[j]) zc[j] = load_page_chunk<STREAM>(zpool, zo);
      }
    }

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

    // ---- latent weighted sum; each chunk's registers then take block i + 1's ----
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      if (zv[j]) {
        const int t = j * TG + tg;
        float x[CE];
        unpack_chunk<C>(zc[j], x);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float pr = p_lds[wave][h][t];
#pragma unroll
          for (int ee = 0; ee < CE; ++ee) acc[h][ee] = fmaf(pr, x[ee], acc[h][ee]);
        }
      }
      if (nxt) {
        int64_t zo;
        zv[j] = z_src(inx, vn, j, zo);
        if (zv[j]) zc[j] = load_page_chunk<STREAM>(zpool, zo);
      }
      if (G >= 8) __builtin_amdgcn_sched_barrier(0);  // bound the hoisted probability reads
    }
    wave_lds_sync();
    // keep the next block's work from being hoisted into this one (registers)
    __builtin_amdgcn_sched_barrier(0);
  }
  }

  // ---- per-wavefront softmax state into LDS ----
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float lw = wave_sum(l_lane[h]);
    if (lane == 0) {
      m_lds[wave][h] = m_run[h];
      l_lds[wave][h] = lw;
    }
  }

  // ---- per pass of HC heads: the token groups' sums into LDS, then token
  // groups and wavefronts merged in a fixed order; u written (one split) or
  // this split's record ----
  const int rec = RV + 2;
#pragma unroll
  for (int h0 = 0; h0 < G; h0 += HC) {
    if (h0 > 0) __syncthreads();  // the previous pass has read u_part
    if (tg < TG) {
#pragma unroll
      for (int hh = 0; hh < HC; ++hh) {
        float *dst = &u_part[wave][tg][hh][vc * CE];
#pragma unroll
        for (int ee = 0; ee < CE; ee += 4)
          *reinterpret_cast<float4 *>(dst + ee) = make_float4(
              acc[h0 + hh][ee], acc[h0 + hh][ee + 1], acc[h0 + hh][ee + 2], acc[h0 + hh][ee + 3]);
      }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < HC * RV; i += blockDim.x) {
      const int hh = i / RV, d = i % RV, h = h0 + hh;
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < NW; ++w) M = fmaxf(M, m_lds[w][h]);
      float lsum = 0.f, usum = 0.f;
      if (M != -INFINITY) {
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          float uw = 0.f;
#pragma unroll
          for (int t = 0; t < TG; ++t) uw += u_part[w][t][hh][d];
          const float f = exp2f(m_lds[w][h] - M);
          lsum = fmaf(l_lds[w][h], f, lsum);
          usum = fmaf(uw, f, usum);
        }
      }
      const int64_t row = (int64_t)b * a.n_q + (int64_t)gv * G + h;
      if (a.n_split == 1) {
        const float uv = lsum > 0.f ? usum / lsum : 0.f;
        u_out[row * RV + d] = uv;
        if (a.u_tiles) store_u_tiles(a.u_tiles, b, (gv * G + h) * RV + d, a.n_q * RV, uv);
      } else {
        float *rp = part + (row * a.n_split + split) * rec;
        store_coherent(rp + 2 + d, usum);
        if (d == 0) {
          store_coherent(rp, M);
          store_coherent(rp + 1, lsum);
        }
      }
    }
  }
  if (a.n_split == 1) return;

  // ---- the last split of the (sequence, query subgroup) to finish merges them all ----
  //   u = sum_s u_s 2^(m_s - M) / sum_s l_s 2^(m_s - M),  M = max_s m_s,
  // in split order (running maximum per batch of records, earlier sums
  // rescaled when it grows); a head with no valid token gets u = 0.  Every
  // thread requests the records of all its outputs before combining any.
  if (!last_to_arrive(a.counters + bv, a.n_split)) return;
  constexpr int NT = NW * kWave;
  constexpr int NI = (G * RV + NT - 1) / NT;     // outputs per thread
  constexpr int U = 16 / NI < 4 ? 4 : 16 / NI;   // records per batch of loads
  float Mx[NI], lsum[NI], usum[NI];
#pragma unroll
  for (int n = 0; n < NI; ++n) {
    Mx[n] = -INFINITY;
    lsum[n] = usum[n] = 0.f;
  }
  for (int s0 = 0; s0 < a.n_split; s0 += U) {
    float m[NI][U], l[NI][U], uu[NI][U];
#pragma unroll
    for (int n = 0; n < NI; ++n) {
      const int i = n * NT + threadIdx.x;
      const int h = i / RV, d = i % RV;
      const float *base = part + ((int64_t)b * a.n_q + (int64_t)gv * G + h) * a.n_split * rec;
#pragma unroll
      for (int k = 0; k < U; ++k) {
        const bool ok = i < G * RV && s0 + k < a.n_split;
        const float *r = base + (s0 + k) * rec;
        m[n][k] = ok ? load_coherent(r) : -INFINITY;
        l[n][k] = ok ? load_coherent(r + 1) : 0.f;
        uu[n][k] = ok ? load_coherent(r + 2 + d) : 0.f;
      }
    }
#pragma unroll
    for (int n = 0; n < NI; ++n) {
      float Mb = Mx[n];
#pragma unroll
      for (int k = 0; k < U; ++k) Mb = fmaxf(Mb, m[n][k]);
      if (Mb != -INFINITY) {
        const float f0 = exp2f(Mx[n] - Mb);  // 0 while the maximum is -inf
        lsum[n] *= f0;
        usum[n] *= f0;
#pragma unroll
        for (int k = 0; k < U; ++k) {
          const float f = exp2f(m[n][k] - Mb);
          lsum[n] = fmaf(l[n][k], f, lsum[n]);
          usum[n] = fmaf(uu[n][k], f, usum[n]);
        }
        Mx[n] = Mb;
      }
    }
  }
#pragma unroll
  for (int n = 0; n < NI; ++n) {
    const int i = n * NT + threadIdx.x;
    if (i < G * RV) {
      const int h = i / RV, d = i % RV;
      const int64_t row = (int64_t)b * a.n_q + (int64_t)gv * G + h;
      const float uv = lsum[n] > 0.f ? usum[n] / lsum[n] : 0.f;
      u_out[row * RV + d] = uv;
      if (a.u_tiles) store_u_tiles(a.u_tiles, b, (gv * G + h) * RV + d, a.n_q * RV, uv);
    }
  }
}

struct AttendVariant {
  int dtype, G, rv;
  const void *fn1, *fn;  // one block per wavefront and round; kAttendBlocks
  const void *fn_nt;     // kAttendBlocks with non-temporal gathers (null: not built)
  const void *fn3;       // kAttendRopeBlocks (RoPE kernels; null otherwise)
};

// non-temporal variants for the 4-head kernels (the 8B-shaped group, and the
// halves of split 8-head groups), whose gathers are long streams
#define BKV_ATT(T, C, DT, G, RV)                                                                 \
  {DT, G, RV,                                                                                    \
   reinterpret_cast<const void *>(&attend_split_kernel<T, C, G, (RV) / Elem<C>::CE, 1, false>), \
   reinterpret_cast<const void *>(                                                               \
       &attend_split_kernel<T, C, G, (RV) / Elem<C>::CE, kAttendBlocks, false>),                 \
   (G) == 4 ? reinterpret_cast<const void *>(                                                    \
                  &attend_split_kernel<T, C, G, (RV) / Elem<C>::CE, kAttendBlocks, ((G) == 4)>)  \
            : nullptr,                                                                           \
   nullptr}
#define BKV_ATT_G(T, C, DT, RV)                                                  \
  BKV_ATT(T, C, DT, 1, RV), BKV_ATT(T, C, DT, 2, RV), BKV_ATT(T, C, DT, 4, RV), \
      BKV_ATT(T, C, DT, 8, RV)

// (r_v = 128 serves the dense baseline, which sums Values in the latent's place)
static const AttendVariant kAttendVariants[] = {
    BKV_ATT_G(uint16_t, uint16_t, BASISKV_BF16, 64),
    BKV_ATT_G(uint16_t, uint16_t, BASISKV_BF16, 96),
    BKV_ATT_G(uint16_t, uint16_t, BASISKV_BF16, 32),
    BKV_ATT_G(uint16_t, uint16_t, BASISKV_BF16, 128),
    BKV_ATT_G(float, float, BASISKV_F32, 64),
    BKV_ATT_G(float, float, BASISKV_F32, 32),
    BKV_ATT_G(uint16_t, uint8_t, BASISKV_BF16_FP8_E4M3, 64),
    BKV_ATT_G(uint16_t, uint8_t, BASISKV_BF16_FP8_E4M3, 96),
    BKV_ATT_G(uint16_t, uint8_t, BASISKV_BF16_FP8_E4M3, 128),
};

// RoPE variants: pre-RoPE Keys rotated to their positions (float32 scores)
#define BKV_ATT_ROPE(T, C, DT, G, RV)                                                                 \
  {DT, G, RV,                                                                                         \
   reinterpret_cast<const void *>(&attend_split_kernel<T, C, G, (RV) / Elem<C>::CE, 1, false, true>), \
   reinterpret_cast<const void *>(                                                                    \
       &attend_split_kernel<T, C, G, (RV) / Elem<C>::CE, kAttendBlocks, false, true>),                \
   nullptr,                                                                                           \
   reinterpret_cast<const void *>(                                                                    \
       &attend_split_kernel<T, C, G, (RV) / Elem<C>::CE, kAttendRopeBlocks, false, true>)}
static const AttendVariant kAttendRopeVariants[] = {
    BKV_ATT_ROPE(uint16_t, uint16_t, BASISKV_BF16, 4, 64),
    BKV_ATT_ROPE(uint16_t, uint16_t, BASISKV_BF16, 4, 96),
    BKV_ATT_ROPE(uint16_t, uint16_t, BASISKV_BF16, 8, 64),
    BKV_ATT_ROPE(uint16_t, uint8_t, BASISKV_BF16_FP8_E4M3, 4, 64),
    BKV_ATT_ROPE(uint16_t, uint8_t, BASISKV_BF16_FP8_E4M3, 4, 96),
    BKV_ATT_ROPE(uint16_t, uint8_t, BASISKV_BF16_FP8_E4M3, 8, 64),
};

}  // namespace bkv

namespace bkv_host {
using namespace bkv;

static int ilog2i(int x) {
  int l = 0;
  while ((1 << l) < x) ++l;
  return l;
}

// Query subgroups per KV head.  A bf16 group of 8 heads with latents of 96 or
// more dims is taken as two groups of 4 sharing the KV head's pages: the
// 8-head kernel needs the whole register file (one wavefront per SIMD, little
// latency hiding), two 4-head wavefronts fit two per SIMD and each does half
// the arithmetic, at the price of gathering the pages twice (the second time
// mostly from cache).
int attend_group_split(const basiskv_dims &d) {
  const int G = d.n_q_heads / d.n_kv_heads;
  return act_bf16(d) && G == 8 && d.r_v >= 96 ? 2 : 1;
}

// Pages per split and 64-token blocks per wavefront and round (nb).  A split
// is kAttendWaves wavefronts x nb blocks, grown by whole rounds when that would
// leave more than kMaxSplits splits (the kernel loops over them).  Position-free
// kernels take kAttendBlocks blocks when one block per wavefront would need more
// wavefronts than the chip holds at once (two per SIMD: 2048), which would leave
// a second, partial round waiting for the first, and one block otherwise (more,
// smaller workgroups).  RoPE kernels (one wavefront per SIMD: 1024) take the
// block count among 1, kAttendBlocks and kAttendRopeBlocks with the fewest block
// times -- rounds of resident wavefronts x blocks per wavefront and round x
// rounds per split -- and, of equals, the fewest splits.
#ifndef BKV_ATTEND_RESIDENT_WAVES
#define BKV_ATTEND_RESIDENT_WAVES 2048
#endif
struct SplitPlan {
  int nb, pages;
};
static SplitPlan split_plan_for(const basiskv_dims &d, int32_t entries, int nb) {
  const int ppi = 64 / d.page_size;
  const int per_round = kAttendWaves * nb * ppi;
  const int64_t need = ((int64_t)entries + kMaxSplits - 1) / kMaxSplits;
  const int rounds = need > per_round ? (int)((need + per_round - 1) / per_round) : 1;
  return {nb, per_round * rounds};
}
static SplitPlan split_plan(const basiskv_dims &d, int32_t entries, bool rope) {
  const int ppi = 64 / d.page_size;
  const int64_t rows = (int64_t)d.batch * d.n_kv_heads * attend_group_split(d);
  const int64_t blocks = rows * (((int64_t)entries + ppi - 1) / ppi);
  const int64_t need = ((int64_t)entries + kMaxSplits - 1) / kMaxSplits;
  if (!rope) {
    const int nb = blocks > BKV_ATTEND_RESIDENT_WAVES || need > kAttendWaves * ppi ? kAttendBlocks : 1;
    return split_plan_for(d, entries, nb);
  }
  const int64_t resident = BKV_ATTEND_RESIDENT_WAVES / 2;
  SplitPlan best{0, 0};
  int64_t best_t = 0, best_s = 0;
  for (int nb : {1, kAttendBlocks, kAttendRopeBlocks}) {
    const SplitPlan p = split_plan_for(d, entries, nb);
    const int64_t splits = ((int64_t)entries + p.pages - 1) / p.pages;
    const int64_t waves = rows * splits * kAttendWaves;
    const int64_t t = (waves + resident - 1) / resident * p.pages / (kAttendWaves * ppi);
    if (best.nb == 0 || t < best_t || (t == best_t && splits < best_s)) {
      best = p;
      best_t = t;
      best_s = splits;
    }
  }
  return best;
}

// Entries of one row: the top_k routed pages, then room for the recent
// window's pages (ceil(W / page_size) + 1: the window may start mid-page).
static int attend_entries(const basiskv_dims &d, int32_t top_k) {
  if (d.recent_tokens <= 0) return top_k;
  const int w = d.recent_tokens < d.max_pages_per_seq * d.page_size
                    ? d.recent_tokens : d.max_pages_per_seq * d.page_size;
  return top_k + (w + d.page_size - 1) / d.page_size + 1;
}

// Splits per row: the larger of the two kernels' counts (the workspace is
// sized from dims alone, before it is known whether the cache has positions)
int attend_splits(const basiskv_dims &d, int32_t top_k) {
  const int n = attend_entries(d, top_k);
  const int pa = split_plan(d, n, false).pages, pb = split_plan(d, n, true).pages;
  const int sa = (n + pa - 1) / pa, sb = (n + pb - 1) / pb;
  return sa > sb ? sa : sb;
}

static const AttendVariant *find_attend(const basiskv_dims &d, bool rope) {
  const int G = d.n_q_heads / d.n_kv_heads;
  const int gs = attend_group_split(d);
  if (rope) {
    for (const auto &v : kAttendRopeVariants)
      if (v.dtype == d.dtype && v.G == G / gs && v.rv == d.r_v) return &v;
    return nullptr;
  }
  for (const auto &v : kAttendVariants)
    if (v.dtype == d.dtype && v.G == G / gs && v.rv == d.r_v) return &v;
  return nullptr;
}

bool attend_supported(const basiskv_dims &d, bool rope) { return find_attend(d, rope) != nullptr; }

hipError_t launch_attend(const basiskv_dims &d, const void *q, const basiskv_cache &c,
                         const int32_t *sel, int32_t top_k, float scale, float *u, float *part,
                         int32_t *counters, uint16_t *u_tiles, hipStream_t s, bool *unsupported) {
  const bool rope = sel != nullptr && c.rope_inv_freq != nullptr;  // (the dense baseline has none)
  const AttendVariant *v = find_attend(d, rope);
  if (!v) {
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
  // no selection given: dense attention over every page of the sequence
  a.all_pages = sel == nullptr;
  if (a.all_pages) top_k = d.max_pages_per_seq;
  a.top_k = top_k;
  a.recent = a.all_pages ? 0 : d.recent_tokens;
  a.n_entries = a.all_pages ? top_k : attend_entries(d, top_k);
  a.gs = attend_group_split(d);
  const SplitPlan plan = split_plan(d, a.n_entries, rope);
  a.pages_per_split = plan.pages;
  a.n_split = (a.n_entries + a.pages_per_split - 1) / a.pages_per_split;
  a.total = d.batch * d.n_kv_heads * a.gs * a.n_split;
  a.padded = (a.total + kXcds - 1) / kXcds * kXcds;
  a.scale_log2 = scale * kLog2e;
  a.counters = counters;
  a.u_tiles = u_tiles;
  a.geom = pool_geom(d);
  a.rope = rope ? c.rope_inv_freq : nullptr;
  void *args[] = {(void *)&q,           (void *)&c.k_pages,  (void *)&c.z_pages,
                  (void *)&c.block_table, (void *)&c.seq_lens, (void *)&sel,
                  (void *)&part,        (void *)&u,          (void *)&a};
  // a split of at most one block per wavefront takes the one-block kernel;
  // non-temporal gathers when the launch is a long stream (the two-block
  // kernel: measured slower on the short launches, whose time is latency),
  // each load instruction reads whole 128-byte lines and no other subgroup
  // reads the same pages
  const bool one = plan.nb == 1;
  const bool nt = v->fn_nt && plan.nb == kAttendBlocks && a.gs == 1 && d.page_size >= 8;
  const void *fn = nt ? v->fn_nt : one ? v->fn1 : plan.nb == kAttendBlocks ? v->fn : v->fn3;
  if (!fn) {
    *unsupported = true;
    return hipSuccess;
  }
  return hipLaunchKernel(fn, dim3(a.padded), dim3(256), args, 0, s);
}

}  // namespace bkv_host
