// Device bodies shared by separate launches and by the fused decode-step
// launch: the one-token compression of new tokens (a0) and the routing
// projection of the queries (a1).  BasisKV (arXiv 2611.02583): abstract (the
// Value kept only as a low-rank latent, a Key-specific residual for what the
// latent cannot predict, routing from the latent plus the residual) and
// appendix Table 4 (the three cached states; routing read widths).
#pragma once

#include "common.hpp"

namespace bkv {

// ---------------------------------------------------------------------------
// (a0) for a handful of new tokens (the per-step decode append): the same
// compression as the prefill MFMA kernel as three float32 matrix-vector
// products per (token, KV head):
//   z = v A_g,  z_s = round(z);  r = (k - z_s[:r_b] P_g) E_g,  r_s = round(r)
// and the stores of z_s, r_s and k into their pages.  With one or a few rows
// per head, staging the factors for MFMA costs more than it saves; here every
// workgroup requests all of its head's factor chunks at once (they come from
// L2 after the first sequence), so the body costs one memory round trip plus
// three LDS reductions.
// ---------------------------------------------------------------------------
struct AppendArgs {
  int n_tokens, n_kv, rv, rb, rq, max_pages, num_phys, page_size, cap;
  PoolGeom geom;  // chunk positions of the latent and residual pages
};

// Sums over the slices of a phase.  Lane l of a wavefront holds the partial
// of chunk l % cp over one slice (cp a power of two): the wavefront's slices
// are summed by butterflies over the lanes l ^ cp, l ^ 2 cp, ..., after which
// lanes l < cp hold the wavefront's sums; those go to red[wave], and after a
// barrier output n is red[0][n] + red[1][n] + red[2][n] + red[3][n].
template <int CE>
__device__ __forceinline__ void slice_sums(float (&acc)[CE], int cp, int c, int n_chunks,
                                           float (*red)[kHeadDim]) {
  for (int m = cp; m < kWave; m <<= 1) {
#pragma unroll
    for (int e = 0; e < CE; ++e) acc[e] += __shfl_xor(acc[e], m);
  }
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  if (lane < cp && c < n_chunks) {
#pragma unroll
    for (int e = 0; e < CE; ++e) red[wave][c * CE + e] = acc[e];
  }
}

__device__ __forceinline__ int pow2_at_least(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

// Compression of token `row` (= b * n_tokens + t) for KV head g, by a
// workgroup of 256 threads.  T: input and factor elements; C: cache elements
// (T itself, or E4M3 codes beside bf16 inputs: then the Key is rounded too).
// LOWREG: each phase requests its own factor chunks, four at a time, when it
// starts, instead of all of them up front -- the same arithmetic in the same
// order (identical results) in far fewer registers, for a body that runs
// inside another launch whose register budget it must not raise.
template <typename T, typename C, bool LOWREG = false>
__device__ __forceinline__ void append_body(
    const T *__restrict__ kin, const T *__restrict__ vin, const int32_t *__restrict__ start_pos,
    const T *__restrict__ A, const T *__restrict__ P, const T *__restrict__ E,
    C *__restrict__ zpool, C *__restrict__ rpool, C *__restrict__ kpool,
    const int32_t *__restrict__ block_table, const AppendArgs &a, int g, int row) {
  constexpr int DH = kHeadDim;
  constexpr int CE = Elem<T>::CE;
  constexpr int CC = Elem<C>::CE;  // cache elements per 16-byte chunk
  constexpr bool kRoundKey = sizeof(C) != sizeof(T);
  constexpr int MAXL = 64 / CE;  // factor chunks per thread and phase (see the roles below)
  __shared__ float v_s[DH], k_s[DH], x_s[DH], zf[DH];
  __shared__ float red[4][DH];
  __shared__ __align__(16) C zst[DH];
  __shared__ __align__(16) C rst[DH];
  __shared__ __align__(16) C kst[kRoundKey ? DH : CC];
  const int b = row / a.n_tokens, t = row - b * a.n_tokens;
  const int tid = threadIdx.x;
  const int64_t in_off = (((int64_t)b * a.n_tokens + t) * a.n_kv + g) * DH;

  // Roles: each phase splits its output into 16-byte chunks (C of them,
  // padded to a power of two Cp) and its contraction into S = 256 / Cp slices
  // of L entries; thread tid sums slice tid / Cp of chunk tid % Cp.  Every
  // factor chunk is requested up front, since none depends on the token.
  const int C1 = a.rv / CE, P1 = pow2_at_least(C1), S1 = 256 / P1, L1 = (DH + S1 - 1) / S1;
  const int C2 = DH / CE, P2 = pow2_at_least(C2), S2 = 256 / P2, L2 = (a.rb + S2 - 1) / S2;
  const int C3 = a.rq / CE, P3 = pow2_at_least(C3), S3 = 256 / P3, L3 = (DH + S3 - 1) / S3;
  const int c1 = tid % P1, s1 = tid / P1;  // z = v A
  const int c2 = tid % P2, s2 = tid / P2;  // c = z_s P
  const int c3 = tid % P3, s3 = tid / P3;  // r = x E
  const T *Ag = A + (int64_t)g * DH * a.rv;
  const T *Pg = P + (int64_t)g * a.rb * DH;
  const T *Eg = E + (int64_t)g * DH * a.rq;
  constexpr int NF = LOWREG ? 1 : MAXL;  // prefetched chunks per factor
  uint4 fa[NF], fp[NF], fe[NF];
  if constexpr (!LOWREG) {
#pragma unroll
    for (int l = 0; l < MAXL; ++l) {
      const int d = s1 * L1 + l;
      if (c1 < C1 && l < L1 && d < DH)
        fa[l] = *reinterpret_cast<const uint4 *>(Ag + (int64_t)d * a.rv + c1 * CE);
      const int j = s2 * L2 + l;
      if (c2 < C2 && l < L2 && j < a.rb)
        fp[l] = *reinterpret_cast<const uint4 *>(Pg + (int64_t)j * DH + c2 * CE);
      const int d3 = s3 * L3 + l;
      if (c3 < C3 && l < L3 && d3 < DH)
        fe[l] = *reinterpret_cast<const uint4 *>(Eg + (int64_t)d3 * a.rq + c3 * CE);
    }
  }
  // acc[e] += w(l) * row l of a factor, l in order; rows come from the
  // prefetched chunks or (LOWREG) four at a time from memory
  auto phase = [&](float (&acc)[CE], const uint4 *pre, bool on, int n_rows, int lim, int first,
                   const T *base, int64_t stride, int col, const float *wv) {
    if constexpr (!LOWREG) {
#pragma unroll
      for (int l = 0; l < MAXL; ++l) {
        const int r = first + l;
        if (on && l < n_rows && r < lim) {
          float x[CE];
          unpack_chunk<T>(pre[l], x);
          const float w = wv[r];
#pragma unroll
          for (int e = 0; e < CE; ++e) acc[e] = fmaf(w, x[e], acc[e]);
        }
      }
    } else {
#pragma unroll 1
      for (int l0 = 0; l0 < MAXL; l0 += 4) {
        uint4 ch[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int l = l0 + u, r = first + l;
          if (on && l < n_rows && r < lim)
            ch[u] = *reinterpret_cast<const uint4 *>(base + (int64_t)r * stride + col * CE);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int l = l0 + u, r = first + l;
          if (on && l < n_rows && r < lim) {
            float x[CE];
            unpack_chunk<T>(ch[u], x);
            const float w = wv[r];
#pragma unroll
            for (int e = 0; e < CE; ++e) acc[e] = fmaf(w, x[e], acc[e]);
          }
        }
      }
    }
  };
  // the destination slot, looked up while the factors are in flight
  const int pos = start_pos[b] + t;
  const bool pos_ok = pos >= 0 && pos < a.cap;
  const int page = pos_ok ? pos / a.page_size : 0;
  const int slot = pos - page * a.page_size;
  const int phys = pos_ok ? block_table[(int64_t)b * a.max_pages + page] : -1;
  if (tid < DH) {
    v_s[tid] = to_f32(vin[in_off + tid]);
    k_s[tid] = to_f32(kin[in_off + tid]);
  }
  __syncthreads();

  float acc[CE];
  // ---- z = v A_g; z_s = round(z) ----
#pragma unroll
  for (int e = 0; e < CE; ++e) acc[e] = 0.f;
  phase(acc, fa, c1 < C1, L1, DH, s1 * L1, Ag, a.rv, c1, v_s);
  slice_sums<CE>(acc, P1, c1, C1, red);
  __syncthreads();
  if (tid < a.rv) {
    const float z = red[0][tid] + red[1][tid] + red[2][tid] + red[3][tid];
    const C zs = from_f32<C>(z);
    zst[tid] = zs;
    zf[tid] = to_f32(zs);
  }
  __syncthreads();

  // ---- x = k - z_s[:r_b] P_g ----
#pragma unroll
  for (int e = 0; e < CE; ++e) acc[e] = 0.f;
  phase(acc, fp, c2 < C2, L2, a.rb, s2 * L2, Pg, DH, c2, zf);
  slice_sums<CE>(acc, P2, c2, C2, red);
  __syncthreads();
  if (tid < DH) x_s[tid] = k_s[tid] - (red[0][tid] + red[1][tid] + red[2][tid] + red[3][tid]);
  __syncthreads();

  // ---- r = x E_g; r_s = round(r) ----
#pragma unroll
  for (int e = 0; e < CE; ++e) acc[e] = 0.f;
  phase(acc, fe, c3 < C3, L3, DH, s3 * L3, Eg, a.rq, c3, x_s);
  slice_sums<CE>(acc, P3, c3, C3, red);
  __syncthreads();
  if (tid < a.rq)
    rst[tid] = from_f32<C>(red[0][tid] + red[1][tid] + red[2][tid] + red[3][tid]);
  if (kRoundKey && tid < DH) kst[tid] = from_f32<C>(k_s[tid]);
  __syncthreads();

  // ---- page stores: one 16-byte chunk per thread ----
  if (!pos_ok || phys < 0 || phys >= a.num_phys) return;
  const int64_t hp = (int64_t)g * a.num_phys + phys;
  const int zc = a.rv / CC, rc = a.rq / CC, kc = DH / CC;
  if (tid < zc + rc + kc) {
    uint4 val;
    char *dst;
    if (tid < zc) {
      val = *reinterpret_cast<const uint4 *>(zst + tid * CC);
      dst = reinterpret_cast<char *>(zpool) +
            ((hp * a.geom.z_page_chunks + z_chunk_slot(a.geom, tid)) * a.page_size + slot) * 16;
    } else if (tid < zc + rc) {
      const int c = tid - zc;
      val = *reinterpret_cast<const uint4 *>(rst + c * CC);
      dst = reinterpret_cast<char *>(rpool) +
            ((hp * a.geom.r_page_chunks + a.geom.r_first + c) * a.page_size + slot) * 16;
    } else {
      const int c = tid - zc - rc;
      if constexpr (kRoundKey)
        val = *reinterpret_cast<const uint4 *>(kst + c * CC);
      else
        val = *reinterpret_cast<const uint4 *>(kin + in_off + c * CC);
      dst = reinterpret_cast<char *>(kpool) + ((hp * kc + c) * a.page_size + slot) * 16;
    }
    *reinterpret_cast<uint4 *>(dst) = val;
  }
}

// ---------------------------------------------------------------------------
// (a1) q_proj[b][h] = [P_g q_bh, Q_g q_bh]   (float32; bf16 products are exact)
// Rows j of [P_g; Q_g] (head_dim elements each) lie 16 lanes to a row, 8 dims
// per lane, so a load instruction reads whole rows (256 or 512 contiguous
// bytes each) rather than one 16-byte piece of 64 different rows.  A
// workgroup of NT threads takes the NT / 16 rows of row block xblk of KV
// head g for sequence b; its factor loads are in flight while the group's
// queries are staged in LDS.  Each lane forms its 8-dim partial dot for every
// head of the group, the row's 16 lanes sum them (DPP), and lane h of the row
// stores head h's output.  TAG (the projection inside the scoring launch):
// the outputs are written through to the agent's coherence point, and once
// every one of them has been acknowledged thread 0 writes `tag` to *done the
// same way, so a reader on any XCD that sees the tag (reading as
// load_coherent does) reads this block's values, not older ones.
// ---------------------------------------------------------------------------
template <typename T, int NT, bool TAG = false>
__device__ __forceinline__ void project_body(const T *__restrict__ q, const T *__restrict__ P,
                                             const T *__restrict__ Q, float *__restrict__ q_proj,
                                             int n_q, int n_kv, int rb, int rq, int xblk, int g,
                                             int b, uint32_t *done = nullptr, uint32_t tag = 0) {
  constexpr int RPW = NT / 16;                    // rows per workgroup
  constexpr int NL = 8 * (int)sizeof(T) / 16;     // 16-byte loads per lane: 1 (bf16), 2 (float32)
  constexpr int CE = Elem<T>::CE;
  __shared__ __align__(16) float qs[16][kHeadDim];
  const int G = n_q / n_kv;
  const int w = rb + rq;
  const int c = threadIdx.x & 15;  // dims 8 c .. 8 c + 7
  const int j = xblk * RPW + (threadIdx.x >> 4);
  const bool active = j < w;
  uint4 raw[NL];
#pragma unroll
  for (int l = 0; l < NL; ++l) raw[l] = make_uint4(0u, 0u, 0u, 0u);
  if (active) {  // the factor row's 8 dims are in flight while the queries are staged
    const T *row = j < rb ? P + ((int64_t)g * rb + j) * kHeadDim
                          : Q + ((int64_t)g * rq + (j - rb)) * kHeadDim;
#pragma unroll
    for (int l = 0; l < NL; ++l) raw[l] = reinterpret_cast<const uint4 *>(row + 8 * c)[l];
  }
  {  // the group's queries: G * head_dim elements (G <= 16), one batch of loads
    constexpr int QL = 16 * kHeadDim / NT;
    const T *qg = q + ((int64_t)b * n_q + g * G) * kHeadDim;
    T qv[QL];
#pragma unroll
    for (int u = 0; u < QL; ++u) {
      const int i = u * NT + threadIdx.x;
      if (i < G * kHeadDim) qv[u] = qg[i];
    }
#pragma unroll
    for (int u = 0; u < QL; ++u) {
      const int i = u * NT + threadIdx.x;
      if (i < G * kHeadDim) qs[i / kHeadDim][i % kHeadDim] = to_f32(qv[u]);
    }
  }
  __syncthreads();
  float x[8];
#pragma unroll
  for (int l = 0; l < NL; ++l) unpack_chunk<T>(raw[l], x + l * CE);
  // every lane takes part (inactive rows hold zeros): the sums read whole rows of lanes
  float mine = 0.f;
  for (int h = 0; h < G; ++h) {
    const float4 q0 = *reinterpret_cast<const float4 *>(&qs[h][8 * c]);
    const float4 q1 = *reinterpret_cast<const float4 *>(&qs[h][8 * c + 4]);
    float part = x[0] * q0.x;
    part = fmaf(x[1], q0.y, part);
    part = fmaf(x[2], q0.z, part);
    part = fmaf(x[3], q0.w, part);
    part = fmaf(x[4], q1.x, part);
    part = fmaf(x[5], q1.y, part);
    part = fmaf(x[6], q1.z, part);
    part = fmaf(x[7], q1.w, part);
    part += dpp_move<0xB1>(part);   // lanes c ^ 1
    part += dpp_move<0x4E>(part);   // lanes c ^ 2
    part += dpp_move<0x141>(part);  // the other quad of the half-row
    part += dpp_move<0x140>(part);  // the other half of the row
    if (c == h) mine = part;
  }
  if (active && c < G) {
    const int64_t o = ((int64_t)b * n_q + g * G + c) * w + j;
    if constexpr (TAG)
      store_coherent(q_proj + o, mine);
    else
      q_proj[o] = mine;
  }
  if constexpr (TAG) {
    wait_stores_done();
    __syncthreads();
    if (threadIdx.x == 0) store_coherent_u32(done, tag);
  }
}

}  // namespace bkv

namespace bkv_host {
// The decode step's append: one new token per sequence.
inline bkv::AppendArgs step_append_args(const basiskv_dims &d) {
  bkv::AppendArgs a;
  a.n_tokens = 1;
  a.n_kv = d.n_kv_heads;
  a.rv = d.r_v;
  a.rb = d.r_b;
  a.rq = d.r_q;
  a.max_pages = d.max_pages_per_seq;
  a.num_phys = d.num_phys_pages;
  a.page_size = d.page_size;
  a.cap = d.max_pages_per_seq * d.page_size;
  a.geom = pool_geom(d);
  return a;
}
}  // namespace bkv_host
