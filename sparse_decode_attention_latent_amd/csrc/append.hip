// (a0) for a handful of new tokens (the per-step decode append): the same
// compression as the prefill MFMA kernel -- BasisKV abstract (the Value is
// kept only as a low-rank latent; a Key-specific residual holds what the
// latent cannot predict) and appendix Table 4 (latent, residual and exact Key
// per token) -- as three float32 matrix-vector products per (token, KV head):
//   z = v A_g,  z_s = round(z);  r = (k - z_s[:r_b] P_g) E_g,  r_s = round(r)
// and the stores of z_s, r_s and k into their pages.  With one or a few rows
// per head, staging the factors for MFMA costs more than it saves; here every
// workgroup requests all of its head's factor chunks at once (they come from
// L2 after the first sequence), so the kernel costs one memory round trip
// plus three LDS reductions.
// grid (n_kv, batch * n_tokens), 256 threads.
#include "common.hpp"

namespace bkv {

struct AppendArgs {
  int n_tokens, n_kv, rv, rb, rq, max_pages, num_phys, page_size, cap;
};

template <typename T>
__global__ __launch_bounds__(256) void append_kernel(
    const T *__restrict__ kin, const T *__restrict__ vin, const int32_t *__restrict__ start_pos,
    const T *__restrict__ A, const T *__restrict__ P, const T *__restrict__ E,
    T *__restrict__ zpool, T *__restrict__ rpool, T *__restrict__ kpool,
    const int32_t *__restrict__ block_table, AppendArgs a) {
  constexpr int DH = kHeadDim;
  constexpr int CE = Elem<T>::CE;
  constexpr int MAXL = 64 / CE;  // factor chunks per thread and phase (see the roles below)
  __shared__ float v_s[DH], k_s[DH], x_s[DH], zf[DH];
  __shared__ float red[256 * CE];
  __shared__ __align__(16) T zst[DH];
  __shared__ __align__(16) T rst[DH];
  const int g = blockIdx.x, row = blockIdx.y;
  const int b = row / a.n_tokens, t = row - b * a.n_tokens;
  const int tid = threadIdx.x;
  const int64_t in_off = (((int64_t)b * a.n_tokens + t) * a.n_kv + g) * DH;

  // Roles: each phase splits its output into 16-byte chunks (C) and its
  // contraction into slices (S = 256 / C, L entries each); thread (c, s) sums
  // slice s of chunk c.  Every factor chunk is requested up front, since none
  // depends on the token.
  const int C1 = a.rv / CE, S1 = 256 / C1, L1 = (DH + S1 - 1) / S1;    // z = v A
  const int C2 = DH / CE, S2 = 256 / C2, L2 = (a.rb + S2 - 1) / S2;    // c = z_s P
  const int C3 = a.rq / CE, S3 = 256 / C3, L3 = (DH + S3 - 1) / S3;    // r = x E
  const int c1 = tid % C1, s1 = tid / C1;
  const int c2 = tid % C2, s2 = tid / C2;
  const int c3 = tid % C3, s3 = tid / C3;
  const T *Ag = A + (int64_t)g * DH * a.rv;
  const T *Pg = P + (int64_t)g * a.rb * DH;
  const T *Eg = E + (int64_t)g * DH * a.rq;
  uint4 fa[MAXL], fp[MAXL], fe[MAXL];
#pragma unroll
  for (int l = 0; l < MAXL; ++l) {
    const int d = s1 * L1 + l;
    if (s1 < S1 && l < L1 && d < DH)
      fa[l] = *reinterpret_cast<const uint4 *>(Ag + (int64_t)d * a.rv + c1 * CE);
    const int j = s2 * L2 + l;
    if (s2 < S2 && l < L2 && j < a.rb)
      fp[l] = *reinterpret_cast<const uint4 *>(Pg + (int64_t)j * DH + c2 * CE);
    const int d3 = s3 * L3 + l;
    if (s3 < S3 && l < L3 && d3 < DH)
      fe[l] = *reinterpret_cast<const uint4 *>(Eg + (int64_t)d3 * a.rq + c3 * CE);
  }
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
  if (s1 < S1) {
#pragma unroll
    for (int l = 0; l < MAXL; ++l) {
      const int d = s1 * L1 + l;
      if (l < L1 && d < DH) {
        float x[CE];
        unpack_chunk<T>(fa[l], x);
        const float vd = v_s[d];
#pragma unroll
        for (int e = 0; e < CE; ++e) acc[e] = fmaf(vd, x[e], acc[e]);
      }
    }
#pragma unroll
    for (int e = 0; e < CE; ++e) red[s1 * a.rv + c1 * CE + e] = acc[e];
  }
  __syncthreads();
  if (tid < a.rv) {
    float z = 0.f;
    for (int s = 0; s < S1; ++s) z += red[s * a.rv + tid];
    const T zs = from_f32<T>(z);
    zst[tid] = zs;
    zf[tid] = to_f32(zs);
  }
  __syncthreads();

  // ---- x = k - z_s[:r_b] P_g ----
#pragma unroll
  for (int e = 0; e < CE; ++e) acc[e] = 0.f;
  if (s2 < S2) {
#pragma unroll
    for (int l = 0; l < MAXL; ++l) {
      const int j = s2 * L2 + l;
      if (l < L2 && j < a.rb) {
        float x[CE];
        unpack_chunk<T>(fp[l], x);
        const float zj = zf[j];
#pragma unroll
        for (int e = 0; e < CE; ++e) acc[e] = fmaf(zj, x[e], acc[e]);
      }
    }
#pragma unroll
    for (int e = 0; e < CE; ++e) red[s2 * DH + c2 * CE + e] = acc[e];
  }
  __syncthreads();
  if (tid < DH) {
    float c = 0.f;
    for (int s = 0; s < S2; ++s) c += red[s * DH + tid];
    x_s[tid] = k_s[tid] - c;
  }
  __syncthreads();

  // ---- r = x E_g; r_s = round(r) ----
#pragma unroll
  for (int e = 0; e < CE; ++e) acc[e] = 0.f;
  if (s3 < S3) {
#pragma unroll
    for (int l = 0; l < MAXL; ++l) {
      const int d = s3 * L3 + l;
      if (l < L3 && d < DH) {
        float x[CE];
        unpack_chunk<T>(fe[l], x);
        const float xd = x_s[d];
#pragma unroll
        for (int e = 0; e < CE; ++e) acc[e] = fmaf(xd, x[e], acc[e]);
      }
    }
#pragma unroll
    for (int e = 0; e < CE; ++e) red[s3 * a.rq + c3 * CE + e] = acc[e];
  }
  __syncthreads();
  if (tid < a.rq) {
    float r = 0.f;
    for (int s = 0; s < S3; ++s) r += red[s * a.rq + tid];
    rst[tid] = from_f32<T>(r);
  }
  __syncthreads();

  // ---- page stores: one 16-byte chunk per thread ----
  if (!pos_ok || phys < 0 || phys >= a.num_phys) return;
  const int64_t hp = (int64_t)g * a.num_phys + phys;
  const int zc = a.rv / CE, rc = a.rq / CE, kc = DH / CE;
  if (tid < zc + rc + kc) {
    uint4 val;
    char *dst;
    if (tid < zc) {
      val = *reinterpret_cast<const uint4 *>(zst + tid * CE);
      dst = reinterpret_cast<char *>(zpool) + ((hp * zc + tid) * a.page_size + slot) * 16;
    } else if (tid < zc + rc) {
      const int c = tid - zc;
      val = *reinterpret_cast<const uint4 *>(rst + c * CE);
      dst = reinterpret_cast<char *>(rpool) + ((hp * rc + c) * a.page_size + slot) * 16;
    } else {
      const int c = tid - zc - rc;
      val = *reinterpret_cast<const uint4 *>(kin + in_off + c * CE);
      dst = reinterpret_cast<char *>(kpool) + ((hp * kc + c) * a.page_size + slot) * 16;
    }
    *reinterpret_cast<uint4 *>(dst) = val;
  }
}

}  // namespace bkv

namespace bkv_host {
using namespace bkv;

template <typename T>
static hipError_t append_t(const basiskv_dims &d, const void *k, const void *v,
                           const int32_t *start_pos, int32_t n_tokens, const void *A,
                           const void *P, const void *E, const basiskv_cache &c, hipStream_t s) {
  AppendArgs a;
  a.n_tokens = n_tokens;
  a.n_kv = d.n_kv_heads;
  a.rv = d.r_v;
  a.rb = d.r_b;
  a.rq = d.r_q;
  a.max_pages = d.max_pages_per_seq;
  a.num_phys = d.num_phys_pages;
  a.page_size = d.page_size;
  a.cap = d.max_pages_per_seq * d.page_size;
  hipLaunchKernelGGL(append_kernel<T>, dim3(d.n_kv_heads, d.batch * n_tokens), dim3(256), 0, s,
                     (const T *)k, (const T *)v, start_pos, (const T *)A, (const T *)P,
                     (const T *)E, (T *)c.z_pages, (T *)c.r_pages, (T *)c.k_pages, c.block_table, a);
  return hipGetLastError();
}

hipError_t launch_append(const basiskv_dims &d, const void *k, const void *v,
                         const int32_t *start_pos, int32_t n_tokens, const void *A, const void *P,
                         const void *E, const basiskv_cache &c, hipStream_t s) {
  return d.dtype == BASISKV_BF16 ? append_t<uint16_t>(d, k, v, start_pos, n_tokens, A, P, E, c, s)
                                 : append_t<float>(d, k, v, start_pos, n_tokens, A, P, E, c, s);
}

}  // namespace bkv_host
