// (a0) one-token (decode) compression launch; the body is in decode_bodies.hpp.
// grid (n_kv, batch * n_tokens), 256 threads.
#include "decode_bodies.hpp"

namespace bkv {

template <typename T, typename C>
__global__ __launch_bounds__(256) void append_kernel(
    const T *__restrict__ kin, const T *__restrict__ vin, const int32_t *__restrict__ start_pos,
    const T *__restrict__ A, const T *__restrict__ P, const T *__restrict__ E,
    C *__restrict__ zpool, C *__restrict__ rpool, C *__restrict__ kpool,
    const int32_t *__restrict__ block_table, AppendArgs a) {
  append_body<T, C>(kin, vin, start_pos, A, P, E, zpool, rpool, kpool, block_table, a, blockIdx.x,
                    blockIdx.y);
}

}  // namespace bkv

namespace bkv_host {
using namespace bkv;

template <typename T, typename C>
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
  a.geom = pool_geom(d);
  hipLaunchKernelGGL((append_kernel<T, C>), dim3(d.n_kv_heads, d.batch * n_tokens), dim3(256), 0,
                     s, (const T *)k, (const T *)v, start_pos, (const T *)A, (const T *)P,
                     (const T *)E, (C *)c.z_pages, (C *)residual_pool(d, c), (C *)c.k_pages,
                     c.block_table, a);
  return hipGetLastError();
}

hipError_t launch_append(const basiskv_dims &d, const void *k, const void *v,
                         const int32_t *start_pos, int32_t n_tokens, const void *A, const void *P,
                         const void *E, const basiskv_cache &c, hipStream_t s) {
  if (cache_fp8(d)) return append_t<uint16_t, uint8_t>(d, k, v, start_pos, n_tokens, A, P, E, c, s);
  return act_bf16(d) ? append_t<uint16_t, uint16_t>(d, k, v, start_pos, n_tokens, A, P, E, c, s)
                     : append_t<float, float>(d, k, v, start_pos, n_tokens, A, P, E, c, s);
}

}  // namespace bkv_host
