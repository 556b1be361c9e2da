// One launch for the start of a decode step: the new token's compression
// (a0) and the routing projection of the queries (a1) are independent, so
// their workgroups share one grid (the first n_kv * batch workgroups
// compress, the rest project).  The first workgroup also zeroes the counters
// with which the step's attention launch elects its merging workgroups (they
// are left at zero by every call; clearing them here makes the step
// independent of what an earlier call left in the workspace).  Bodies in
// decode_bodies.hpp.
#include "decode_bodies.hpp"

namespace bkv {

struct PrologueArgs {
  AppendArgs ap;
  int n_append, proj_x, n_q, n_kv, rb, rq;
  int32_t *counters;  // attention merge counters to zero (n_counters of them)
  int n_counters;
};

template <typename T, typename C>
__global__ __launch_bounds__(256) void step_prologue_kernel(
    const T *__restrict__ k_new, const T *__restrict__ v_new, const int32_t *__restrict__ start_pos,
    const T *__restrict__ A, const T *__restrict__ P, const T *__restrict__ E,
    const T *__restrict__ Q, const T *__restrict__ q, C *__restrict__ zpool,
    C *__restrict__ rpool, C *__restrict__ kpool, const int32_t *__restrict__ block_table,
    float *__restrict__ q_proj, PrologueArgs a) {
  const int idx = blockIdx.x;
  if (idx == 0)
    for (int i = threadIdx.x; i < a.n_counters; i += blockDim.x) a.counters[i] = 0;
  if (idx < a.n_append) {
    append_body<T, C>(k_new, v_new, start_pos, A, P, E, zpool, rpool, kpool, block_table, a.ap,
                   idx % a.n_kv, idx / a.n_kv);
  } else {
    const int j = idx - a.n_append;
    const int xblk = j % a.proj_x, rest = j / a.proj_x;
    project_body<T, 256>(q, P, Q, q_proj, a.n_q, a.n_kv, a.rb, a.rq, xblk, rest % a.n_kv,
                         rest / a.n_kv);
  }
}

}  // namespace bkv

namespace bkv_host {
using namespace bkv;

template <typename T, typename C>
static hipError_t prologue_t(const basiskv_dims &d, const void *q, const void *k_new,
                             const void *v_new, const int32_t *start_pos, const void *A,
                             const void *P, const void *Q, const void *E, const basiskv_cache &c,
                             float *q_proj, int32_t *counters, int n_counters, hipStream_t s) {
  PrologueArgs a;
  a.counters = counters;
  a.n_counters = n_counters;
  a.ap.n_tokens = 1;
  a.ap.n_kv = d.n_kv_heads;
  a.ap.rv = d.r_v;
  a.ap.rb = d.r_b;
  a.ap.rq = d.r_q;
  a.ap.max_pages = d.max_pages_per_seq;
  a.ap.num_phys = d.num_phys_pages;
  a.ap.page_size = d.page_size;
  a.ap.cap = d.max_pages_per_seq * d.page_size;
  a.ap.geom = pool_geom(d);
  a.n_append = d.n_kv_heads * d.batch;
  const int G = d.n_q_heads / d.n_kv_heads;
  a.proj_x = (G * (d.r_b + d.r_q) + 255) / 256;
  a.n_q = d.n_q_heads;
  a.n_kv = d.n_kv_heads;
  a.rb = d.r_b;
  a.rq = d.r_q;
  const int grid = a.n_append + a.proj_x * d.n_kv_heads * d.batch;
  hipLaunchKernelGGL((step_prologue_kernel<T, C>), dim3(grid), dim3(256), 0, s,
                     (const T *)k_new, (const T *)v_new, start_pos, (const T *)A, (const T *)P,
                     (const T *)E, (const T *)Q, (const T *)q, (C *)c.z_pages, (C *)residual_pool(d, c),
                     (C *)c.k_pages, c.block_table, q_proj, a);
  return hipGetLastError();
}

hipError_t launch_step_prologue(const basiskv_dims &d, const void *q, const void *k_new,
                                const void *v_new, const int32_t *start_pos, const void *A,
                                const void *P, const void *Q, const void *E,
                                const basiskv_cache &c, float *q_proj, int32_t *counters,
                                int n_counters, hipStream_t s) {
  if (cache_fp8(d))
    return prologue_t<uint16_t, uint8_t>(d, q, k_new, v_new, start_pos, A, P, Q, E, c, q_proj,
                                         counters, n_counters, s);
  return act_bf16(d)
             ? prologue_t<uint16_t, uint16_t>(d, q, k_new, v_new, start_pos, A, P, Q, E, c, q_proj,
                                              counters, n_counters, s)
             : prologue_t<float, float>(d, q, k_new, v_new, start_pos, A, P, Q, E, c, q_proj,
                                        counters, n_counters, s);
}

}  // namespace bkv_host
