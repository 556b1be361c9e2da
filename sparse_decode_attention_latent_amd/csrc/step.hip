// One launch for the start of a decode step: the new token's compression
// (a0) and the routing projection of the queries (a1) are independent, so
// their workgroups share one grid (the first n_kv * batch workgroups
// compress, the rest project).  Without with_append only the projection runs
// here (the compression then runs inside the scoring launch; rotary-position
// steps keep it here).  The first workgroup also zeroes the counters
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

// The start of a decode step whose compression runs inside the scoring
// launch: the query projection alone (8 rows of [P; Q] per 128-thread
// workgroup, as basiskv_project_queries), and the first workgroup zeroes the
// attention's merge counters.
template <typename T>
__global__ __launch_bounds__(128) void step_project_kernel(
    const T *__restrict__ q, const T *__restrict__ P, const T *__restrict__ Q,
    float *__restrict__ q_proj, int n_q, int n_kv, int rb, int rq, int32_t *__restrict__ counters,
    int n_counters) {
  if (blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0)
    for (int i = threadIdx.x; i < n_counters; i += blockDim.x) counters[i] = 0;
  project_body<T, 128>(q, P, Q, q_proj, n_q, n_kv, rb, rq, blockIdx.x, blockIdx.y, blockIdx.z);
}

}  // namespace bkv

namespace bkv_host {
using namespace bkv;

template <typename T, typename C>
static hipError_t prologue_t(const basiskv_dims &d, const void *q, const void *k_new,
                             const void *v_new, const int32_t *start_pos, const void *A,
                             const void *P, const void *Q, const void *E, const basiskv_cache &c,
                             float *q_proj, int32_t *counters, int n_counters, hipStream_t s,
                             bool with_append) {
  PrologueArgs a;
  a.counters = counters;
  a.n_counters = n_counters;
  a.ap = step_append_args(d);
  a.n_append = with_append ? d.n_kv_heads * d.batch : 0;
  a.proj_x = (d.r_b + d.r_q + 15) / 16;  // 16 rows per 256-thread workgroup
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
                                int n_counters, hipStream_t s, bool with_append) {
  if (!with_append) {
    const dim3 grid((d.r_b + d.r_q + 7) / 8, d.n_kv_heads, d.batch);
    if (act_bf16(d))
      hipLaunchKernelGGL(step_project_kernel<uint16_t>, grid, dim3(128), 0, s, (const uint16_t *)q,
                         (const uint16_t *)P, (const uint16_t *)Q, q_proj, d.n_q_heads,
                         d.n_kv_heads, d.r_b, d.r_q, counters, n_counters);
    else
      hipLaunchKernelGGL(step_project_kernel<float>, grid, dim3(128), 0, s, (const float *)q,
                         (const float *)P, (const float *)Q, q_proj, d.n_q_heads, d.n_kv_heads,
                         d.r_b, d.r_q, counters, n_counters);
    return hipGetLastError();
  }
  if (cache_fp8(d))
    return prologue_t<uint16_t, uint8_t>(d, q, k_new, v_new, start_pos, A, P, Q, E, c, q_proj,
                                         counters, n_counters, s, with_append);
  return act_bf16(d)
             ? prologue_t<uint16_t, uint16_t>(d, q, k_new, v_new, start_pos, A, P, Q, E, c, q_proj,
                                              counters, n_counters, s, with_append)
             : prologue_t<float, float>(d, q, k_new, v_new, start_pos, A, P, Q, E, c, q_proj,
                                        counters, n_counters, s, with_append);
}

}  // namespace bkv_host
