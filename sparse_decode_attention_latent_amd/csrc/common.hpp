// Device helpers shared by the gfx950 kernels of libbasiskv.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "basiskv.h"

namespace bkv {

constexpr int kHeadDim = 128;   // the only head dim the kernels are built for
constexpr int kWave = 64;       // CDNA wavefront width
constexpr int kXcds = 8;        // MI355X: 8 accelerator dies, each with its own L2
constexpr float kLog2e = 1.4426950408889634f;

// Storage element types: float for BASISKV_F32, uint16_t (bf16 bits) for
// BASISKV_BF16 and for the activations of BASISKV_BF16_FP8_E4M3, uint8_t
// (E4M3FN codes) for that format's cache pages.
template <typename T> struct Elem;
template <> struct Elem<float> {
  static constexpr int CE = 4;  // elements per 16-byte chunk
};
template <> struct Elem<uint16_t> {
  static constexpr int CE = 8;
};
template <> struct Elem<uint8_t> {
  static constexpr int CE = 16;
};

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// float32 -> bf16, round to nearest even (gfx950 converts in hardware:
// v_cvt_pk_bf16_f32; checked bit for bit against a software round-to-nearest-
// even over normal, subnormal, tie and NaN inputs).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}
// Two float32 values -> packed bf16 pair (a in the low half).
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float a, float b) {
  typedef __bf16 pair_t __attribute__((ext_vector_type(2)));
  const pair_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// FP8 cache codes: OCP E4M3FN (exponent bias 7, 3 mantissa bits, largest
// finite magnitude 448, no infinities), no scale factor.  gfx950 converts in
// hardware (v_cvt_pk_fp8_f32 / v_cvt_f32_fp8, round to nearest even); its
// encoder gives the NaN code for magnitudes of 464 and more, so the cache
// writes saturate to +-448 first (a NaN input stays NaN).
__device__ __forceinline__ float sat_e4m3(float x) {
  return fabsf(x) > 448.f ? copysignf(448.f, x) : x;
}
// Four float32 values -> four E4M3 codes (a in the lowest byte).
__device__ __forceinline__ uint32_t f32x4_to_fp8x4(float a, float b, float c, float d) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(sat_e4m3(a), sat_e4m3(b), 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(sat_e4m3(c), sat_e4m3(d), lo, true);
}
__device__ __forceinline__ uint8_t f32_to_fp8(float x) {
  return (uint8_t)(__builtin_amdgcn_cvt_pk_fp8_f32(sat_e4m3(x), 0.f, 0, false) & 0xff);
}
__device__ __forceinline__ float fp8_to_f32(uint8_t code) {
  return __builtin_amdgcn_cvt_f32_fp8((int)code, 0);
}

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(uint16_t x) { return bf16_to_f32(x); }
__device__ __forceinline__ float to_f32(uint8_t x) { return fp8_to_f32(x); }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ uint16_t from_f32<uint16_t>(float x) { return f32_to_bf16(x); }
template <> __device__ __forceinline__ uint8_t from_f32<uint8_t>(float x) { return f32_to_fp8(x); }

// x rounded to the cache format C, as float32 (exact: every bf16 and E4M3
// value is a float32).
template <typename C> __device__ __forceinline__ float round_to(float x) {
  return to_f32(from_f32<C>(x));
}

// Widen one 16-byte chunk to float32 (exact for both formats).
template <typename T> __device__ __forceinline__ void unpack_chunk(const uint4 &c, float *x);
template <> __device__ __forceinline__ void unpack_chunk<float>(const uint4 &c, float *x) {
  x[0] = __uint_as_float(c.x);
  x[1] = __uint_as_float(c.y);
  x[2] = __uint_as_float(c.z);
  x[3] = __uint_as_float(c.w);
}
template <> __device__ __forceinline__ void unpack_chunk<uint16_t>(const uint4 &c, float *x) {
  x[0] = __uint_as_float(c.x << 16);
  x[1] = __uint_as_float(c.x & 0xffff0000u);
  x[2] = __uint_as_float(c.y << 16);
  x[3] = __uint_as_float(c.y & 0xffff0000u);
  x[4] = __uint_as_float(c.z << 16);
  x[5] = __uint_as_float(c.z & 0xffff0000u);
  x[6] = __uint_as_float(c.w << 16);
  x[7] = __uint_as_float(c.w & 0xffff0000u);
}
typedef float bkv_f2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void fp8x4_to_f32(uint32_t w, float *x) {
  const bkv_f2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  const bkv_f2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  x[0] = lo[0];
  x[1] = lo[1];
  x[2] = hi[0];
  x[3] = hi[1];
}
template <> __device__ __forceinline__ void unpack_chunk<uint8_t>(const uint4 &c, float *x) {
  fp8x4_to_f32(c.x, x);
  fp8x4_to_f32(c.y, x + 4);
  fp8x4_to_f32(c.z, x + 8);
  fp8x4_to_f32(c.w, x + 12);
}
// Eight E4M3 codes (two words) -> eight bf16 values (exact), as one 8-element
// bf16 chunk's worth of packed pairs.
__device__ __forceinline__ uint4 fp8x8_to_bf16x8(uint32_t w0, uint32_t w1) {
  float x[8];
  fp8x4_to_f32(w0, x);
  fp8x4_to_f32(w1, x + 4);
  return make_uint4(f32x2_to_bf16x2(x[0], x[1]), f32x2_to_bf16x2(x[2], x[3]),
                    f32x2_to_bf16x2(x[4], x[5]), f32x2_to_bf16x2(x[6], x[7]));
}

// acc + a.lo * b.lo + a.hi * b.hi for two packed bf16 pairs (v_dot2c_f32_bf16:
// the products are exact in float32; the result carries float32 rounding).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), acc, false);
}

// Rotary position embedding: sin and cos of the angle pos * w.  The product
// is taken in double precision (exact for positions below 2^24 and float32
// frequencies), reduced to a fraction of a turn, and evaluated by the
// hardware sine and cosine, which take turns (v_sin_f32 / v_cos_f32).
// The same from a frequency given in turns per position (w / (2 pi), double):
// one product and its fraction per angle.
__device__ __forceinline__ void rope_sincos_turns(double pos, double wt, float &sn, float &cs) {
  const float f = (float)__builtin_amdgcn_fract(pos * wt);  // (pos, wt >= 0)
  sn = __builtin_amdgcn_sinf(f);
  cs = __builtin_amdgcn_cosf(f);
}
__device__ __forceinline__ void rope_sincos(int pos, float w, float &sn, float &cs) {
  const double turns = (double)pos * (double)w * 0.15915494309189535;  // 1 / (2 pi)
  const float f = (float)(turns - floor(turns));
  sn = __builtin_amdgcn_sinf(f);
  cs = __builtin_amdgcn_cosf(f);
}

__device__ __forceinline__ uint4 load_chunk(const void *base_bytes, int64_t byte_off) {
  return *reinterpret_cast<const uint4 *>(reinterpret_cast<const char *>(base_bytes) + byte_off);
}

// A 16-byte load marked non-temporal (global_load_dwordx4 ... nt): for page
// data a launch reads once.  On MI355X a streaming read with these loads
// reaches about 7.0-7.2 TB/s, against 6.0-6.3 TB/s with ordinary loads
// (400 MiB, 2K-25K workgroups, 4-16 loads in flight per lane).
typedef unsigned int bkv_u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_chunk_stream(const void *base_bytes, int64_t byte_off) {
  const bkv_u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const bkv_u32x4 *>(
      reinterpret_cast<const char *>(base_bytes) + byte_off));
  return make_uint4(v[0], v[1], v[2], v[3]);
}
template <bool NT>
__device__ __forceinline__ uint4 load_page_chunk(const void *base_bytes, int64_t byte_off) {
  return NT ? load_chunk_stream(base_bytes, byte_off) : load_chunk(base_bytes, byte_off);
}

// Ordering point for LDS traffic between the lanes of one wavefront.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Cross-lane steps through DPP (no LDS round trip).  Control codes of the
// GFX9 data-parallel-primitives modifier: quad_perm [1,0,3,2] (0xB1) and
// [2,3,0,1] (0x4E) swap neighbours at distance 1 and 2; row_half_mirror
// (0x141) reverses each 8-lane half-row; row_mirror (0x140) reverses each
// 16-lane row.  Applied in that order with an associative op, every lane of a
// group of 4 / 8 / 16 ends with the group's result.
template <int CTRL>
__device__ __forceinline__ float dpp_move(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float lane_value(float v, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// Maximum over aligned groups of `width` lanes (1, 2, 4, 8, 16, 32 or 64;
// wave-uniform); every lane of a group receives the group's maximum.
__device__ __forceinline__ float group_max(float v, int width) {
  if (width >= 2) v = fmaxf(v, dpp_move<0xB1>(v));
  if (width >= 4) v = fmaxf(v, dpp_move<0x4E>(v));
  if (width >= 8) v = fmaxf(v, dpp_move<0x141>(v));
  if (width >= 16) v = fmaxf(v, dpp_move<0x140>(v));
  if (width >= 32) {
    const float r0 = lane_value(v, 0), r1 = lane_value(v, 16);
    const float r2 = lane_value(v, 32), r3 = lane_value(v, 48);
    if (width == 32) {
      v = (threadIdx.x & 32) ? fmaxf(r2, r3) : fmaxf(r0, r1);
    } else {
      v = fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
    }
  }
  return v;
}

// Wave-wide maximum and sum; the result is wavefront-uniform.
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_move<0xB1>(v));
  v = fmaxf(v, dpp_move<0x4E>(v));
  v = fmaxf(v, dpp_move<0x141>(v));
  v = fmaxf(v, dpp_move<0x140>(v));
  return fmaxf(fmaxf(lane_value(v, 0), lane_value(v, 16)),
               fmaxf(lane_value(v, 32), lane_value(v, 48)));
}

__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_move<0xB1>(v);
  v += dpp_move<0x4E>(v);
  v += dpp_move<0x141>(v);
  v += dpp_move<0x140>(v);
  return (lane_value(v, 0) + lane_value(v, 16)) + (lane_value(v, 32) + lane_value(v, 48));
}

// Device-coherent hand-off between the workgroups of one launch.  Results
// that another workgroup will read are written with relaxed agent-scope
// atomic stores (they write through to the device coherence point, so every
// XCD's L2 sees them) and read back with relaxed agent-scope atomic loads.
// A workgroup counts itself done only after its own stores have completed
// (s_waitcnt vmcnt(0) in every thread, then a barrier); the workgroup whose
// increment completes the count handles the row.  No L2 write-back or
// invalidate is involved, which a device-scope fence would issue for every
// workgroup.
__device__ __forceinline__ void store_coherent(float *p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float *p) {
  return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_coherent_u32(uint32_t *p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t load_coherent_u32(const uint32_t *p) {
  return __hip_atomic_load(const_cast<uint32_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wait_stores_done() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0); expcnt, lgkmcnt unconstrained
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
// True in every thread of the workgroup that completes `counter` to `total`
// arrivals; that workgroup also resets the counter to zero for the next launch.
__device__ __forceinline__ bool last_to_arrive(int32_t *counter, int total) {
  __shared__ int is_last;
  wait_stores_done();
  __syncthreads();
  if (threadIdx.x == 0) {
    const int prev = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    is_last = prev == total - 1;
    if (is_last) __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  return is_last;
}

// The latent output u as the A operand of the reconstruction MFMA
// (v_mfma_f32_16x16x32_bf16): per row tile of 8 sequences and per
// 32-slot contraction step, one 1 KB run of 64 lanes x 8 bf16, lane
// (r + 16 q) holding row r, slots 8 q .. 8 q + 7.  Rows 0-7 carry the bf16
// rounding of u for the tile's 8 sequences, rows 8-15 the bf16 rounding of
// the remainder (u - hi), so one MFMA sees u to about 16 significant bits.
// Element (b, k), K = n_q * r_v (a multiple of 32):
__device__ __forceinline__ int64_t utile_index(int b, int k, int K, bool lo) {
  const int r = (b & 7) + (lo ? 8 : 0);
  return (((int64_t)(b >> 3) * (K / 32) + k / 32) * 64 + (k % 32) / 8 * 16 + r) * 8 + k % 8;
}
__device__ __forceinline__ void store_u_tiles(uint16_t *ut, int b, int k, int K, float x) {
  const uint16_t hi = f32_to_bf16(x);
  ut[utile_index(b, k, K, false)] = hi;
  ut[utile_index(b, k, K, true)] = f32_to_bf16(x - bf16_to_f32(hi));
}

// Work-item index of this workgroup for a 1-D grid of `padded` (multiple of 8)
// workgroups: consecutive work items land on the same XCD, so workgroups that
// share per-(sequence, head) data (projected queries, block-table rows) hit
// the same L2.  Workgroups are dispatched round-robin over the XCDs.
__device__ __forceinline__ int xcd_work_index(int padded) {
  const int bid = blockIdx.x;
  const int per_xcd = padded / kXcds;
  return (bid % kXcds) * per_xcd + bid / kXcds;
}

// Where a page's latent and residual chunks sit, in 16-byte chunks.  Separate
// pools: latent chunk c is chunk c of a latent page of z_page_chunks = r_v / CE
// chunks, residual chunk c is chunk c of a residual page.  Routing-first: one
// pool whose page holds the first r_b / CE latent chunks, then the residual
// chunks (from r_first = r_b / CE on), then the other latent chunks (shifted
// by z_shift = r_q / CE).
struct PoolGeom {
  int z_page_chunks;  // chunks per page of the latent pool
  int r_page_chunks;  // chunks per page of the residual pool
  int r_first;        // page chunk of residual chunk 0
  int z_split;        // latent chunks from this one on ...
  int z_shift;        // ... sit this many chunks further into the page
};
__host__ __device__ __forceinline__ int z_chunk_slot(const PoolGeom &g, int c) {
  return c < g.z_split ? c : c + g.z_shift;
}

__host__ __device__ __forceinline__ int clamp_len(int L, int cap) {
  return L < 0 ? 0 : (L > cap ? cap : L);
}

}  // namespace bkv

// Host-side launchers (defined in the .hip files, called by abi.hip after validation).
namespace bkv_host {
// bf16 activations (queries, factors, K/V inputs, M, y): BASISKV_BF16 and BASISKV_BF16_FP8_E4M3
inline bool act_bf16(const basiskv_dims &d) { return d.dtype != BASISKV_F32; }
// E4M3 cache pages
inline bool cache_fp8(const basiskv_dims &d) { return d.dtype == BASISKV_BF16_FP8_E4M3; }
// elements per 16-byte chunk of a cache page
inline int cache_chunk(const basiskv_dims &d) {
  return cache_fp8(d) ? 16 : (act_bf16(d) ? 8 : 4);
}
inline bool routing_first(const basiskv_dims &d) {
  return d.page_layout == BASISKV_LAYOUT_ROUTING_FIRST;
}
inline bkv::PoolGeom pool_geom(const basiskv_dims &d) {
  const int ce = cache_chunk(d);
  bkv::PoolGeom g;
  if (routing_first(d)) {
    // pages of whole 128-byte lines: with 4-token pages (a chunk row of 64
    // bytes) an odd chunk count is rounded up by one unused chunk, so that every
    // page -- and its leading routing run -- starts on a line
    const int chunks = (d.r_v + d.r_q) / ce, row = d.page_size * 16;
    const int unit = row >= 128 ? 1 : 128 / row;
    g.z_page_chunks = g.r_page_chunks = (chunks + unit - 1) / unit * unit;
    g.r_first = g.z_split = d.r_b / ce;
    g.z_shift = d.r_q / ce;
  } else {
    g.z_page_chunks = d.r_v / ce;
    g.r_page_chunks = d.r_q / ce;
    g.r_first = 0;
    g.z_split = d.r_v / ce;
    g.z_shift = 0;
  }
  return g;
}
// the residual pool: a pool of its own, or the latent pool (routing-first)
inline void *residual_pool(const basiskv_dims &d, const basiskv_cache &c) {
  return routing_first(d) ? c.z_pages : c.r_pages;
}

hipError_t launch_project(const basiskv_dims &d, const void *q, const void *P, const void *Q,
                          float *q_proj, hipStream_t s);
// A decode step's new tokens (one per sequence), compressed and scored inside
// the scoring launch; the selection launch then folds new_scores into the
// page scores (launch_select's new_pos / new_scores).
struct StepTokens {
  const void *k_new, *v_new, *A, *P, *E;
  const int32_t *start_pos;
  float *new_scores;  // [batch * n_kv_heads]
  // the query projection in the same launch (qtags null: projected before it)
  const void *q, *Q;
  uint32_t *qtags;    // [batch][n_kv_heads][row blocks] the step that last completed each
  uint32_t *epoch;    // the last step's tag (this step's is one more; the selection advances it)
  int32_t *counters;  // the attention's merge counters, zeroed there
  int n_counters;
};
// Whether the scoring launch can take the query projection in (matrix-core
// logits: bf16 or E4M3 pages, groups of a multiple of 4 heads).
bool score_projects(const basiskv_dims &d);
hipError_t launch_score(const basiskv_dims &d, const float *q_proj, const basiskv_cache &c,
                        float *scores, hipStream_t s, bool *unsupported,
                        const StepTokens *step = nullptr);
bool score_rope_supported(const basiskv_dims &d);
hipError_t launch_score_rope(const basiskv_dims &d, const void *q, const void *P, const void *Q,
                             const basiskv_cache &c, float *scores, hipStream_t s,
                             bool *unsupported);
bool attend_supported(const basiskv_dims &d, bool rope);
hipError_t launch_select(const basiskv_dims &d, float *scores, const int32_t *seq_lens,
                         int32_t top_k, int32_t *sel, hipStream_t s,
                         const int32_t *new_pos = nullptr, const float *new_scores = nullptr,
                         uint32_t *epoch = nullptr);
int attend_splits(const basiskv_dims &d, int32_t top_k);
int attend_group_split(const basiskv_dims &d);
hipError_t launch_attend(const basiskv_dims &d, const void *q, const basiskv_cache &c,
                         const int32_t *sel, int32_t top_k, float scale, float *u, float *part,
                         int32_t *counters, uint16_t *u_tiles, hipStream_t s, bool *unsupported);
hipError_t launch_reconstruct(const basiskv_dims &d, const float *u, const uint16_t *u_tiles,
                              const void *M, void *y, hipStream_t s);
hipError_t launch_fuse(const basiskv_dims &d, const void *Bf, const void *W_O, void *M,
                       hipStream_t s);
hipError_t launch_pack_output(const basiskv_dims &d, const void *M_plain, void *M, hipStream_t s);
hipError_t launch_append(const basiskv_dims &d, const void *k, const void *v,
                         const int32_t *start_pos, int32_t n_tokens, const void *A, const void *P,
                         const void *E, const basiskv_cache &c, hipStream_t s);
hipError_t launch_step_prologue(const basiskv_dims &d, const void *q, const void *k_new,
                                const void *v_new, const int32_t *start_pos, const void *A,
                                const void *P, const void *Q, const void *E,
                                const basiskv_cache &c, float *q_proj, int32_t *counters,
                                int n_counters, hipStream_t s, bool with_append = true);
hipError_t launch_compress(const basiskv_dims &d, const void *k, const void *v,
                           const int32_t *start_pos, int32_t n_tokens, const void *A,
                           const void *P, const void *E, const basiskv_cache &c, hipStream_t s);
}  // namespace bkv_host
