// MFMA kernels: output reconstruction (a5), the fused latent-to-output matrix
// (set-up), and compression of new tokens into the cache (a0).
// BasisKV (arXiv 2611.02583): abstract (Value compression tied to the output
// projection; Key-specific residual), Figure 1 (the output is rebuilt from the
// latents), appendix Table 4 (latent, residual and exact Key per token).
//
// All GEMMs use 16x16 MFMA tiles: v_mfma_f32_16x16x32_bf16 for bf16 data and
// v_mfma_f32_16x16x4_f32 for float32 data, float32 accumulation.  Operand
// convention for both: lane l holds row (or column) l % 16 and the k slots of
// group l / 16; A and B fragments are always loaded with the same k slot ->
// k-index map, so the contraction is exact whatever order the unit uses
// internally.  The 16x16 result sits as C[4 * (l / 16) + r][l % 16], r = 0..3.
#include "common.hpp"

namespace bkv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

struct MfmaBf16 {
  using frag = bf16x8;
  static constexpr int KS = 32;  // k per instruction
  static constexpr int KPL = 8;  // k slots per lane
  __device__ static floatx4 mma(frag a, frag b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};
struct MfmaF32 {
  using frag = float;
  static constexpr int KS = 4;
  static constexpr int KPL = 1;
  __device__ static floatx4 mma(frag a, frag b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
};

template <typename T> struct MfmaFor;
template <> struct MfmaFor<uint16_t> { using type = MfmaBf16; };
template <> struct MfmaFor<float> { using type = MfmaF32; };

__device__ __forceinline__ bf16x8 bits_to_frag(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// 8 float32 values -> bf16x8 (nearest-even), and the remainder term lo = x - hi.
__device__ __forceinline__ void split_bf16(const float *x, bf16x8 *hi, bf16x8 *lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h[i] = f32x2_to_bf16x2(x[2 * i], x[2 * i + 1]);
    l[i] = f32x2_to_bf16x2(x[2 * i] - __uint_as_float(h[i] << 16),
                           x[2 * i + 1] - __uint_as_float(h[i] & 0xffff0000u));
  }
  *hi = bits_to_frag(make_uint4(h[0], h[1], h[2], h[3]));
  *lo = bits_to_frag(make_uint4(l[0], l[1], l[2], l[3]));
}

// ---------------------------------------------------------------------------
// Tiled layout of the fused output matrix.  Element (n, k) of M (row n =
// output feature, k = h * r_v + i) sits at
//   ((n / 16 * (K / KSTEP) + k / KSTEP) * 64 + (k % KSTEP) / KPL * 16 + n % 16) * KPL + k % KPL
// with KPL = 16 / sizeof(element) and KSTEP = 4 * KPL: the B fragment of one
// MFMA step (16 output features x KSTEP contraction slots) is one contiguous
// 1 KB run, lane l holding its 16 bytes at l * 16.
// ---------------------------------------------------------------------------
template <typename T>
__host__ __device__ __forceinline__ int64_t mtile_index(int n, int k, int K) {
  constexpr int KPL = 16 / (int)sizeof(T);
  constexpr int KSTEP = 4 * KPL;
  return (((int64_t)(n / 16) * (K / KSTEP) + k / KSTEP) * 64 + (k % KSTEP) / KPL * 16 + n % 16) *
             KPL + k % KPL;
}

// ---------------------------------------------------------------------------
// (a5) y[b][n] = sum_k u[b][k] M[n][k],  K = n_q * r_v, M in the tiled layout.
// One workgroup of 8 wavefronts per 16 output columns; the wavefronts split K
// and their 16x16 tiles are summed through LDS.  bf16: the A rows are
// [hi(u) of 8 sequences ; lo(u) of the same 8], so one MFMA carries both
// terms and y = C[b] + C[b + 8].  float32: 16 sequences per row tile.
// ---------------------------------------------------------------------------
constexpr int kReconWaves = 8;

template <typename T, int RT, bool UT>
__global__ __launch_bounds__(512) void reconstruct_kernel(const float *__restrict__ u,
                                                         const uint16_t *__restrict__ u_tiles,
                                                         const T *__restrict__ M,
                                                         T *__restrict__ y, int batch, int K,
                                                         int N) {
  using MF = typename MfmaFor<T>::type;
  constexpr bool kBf = sizeof(T) == 2;
  constexpr int ROWS = kBf ? 8 : 16;  // sequences per row tile
  __shared__ float red[kReconWaves][RT][16][17];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n0 = blockIdx.x * 16;
  const int i = lane & 15, qg = lane >> 4;
  const int n_steps = (K + MF::KS - 1) / MF::KS;
  floatx4 acc[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) acc[rt] = floatx4{0.f, 0.f, 0.f, 0.f};

  if constexpr (kBf) {
  if constexpr (UT) {
    // u already split into its bf16 A operand (utile_index): fragments are
    // loaded as they are; rows past the batch read as zero
    constexpr int U = 8;
    for (int ks0 = wave; ks0 < n_steps; ks0 += kReconWaves * U) {
      uint4 braw[U], araw[U][RT];
#pragma unroll
      for (int uu = 0; uu < U; ++uu) {
        const int ks = ks0 + uu * kReconWaves;
        braw[uu] = make_uint4(0, 0, 0, 0);
        if (ks < n_steps)
          braw[uu] = reinterpret_cast<const uint4 *>(M)[((int64_t)blockIdx.x * n_steps + ks) * 64 + lane];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          araw[uu][rt] = make_uint4(0, 0, 0, 0);
          if (ks < n_steps && rt * ROWS + (i & 7) < batch)
            araw[uu][rt] = reinterpret_cast<const uint4 *>(u_tiles)[((int64_t)rt * n_steps + ks) * 64 + lane];
        }
      }
#pragma unroll
      for (int uu = 0; uu < U; ++uu)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
          acc[rt] = MF::mma(bits_to_frag(araw[uu][rt]), bits_to_frag(braw[uu]), acc[rt]);
    }
  } else {
    // U k-steps per round: every load of the round is issued before the first MFMA
    constexpr int U = 8 / RT;
    for (int ks0 = wave; ks0 < n_steps; ks0 += kReconWaves * U) {
      uint4 braw[U];
      float4 ux[U][RT][2];
#pragma unroll
      for (int uu = 0; uu < U; ++uu) {
        const int ks = ks0 + uu * kReconWaves;
        const int k = ks * MF::KS + qg * 8;
        braw[uu] = make_uint4(0, 0, 0, 0);
        if (ks < n_steps)
          braw[uu] = reinterpret_cast<const uint4 *>(M)[((int64_t)blockIdx.x * n_steps + ks) * 64 + lane];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          const int b = rt * ROWS + (i & 7);
          ux[uu][rt][0] = ux[uu][rt][1] = make_float4(0.f, 0.f, 0.f, 0.f);
          if (b < batch && k < K) {
            const float4 *up = reinterpret_cast<const float4 *>(u + (int64_t)b * K + k);
            ux[uu][rt][0] = up[0];
            ux[uu][rt][1] = up[1];
          }
        }
      }
#pragma unroll
      for (int uu = 0; uu < U; ++uu) {
        const bf16x8 bfrag = bits_to_frag(braw[uu]);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          const float4 x0 = ux[uu][rt][0], x1 = ux[uu][rt][1];
          const float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
          bf16x8 hi, lo;
          split_bf16(x, &hi, &lo);
          acc[rt] = MF::mma(i < 8 ? hi : lo, bfrag, acc[rt]);
        }
      }
    }
  }
  } else {
    // float32: each lane loads 4 consecutive k and feeds 4 MFMAs (k slot (qg, s) -> k0 + 4 qg + s)
    constexpr int U = 8 / RT;
    const int n_quads = (K + 15) / 16;
    for (int kq0 = wave; kq0 < n_quads; kq0 += kReconWaves * U) {
      float4 bq[U], aq[U][RT];
#pragma unroll
      for (int uu = 0; uu < U; ++uu) {
        const int kq = kq0 + uu * kReconWaves;
        const int k = kq * 16 + qg * 4;
        bq[uu] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (kq < n_quads)
          bq[uu] = reinterpret_cast<const float4 *>(M)[((int64_t)blockIdx.x * n_quads + kq) * 64 + lane];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          const int b = rt * ROWS + i;
          aq[uu][rt] = make_float4(0.f, 0.f, 0.f, 0.f);
          if (b < batch && k < K) aq[uu][rt] = *reinterpret_cast<const float4 *>(u + (int64_t)b * K + k);
        }
      }
#pragma unroll
      for (int uu = 0; uu < U; ++uu)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          acc[rt] = MF::mma(aq[uu][rt].x, bq[uu].x, acc[rt]);
          acc[rt] = MF::mma(aq[uu][rt].y, bq[uu].y, acc[rt]);
          acc[rt] = MF::mma(aq[uu][rt].z, bq[uu].z, acc[rt]);
          acc[rt] = MF::mma(aq[uu][rt].w, bq[uu].w, acc[rt]);
        }
    }
  }
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int r = 0; r < 4; ++r) red[wave][rt][qg * 4 + r][i] = acc[rt][r];
  __syncthreads();
  for (int o = threadIdx.x; o < RT * ROWS * 16; o += blockDim.x) {
    const int rt = o / (ROWS * 16), rem = o % (ROWS * 16);
    const int br = rem / 16, col = rem % 16;
    const int b = rt * ROWS + br;
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < kReconWaves; ++w) {
      s += red[w][rt][br][col];
      if (kBf) s += red[w][rt][br + 8][col];
    }
    if (b < batch && n0 + col < N) y[(int64_t)b * N + n0 + col] = from_f32<T>(s);
  }
}

// ---------------------------------------------------------------------------
// Set-up: M[n][h*r_v + i] = sum_d Bf[h/G][i][d] W_O[h*dh + d][n], stored tiled.
// grid (ceil(N/64), n_q), 256 threads; W_O's 128 x 64 tile staged in LDS.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void fuse_kernel(const T *__restrict__ Bf,
                                                   const T *__restrict__ W_O, T *__restrict__ M,
                                                   int n_q, int n_kv, int rv, int N) {
  __shared__ float wt[kHeadDim][65];
  const int n0 = blockIdx.x * 64, h = blockIdx.y;
  const int g = h / (n_q / n_kv);
  for (int o = threadIdx.x; o < kHeadDim * 64; o += blockDim.x) {
    const int d = o / 64, c = o % 64;
    wt[d][c] = (n0 + c < N) ? to_f32(W_O[((int64_t)h * kHeadDim + d) * N + n0 + c]) : 0.f;
  }
  __syncthreads();
  const int K = n_q * rv;
  for (int o = threadIdx.x; o < 64 * rv; o += blockDim.x) {
    const int c = o / rv, i = o % rv;  // consecutive threads: consecutive i (contiguous in M)
    const T *brow = Bf + ((int64_t)g * rv + i) * kHeadDim;
    float s = 0.f;
    for (int d = 0; d < kHeadDim; ++d) s = fmaf(to_f32(brow[d]), wt[d][c], s);
    if (n0 + c < N) M[mtile_index<T>(n0 + c, h * rv + i, K)] = from_f32<T>(s);
  }
}

// ---------------------------------------------------------------------------
// (a0) compression of new tokens.  Rows are (sequence, token) pairs of one KV
// head g; a wavefront handles 16 rows at a time:
//   Z  = V A_g                 (MFMA)  -> stored latent z_s (rounded)
//   C  = z_s[:, :r_b] P_g      (MFMA)
//   R  = (K - C) E_g           (MFMA; bf16: K - C split into hi + lo terms)
// and writes z_s, round(R) and K into their pages.  The factors are staged once
// per workgroup, transposed so that every B fragment is a contiguous k run.
// grid (workgroups per head, n_kv), 256 threads, dynamic LDS.
// ---------------------------------------------------------------------------
struct CompressArgs {
  int batch, n_tokens, n_kv, rv, rb, rq, rb_pad, max_pages, num_phys, page_size, cap;
};

template <typename T>
__global__ __launch_bounds__(256) void compress_kernel(
    const T *__restrict__ kin, const T *__restrict__ vin, const int32_t *__restrict__ start_pos,
    const T *__restrict__ A, const T *__restrict__ P, const T *__restrict__ E,
    T *__restrict__ zpool, T *__restrict__ rpool, T *__restrict__ kpool,
    const int32_t *__restrict__ block_table, CompressArgs a) {
  using MF = typename MfmaFor<T>::type;
  using frag = typename MF::frag;
  constexpr int CE = Elem<T>::CE;
  constexpr int DH = kHeadDim;
  constexpr bool kBf = sizeof(T) == 2;
  extern __shared__ __align__(16) unsigned char smem[];
  // layout: At [rv][DH] T | Pt [DH][rb_pad] T | Et [rq][DH] T | per wave: Zs [16][rv_pad] T,
  //         C [16][DH+4] float, Rs [16][rq] T
  const int g = blockIdx.y;
  const int rv_pad = (a.rv + MF::KS - 1) / MF::KS * MF::KS;
  T *At = reinterpret_cast<T *>(smem);
  T *Pt = At + a.rv * DH;
  T *Et = Pt + DH * a.rb_pad;
  unsigned char *wave_base = reinterpret_cast<unsigned char *>(Et + a.rq * DH);
  const size_t zs_bytes = (size_t)16 * rv_pad * sizeof(T);
  const size_t c_bytes = (size_t)16 * (DH + 4) * sizeof(float);
  const size_t rs_bytes = (size_t)16 * a.rq * sizeof(T);
  const size_t per_wave = (zs_bytes + c_bytes + rs_bytes + 15) / 16 * 16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  T *Zs = reinterpret_cast<T *>(wave_base + wave * per_wave);
  float *Cs = reinterpret_cast<float *>(wave_base + wave * per_wave + zs_bytes);
  T *Rs = reinterpret_cast<T *>(wave_base + wave * per_wave + zs_bytes + c_bytes);

  // stage transposed factors of head g
  const T *Ag = A + (int64_t)g * DH * a.rv;
  const T *Pg = P + (int64_t)g * a.rb * DH;
  const T *Eg = E + (int64_t)g * DH * a.rq;
  for (int o = threadIdx.x; o < DH * a.rv; o += blockDim.x) {
    const int d = o / a.rv, i = o % a.rv;
    At[i * DH + d] = Ag[o];
  }
  for (int o = threadIdx.x; o < DH * a.rb_pad; o += blockDim.x) {
    const int d = o / a.rb_pad, j = o % a.rb_pad;
    Pt[o] = j < a.rb ? Pg[(int64_t)j * DH + d] : from_f32<T>(0.f);
  }
  for (int o = threadIdx.x; o < DH * a.rq; o += blockDim.x) {
    const int d = o / a.rq, m = o % a.rq;
    Et[m * DH + d] = Eg[o];
  }
  __syncthreads();

  const int rows = a.batch * a.n_tokens;
  const int n_blocks = (rows + 15) / 16;
  const int i = lane & 15, qg = lane >> 4;
  const int zc_total = a.rv / CE, rc_total = a.rq / CE, kc_total = DH / CE;

  // Every wavefront runs the same number of iterations (the barriers below are
  // block-wide); a wavefront past the last row block computes on zero rows and
  // stores nothing.
  for (int base = blockIdx.x * 4; base < n_blocks; base += gridDim.x * 4) {
    const int rb16 = base + wave;
    const int row = rb16 * 16 + i;  // this lane's A row
    const bool row_ok = row < rows;
    const int sb = row_ok ? row / a.n_tokens : 0;
    const int st = row_ok ? row - sb * a.n_tokens : 0;
    const int64_t in_off = (((int64_t)sb * a.n_tokens + st) * a.n_kv + g) * DH;

    // ---- Z = V A ----
    for (int nt = 0; nt < a.rv / 16; ++nt) {
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
      for (int ks = 0; ks < DH / MF::KS; ++ks) {
        const int k = ks * MF::KS + qg * MF::KPL;
        frag af, bfr;
        if constexpr (kBf) {
          af = bits_to_frag(row_ok ? *reinterpret_cast<const uint4 *>(vin + in_off + k)
                                   : make_uint4(0, 0, 0, 0));
          bfr = bits_to_frag(*reinterpret_cast<const uint4 *>(At + (nt * 16 + i) * DH + k));
        } else {
          af = row_ok ? reinterpret_cast<const float *>(vin)[in_off + k] : 0.f;
          bfr = reinterpret_cast<const float *>(At)[(nt * 16 + i) * DH + k];
        }
        acc = MF::mma(af, bfr, acc);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) Zs[(qg * 4 + r) * rv_pad + nt * 16 + i] = from_f32<T>(acc[r]);
    }
    for (int o = lane; o < 16 * (rv_pad - a.rv); o += 64) {
      const int rr = o / (rv_pad - a.rv), cc = a.rv + o % (rv_pad - a.rv);
      Zs[rr * rv_pad + cc] = from_f32<T>(0.f);
    }
    __syncthreads();

    // ---- C = z_s[:, :rb] P ----
    for (int nt = 0; nt < DH / 16; ++nt) {
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
      for (int ks = 0; ks < a.rb_pad / MF::KS; ++ks) {
        const int k = ks * MF::KS + qg * MF::KPL;
        frag af, bfr;
        if constexpr (kBf) {
          // columns past r_b are zero in Pt, so the latent's extra dims drop out
          af = bits_to_frag(*reinterpret_cast<const uint4 *>(Zs + i * rv_pad + k));
          bfr = bits_to_frag(*reinterpret_cast<const uint4 *>(Pt + (nt * 16 + i) * a.rb_pad + k));
        } else {
          af = reinterpret_cast<const float *>(Zs)[i * rv_pad + k];
          bfr = reinterpret_cast<const float *>(Pt)[(nt * 16 + i) * a.rb_pad + k];
        }
        acc = MF::mma(af, bfr, acc);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) Cs[(qg * 4 + r) * (DH + 4) + nt * 16 + i] = acc[r];
    }
    __syncthreads();

    // ---- R = (K - C) E ; also copy K into its pages ----
    for (int nt = 0; nt < a.rq / 16; ++nt) {
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
      for (int ks = 0; ks < DH / MF::KS; ++ks) {
        const int k = ks * MF::KS + qg * MF::KPL;
        if constexpr (kBf) {
          float x[8];
          const uint4 kraw = row_ok ? *reinterpret_cast<const uint4 *>(kin + in_off + k)
                                    : make_uint4(0, 0, 0, 0);
          unpack_chunk<uint16_t>(kraw, x);
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] -= Cs[i * (DH + 4) + k + e];
          bf16x8 hi, lo;
          split_bf16(x, &hi, &lo);
          const bf16x8 bfr = bits_to_frag(*reinterpret_cast<const uint4 *>(Et + (nt * 16 + i) * DH + k));
          acc = MF::mma(hi, bfr, acc);
          acc = MF::mma(lo, bfr, acc);
        } else {
          const float kv = row_ok ? reinterpret_cast<const float *>(kin)[in_off + k] : 0.f;
          const float x = kv - Cs[i * (DH + 4) + k];
          acc = MF::mma(x, reinterpret_cast<const float *>(Et)[(nt * 16 + i) * DH + k], acc);
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) Rs[(qg * 4 + r) * a.rq + nt * 16 + i] = from_f32<T>(acc[r]);
    }
    __syncthreads();

    // ---- page stores: one 16-byte chunk per (row, chunk) ----
    const int per_row = zc_total + rc_total + kc_total;
    for (int o = lane; o < 16 * per_row; o += 64) {
      const int rr = o / per_row, c = o % per_row;
      const int grow = rb16 * 16 + rr;
      if (grow >= rows) continue;
      const int b = grow / a.n_tokens, t = grow - b * a.n_tokens;
      const int pos = start_pos[b] + t;
      if (pos < 0 || pos >= a.cap) continue;
      const int page = pos / a.page_size, slot = pos - page * a.page_size;
      const int phys = block_table[(int64_t)b * a.max_pages + page];
      if (phys < 0 || phys >= a.num_phys) continue;
      const int64_t hp = (int64_t)g * a.num_phys + phys;
      uint4 val;
      char *dst;
      if (c < zc_total) {
        val = *reinterpret_cast<const uint4 *>(Zs + rr * rv_pad + c * CE);
        dst = reinterpret_cast<char *>(zpool) + ((hp * zc_total + c) * a.page_size + slot) * 16;
      } else if (c < zc_total + rc_total) {
        const int cc = c - zc_total;
        val = *reinterpret_cast<const uint4 *>(Rs + rr * a.rq + cc * CE);
        dst = reinterpret_cast<char *>(rpool) + ((hp * rc_total + cc) * a.page_size + slot) * 16;
      } else {
        const int cc = c - zc_total - rc_total;
        val = *reinterpret_cast<const uint4 *>(
            kin + (((int64_t)b * a.n_tokens + t) * a.n_kv + g) * DH + cc * CE);
        dst = reinterpret_cast<char *>(kpool) + ((hp * kc_total + cc) * a.page_size + slot) * 16;
      }
      *reinterpret_cast<uint4 *>(dst) = val;
    }
    __syncthreads();
  }
}

template <typename T>
static size_t compress_lds_bytes(const basiskv_dims &d, int rb_pad) {
  const int ks = sizeof(T) == 2 ? 32 : 4;
  const int rv_pad = (d.r_v + ks - 1) / ks * ks;
  const size_t fac = (size_t)(d.r_v * kHeadDim + kHeadDim * rb_pad + d.r_q * kHeadDim) * sizeof(T);
  const size_t per_wave = ((size_t)16 * rv_pad * sizeof(T) + (size_t)16 * (kHeadDim + 4) * 4 +
                           (size_t)16 * d.r_q * sizeof(T) + 15) / 16 * 16;
  return fac + 4 * per_wave;
}

}  // namespace bkv

namespace bkv_host {
using namespace bkv;

template <typename T>
static hipError_t recon_t(const basiskv_dims &d, const float *u, const uint16_t *u_tiles,
                          const void *M, void *y, hipStream_t s) {
  const int rows = sizeof(T) == 2 ? 8 : 16;
  const int rt = (d.batch + rows - 1) / rows;
  const int K = d.n_q_heads * d.r_v, N = d.hidden;
  dim3 grid((N + 15) / 16), block(512);
  const T *Mt = (const T *)M;
  T *yt = (T *)y;
#define BKV_RECON(RTV, UTV)                                                                    \
  hipLaunchKernelGGL((reconstruct_kernel<T, RTV, UTV>), grid, block, 0, s, u, u_tiles, Mt, yt, \
                     d.batch, K, N)
  const bool ut = sizeof(T) == 2 && u_tiles != nullptr;
  if (rt <= 1) {
    if (ut) BKV_RECON(1, true); else BKV_RECON(1, false);
  } else if (rt <= 2) {
    if (ut) BKV_RECON(2, true); else BKV_RECON(2, false);
  } else {
    if (ut) BKV_RECON(4, true); else BKV_RECON(4, false);
  }
#undef BKV_RECON
  return hipGetLastError();
}

hipError_t launch_reconstruct(const basiskv_dims &d, const float *u, const uint16_t *u_tiles,
                              const void *M, void *y, hipStream_t s) {
  return d.dtype == BASISKV_BF16 ? recon_t<uint16_t>(d, u, u_tiles, M, y, s)
                                 : recon_t<float>(d, u, nullptr, M, y, s);
}

template <typename T>
static hipError_t fuse_t(const basiskv_dims &d, const void *Bf, const void *W_O, void *M,
                         hipStream_t s) {
  hipLaunchKernelGGL(fuse_kernel<T>, dim3((d.hidden + 63) / 64, d.n_q_heads), dim3(256), 0, s,
                     (const T *)Bf, (const T *)W_O, (T *)M, d.n_q_heads, d.n_kv_heads, d.r_v,
                     d.hidden);
  return hipGetLastError();
}

hipError_t launch_fuse(const basiskv_dims &d, const void *Bf, const void *W_O, void *M,
                       hipStream_t s) {
  return d.dtype == BASISKV_BF16 ? fuse_t<uint16_t>(d, Bf, W_O, M, s) : fuse_t<float>(d, Bf, W_O, M, s);
}

template <typename T>
static hipError_t compress_t(const basiskv_dims &d, const void *k, const void *v,
                             const int32_t *start_pos, int32_t n_tokens, const void *A,
                             const void *P, const void *E, const basiskv_cache &c, hipStream_t s) {
  const int ks = sizeof(T) == 2 ? 32 : 4;
  CompressArgs a;
  a.batch = d.batch;
  a.n_tokens = n_tokens;
  a.n_kv = d.n_kv_heads;
  a.rv = d.r_v;
  a.rb = d.r_b;
  a.rq = d.r_q;
  a.rb_pad = (d.r_b + ks - 1) / ks * ks;
  a.max_pages = d.max_pages_per_seq;
  a.num_phys = d.num_phys_pages;
  a.page_size = d.page_size;
  a.cap = d.max_pages_per_seq * d.page_size;
  const size_t lds = compress_lds_bytes<T>(d, a.rb_pad);
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&compress_kernel<T>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  const int rows = d.batch * n_tokens;
  const int n_blocks = (rows + 15) / 16;
  int wgs = (n_blocks + 3) / 4;
  if (wgs > 32) wgs = 32;  // persistent: factors are staged once per workgroup
  hipLaunchKernelGGL(compress_kernel<T>, dim3(wgs, d.n_kv_heads), dim3(256), lds, s, (const T *)k,
                     (const T *)v, start_pos, (const T *)A, (const T *)P, (const T *)E,
                     (T *)c.z_pages, (T *)c.r_pages, (T *)c.k_pages, c.block_table, a);
  return hipGetLastError();
}

// Few rows per head (the decode append): matrix-vector kernel; otherwise MFMA.
constexpr int kAppendMaxRows = 64;

hipError_t launch_compress(const basiskv_dims &d, const void *k, const void *v,
                           const int32_t *start_pos, int32_t n_tokens, const void *A,
                           const void *P, const void *E, const basiskv_cache &c, hipStream_t s) {
  if ((int64_t)d.batch * n_tokens <= kAppendMaxRows && d.r_v <= kHeadDim && d.r_q <= kHeadDim)
    return launch_append(d, k, v, start_pos, n_tokens, A, P, E, c, s);
  return d.dtype == BASISKV_BF16 ? compress_t<uint16_t>(d, k, v, start_pos, n_tokens, A, P, E, c, s)
                                 : compress_t<float>(d, k, v, start_pos, n_tokens, A, P, E, c, s);
}

size_t compress_lds(const basiskv_dims &d) {
  const int ks = d.dtype == BASISKV_BF16 ? 32 : 4;
  const int rb_pad = (d.r_b + ks - 1) / ks * ks;
  return d.dtype == BASISKV_BF16 ? compress_lds_bytes<uint16_t>(d, rb_pad)
                                 : compress_lds_bytes<float>(d, rb_pad);
}

}  // namespace bkv_host
