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
// One workgroup of 8 wavefronts per 16 output columns and group of RT row
// tiles (blockIdx.y); the wavefronts split K and their 16x16 tiles are summed
// through LDS.  bf16: the A rows are
// [hi(u) of 8 sequences ; lo(u) of the same 8], so one MFMA carries both
// terms and y = C[b] + C[b + 8].  float32: 16 sequences per row tile.
// ---------------------------------------------------------------------------
#ifndef BKV_RECON_WAVES
#define BKV_RECON_WAVES 8
#endif
constexpr int kReconWaves = BKV_RECON_WAVES;

template <typename T, int RT, bool UT>
__global__ __launch_bounds__(64 * kReconWaves) void reconstruct_kernel(const float *__restrict__ u,
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
  const int rt0 = blockIdx.y * RT;  // this workgroup's first row tile
  const int i = lane & 15, qg = lane >> 4;
  const int n_steps = (K + MF::KS - 1) / MF::KS;
  floatx4 acc[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) acc[rt] = floatx4{0.f, 0.f, 0.f, 0.f};

  if constexpr (kBf) {
  if constexpr (UT) {
    // u already split into its bf16 A operand (utile_index): fragments are
    // loaded as they are.  Every load is unpredicated: the operand holds whole
    // row tiles, and a row past the batch only feeds output rows that are not
    // stored.  Rounds of U k-steps per wavefront, software-pipelined: the next
    // round's loads are in flight while the current round's MFMAs run.
    constexpr int U = 4;
    constexpr int kStride = kReconWaves * U;  // k-steps per round, whole workgroup
    const int n_tiles = (batch + ROWS - 1) / ROWS;  // row tiles the operand holds
    uint4 b0[U], a0[U][RT], b1[U], a1[U][RT];
    auto load = [&](int ks0, uint4 (&braw)[U], uint4 (&araw)[U][RT]) {
#pragma unroll
      for (int uu = 0; uu < U; ++uu) {
        const int ks = min(ks0 + uu * kReconWaves, n_steps - 1);  // (clamped: used only below n_steps)
        braw[uu] = reinterpret_cast<const uint4 *>(M)[((int64_t)blockIdx.x * n_steps + ks) * 64 + lane];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
          araw[uu][rt] = rt0 + rt < n_tiles  // (wavefront-uniform)
              ? reinterpret_cast<const uint4 *>(u_tiles)[((int64_t)(rt0 + rt) * n_steps + ks) * 64 + lane]
              : make_uint4(0u, 0u, 0u, 0u);
      }
    };
    auto mma = [&](int ks0, const uint4 (&braw)[U], const uint4 (&araw)[U][RT]) {
#pragma unroll
      for (int uu = 0; uu < U; ++uu)
        if (ks0 + uu * kReconWaves < n_steps) {
#pragma unroll
          for (int rt = 0; rt < RT; ++rt)
            acc[rt] = MF::mma(bits_to_frag(araw[uu][rt]), bits_to_frag(braw[uu]), acc[rt]);
        }
    };
    if (wave < n_steps) {
      load(wave, b0, a0);
      for (int ks0 = wave;; ks0 += 2 * kStride) {
        const bool more1 = ks0 + kStride < n_steps;
        if (more1) load(ks0 + kStride, b1, a1);
        mma(ks0, b0, a0);
        if (!more1) break;
        const bool more2 = ks0 + 2 * kStride < n_steps;
        if (more2) load(ks0 + 2 * kStride, b0, a0);
        mma(ks0 + kStride, b1, a1);
        if (!more2) break;
      }
    }
  } else {
    // float32 u, split into bf16 hi + lo at use.  Rounds of U k-steps per
    // wavefront, software-pipelined as above.  Loads are unpredicated: rows past
    // the batch read the last row (they feed output rows that are not stored),
    // slots past K read the row's last 8 and are zeroed at use.
    constexpr int U = 4 / RT;
    constexpr int kStride = kReconWaves * U;
    uint4 b0[U], b1[U];
    float4 x0[U][RT][2], x1[U][RT][2];
    auto load = [&](int ks0, uint4 (&braw)[U], float4 (&ux)[U][RT][2]) {
#pragma unroll
      for (int uu = 0; uu < U; ++uu) {
        const int ks = min(ks0 + uu * kReconWaves, n_steps - 1);
        const int k = min(ks * MF::KS + qg * 8, K - 8);
        braw[uu] = reinterpret_cast<const uint4 *>(M)[((int64_t)blockIdx.x * n_steps + ks) * 64 + lane];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          const int b = min((rt0 + rt) * ROWS + (i & 7), batch - 1);
          const float4 *up = reinterpret_cast<const float4 *>(u + (int64_t)b * K + k);
          ux[uu][rt][0] = up[0];
          ux[uu][rt][1] = up[1];
        }
      }
    };
    auto mma = [&](int ks0, const uint4 (&braw)[U], const float4 (&ux)[U][RT][2]) {
#pragma unroll
      for (int uu = 0; uu < U; ++uu) {
        const int ks = ks0 + uu * kReconWaves;
        if (ks < n_steps) {
          const bool in_k = ks * MF::KS + qg * 8 < K;
          const bf16x8 bfrag = bits_to_frag(braw[uu]);
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) {
            const float4 y0 = ux[uu][rt][0], y1 = ux[uu][rt][1];
            float x[8] = {y0.x, y0.y, y0.z, y0.w, y1.x, y1.y, y1.z, y1.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = in_k ? x[e] : 0.f;
            bf16x8 hi, lo;
            split_bf16(x, &hi, &lo);
            acc[rt] = MF::mma(i < 8 ? hi : lo, bfrag, acc[rt]);
          }
        }
      }
    };
    if (wave < n_steps) {
      load(wave, b0, x0);
      for (int ks0 = wave;; ks0 += 2 * kStride) {
        const bool more1 = ks0 + kStride < n_steps;
        if (more1) load(ks0 + kStride, b1, x1);
        mma(ks0, b0, x0);
        if (!more1) break;
        const bool more2 = ks0 + 2 * kStride < n_steps;
        if (more2) load(ks0 + 2 * kStride, b0, x0);
        mma(ks0 + kStride, b1, x1);
        if (!more2) break;
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
          const int b = (rt0 + rt) * ROWS + i;
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
    const int b = (rt0 + rt) * ROWS + br;
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
// Set-up: a caller's plain fused matrix Mp [K][N] (row k = h * r_v + i, the
// latent slot; column n, the output feature) -> the tiled layout above.
// grid (ceil(N/64), ceil(K/64)), 256 threads: a 64 x 64 block is read row by
// row (coalesced) into LDS and written out as whole 16-byte tile chunks.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void pack_kernel(const T *__restrict__ Mp, T *__restrict__ Mt,
                                                   int K, int N) {
  constexpr int KPL = 16 / (int)sizeof(T);
  __shared__ T tile[64][64 + KPL];
  const int n0 = blockIdx.x * 64, k0 = blockIdx.y * 64;
  for (int o = threadIdx.x; o < 64 * 64; o += blockDim.x) {
    const int kk = o / 64, nn = o % 64;
    tile[kk][nn] = (k0 + kk < K && n0 + nn < N) ? Mp[(int64_t)(k0 + kk) * N + n0 + nn] : T(0);
  }
  __syncthreads();
  // thread -> (column nn, run of KPL consecutive k): one 16-byte chunk of the tiled matrix
  for (int o = threadIdx.x; o < 64 * (64 / KPL); o += blockDim.x) {
    const int nn = o / (64 / KPL), kk = (o % (64 / KPL)) * KPL;
    const int n = n0 + nn, k = k0 + kk;
    if (n >= N || k >= K) continue;  // K % KPL == 0: a chunk is whole or absent
    T v[KPL];
#pragma unroll
    for (int j = 0; j < KPL; ++j) v[j] = tile[kk + j][nn];
    *reinterpret_cast<uint4 *>(Mt + mtile_index<T>(n, k, K)) = *reinterpret_cast<const uint4 *>(v);
  }
}

// ---------------------------------------------------------------------------
// (a0) compression of new tokens.  Rows are (sequence, token) pairs of one KV
// head g; every wavefront walks its own 16-row blocks:
//   Z  = V A_g                                (MFMA)  -> stored latent z_s (rounded)
//   R  = K E_g - z_s[:, :r_b] (P_g E_g)       (MFMA)  -> stored residual (rounded)
// i.e. r = (k - z_s P_g) E_g with the product taken in the other association
// (same value up to float32 rounding), and K is copied into its pages.  The
// workgroup stages A_g and E_g transposed (every B fragment one contiguous k
// run) and forms P_g E_g once with MFMA (bf16: kept as hi + lo bf16 terms, so
// no precision is lost before the product).  A wavefront's V and K rows go
// straight from HBM into the A fragments, the next block's requested while
// the current one is computed; its latents and residuals pass through a
// wavefront-private LDS tile to the page stores, so wavefronts never wait for
// one another.
// grid (workgroups per head, n_kv), 256 threads, dynamic LDS.
// ---------------------------------------------------------------------------
struct CompressArgs {
  int batch, n_tokens, n_kv, rv, rb, rq, rb_pad, max_pages, num_phys, page_size, cap;
  PoolGeom geom;  // chunk positions of the latent and residual pages
};

// LDS rows are padded by 16 bytes, so the 16 rows a fragment load touches
// start in different banks.
template <typename T>
struct CompressLds {  // byte offsets into the dynamic LDS block; strides in elements
  int at, et, pe_hi, pe_lo, wave0, per_wave, zs_stride, fs, pe_stride, total;
  __host__ __device__ CompressLds(int rv, int rq, int rb_pad) {
    constexpr int KS = sizeof(T) == 2 ? 32 : 4;
    constexpr int PAD = 16 / (int)sizeof(T);
    const int rv_pad = (rv + KS - 1) / KS * KS;
    const int e = (int)sizeof(T);
    fs = kHeadDim + PAD;
    pe_stride = rb_pad + PAD;
    zs_stride = rv_pad + PAD;
    at = 0;
    et = at + rv * fs * e;
    pe_hi = et + rq * fs * e;
    pe_lo = pe_hi + rq * pe_stride * e;
    wave0 = pe_lo + (sizeof(T) == 2 ? rq * pe_stride * e : 0);
    per_wave = ((16 * zs_stride + 16 * rq) * e + 15) / 16 * 16;
    total = wave0 + 4 * per_wave;
  }
};

// T: input and factor elements; C: cache elements (T, or E4M3 codes beside
// bf16 inputs: the latent and residual tiles then hold E4M3-rounded values in
// bf16, which is exact, and the Key is rounded on its way to the pages).
template <typename T, typename C>
__global__ __launch_bounds__(256) void compress_kernel(
    const T *__restrict__ kin, const T *__restrict__ vin, const int32_t *__restrict__ start_pos,
    const T *__restrict__ A, const T *__restrict__ P, const T *__restrict__ E,
    C *__restrict__ zpool, C *__restrict__ rpool, C *__restrict__ kpool,
    const int32_t *__restrict__ block_table, CompressArgs a) {
  using MF = typename MfmaFor<T>::type;
  using frag = typename MF::frag;
  constexpr int CE = Elem<T>::CE;
  constexpr int CC = Elem<C>::CE;  // cache elements per 16-byte chunk
  constexpr bool kFp8 = sizeof(C) == 1;
  static_assert(sizeof(C) == sizeof(T) || (kFp8 && sizeof(T) == 2), "E4M3 goes with bf16 inputs");
  // a float32 result as it is stored (cache rounding), in the tile's type T
  auto stored = [](float x) {
    if constexpr (kFp8) return from_f32<T>(round_to<C>(x));
    else return from_f32<T>(x);
  };
  constexpr int DH = kHeadDim;
  constexpr bool kBf = sizeof(T) == 2;
  constexpr int NKS = DH / MF::KS;  // k steps over head_dim
  extern __shared__ __align__(16) unsigned char smem[];
  const CompressLds<T> L(a.rv, a.rq, a.rb_pad);
  T *At = reinterpret_cast<T *>(smem + L.at);        // [rv][fs]
  T *Et = reinterpret_cast<T *>(smem + L.et);        // [rq][fs]
  T *PEh = reinterpret_cast<T *>(smem + L.pe_hi);    // [rq][pe_stride]: (P E)^T, hi term
  T *PEl = reinterpret_cast<T *>(smem + L.pe_lo);    // bf16: lo term
  const int fs = L.fs, ps = L.pe_stride;
  const int g = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i = lane & 15, qg = lane >> 4;
  T *Zs = reinterpret_cast<T *>(smem + L.wave0 + wave * L.per_wave);  // [16][zs_stride]
  T *Rs = Zs + 16 * L.zs_stride;                                       // [16][rq]

  // ---- stage A_g and E_g transposed ----
  const T *Ag = A + (int64_t)g * DH * a.rv;
  const T *Pg = P + (int64_t)g * a.rb * DH;
  const T *Eg = E + (int64_t)g * DH * a.rq;
  // thread (d, chunk): one 16-byte chunk of row d in, CE column entries out
  // (consecutive threads write consecutive d: no bank conflicts)
  auto stage_t = [&](const T *src, int width, T *dst) {
    for (int o = threadIdx.x; o < DH * (width / CE); o += blockDim.x) {
      const int d = o % DH, c0 = (o / DH) * CE;
      float x[CE];
      unpack_chunk<T>(*reinterpret_cast<const uint4 *>(src + (int64_t)d * width + c0), x);
#pragma unroll
      for (int e = 0; e < CE; ++e) dst[(c0 + e) * fs + d] = from_f32<T>(x[e]);
    }
  };
  stage_t(Ag, a.rv, At);
  stage_t(Eg, a.rq, Et);
  __syncthreads();

  // ---- P_g E_g: tile (j tile, m tile) per wavefront, A = rows of P_g ----
  {
    const int jt_n = a.rb_pad / 16, mt_n = a.rq / 16;
    for (int t = wave; t < jt_n * mt_n; t += 4) {
      const int jt = t / mt_n, mt = t % mt_n;
      const int j = jt * 16 + i;
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
      for (int ks = 0; ks < NKS; ++ks) {
        const int k = ks * MF::KS + qg * MF::KPL;
        frag af, bfr;
        if constexpr (kBf) {
          af = bits_to_frag(j < a.rb ? *reinterpret_cast<const uint4 *>(Pg + (int64_t)j * DH + k)
                                     : make_uint4(0, 0, 0, 0));
          bfr = bits_to_frag(*reinterpret_cast<const uint4 *>(Et + (mt * 16 + i) * fs + k));
        } else {
          af = j < a.rb ? reinterpret_cast<const float *>(Pg)[(int64_t)j * DH + k] : 0.f;
          bfr = reinterpret_cast<const float *>(Et)[(mt * 16 + i) * fs + k];
        }
        acc = MF::mma(af, bfr, acc);
      }
      // lane holds (P E)[jt*16 + 4 qg + r][mt*16 + i]
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int jj = jt * 16 + qg * 4 + r, mm = mt * 16 + i;
        if constexpr (kBf) {
          const uint16_t hi = f32_to_bf16(acc[r]);
          PEh[mm * ps + jj] = hi;
          PEl[mm * ps + jj] = f32_to_bf16(acc[r] - bf16_to_f32(hi));
        } else {
          reinterpret_cast<float *>(PEh)[mm * ps + jj] = acc[r];
        }
      }
    }
  }
  __syncthreads();

  const int rows = a.batch * a.n_tokens;
  const int n_blocks = (rows + 15) / 16;
  const int zc_total = a.rv / CC, rc_total = a.rq / CC, kc_total = DH / CC;

  // A fragments of one 16-row block: lane (i, qg) holds row i's k slots of every k step
  frag va[NKS], ka[NKS];
  auto load_rows = [&](int blk, frag (&v)[NKS], frag (&k)[NKS]) {
    const int row = blk * 16 + i;
    const bool ok = blk < n_blocks && row < rows;
    const int sb = ok ? row / a.n_tokens : 0;
    const int st = ok ? row - sb * a.n_tokens : 0;
    const int64_t off = (((int64_t)sb * a.n_tokens + st) * a.n_kv + g) * DH;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const int kk = ks * MF::KS + qg * MF::KPL;
      if constexpr (kBf) {
        v[ks] = bits_to_frag(ok ? *reinterpret_cast<const uint4 *>(vin + off + kk)
                                : make_uint4(0, 0, 0, 0));
        k[ks] = bits_to_frag(ok ? *reinterpret_cast<const uint4 *>(kin + off + kk)
                                : make_uint4(0, 0, 0, 0));
      } else {
        v[ks] = ok ? reinterpret_cast<const float *>(vin)[off + kk] : 0.f;
        k[ks] = ok ? reinterpret_cast<const float *>(kin)[off + kk] : 0.f;
      }
    }
  };
  const int n_waves = gridDim.x * 4;
  int blk = blockIdx.x * 4 + wave;
  load_rows(blk, va, ka);
  for (; blk < n_blocks; blk += n_waves) {  // wavefront-uniform
    // this block's destination slots, looked up while the MFMAs run
    const int row = blk * 16 + i;
    int phys = -1, slot = 0;
    if (row < rows) {
      const int b = row / a.n_tokens, t = row - b * a.n_tokens;
      const int pos = start_pos[b] + t;
      if (pos >= 0 && pos < a.cap) {
        const int page = pos / a.page_size;
        slot = pos - page * a.page_size;
        const int ph = block_table[(int64_t)b * a.max_pages + page];
        if (ph >= 0 && ph < a.num_phys) phys = ph;
      }
    }
    // the next block's rows, in flight during this one (bf16)
    frag vn[kBf ? NKS : 1], kn[kBf ? NKS : 1];
    if constexpr (kBf) load_rows(blk + n_waves, vn, kn);

    // ---- Z = V A ----
    for (int nt = 0; nt < a.rv / 16; ++nt) {
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const int k = ks * MF::KS + qg * MF::KPL;
        frag bfr;
        if constexpr (kBf)
          bfr = bits_to_frag(*reinterpret_cast<const uint4 *>(At + (nt * 16 + i) * fs + k));
        else
          bfr = reinterpret_cast<const float *>(At)[(nt * 16 + i) * fs + k];
        acc = MF::mma(va[ks], bfr, acc);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) Zs[(qg * 4 + r) * L.zs_stride + nt * 16 + i] = stored(acc[r]);
    }
    for (int o = lane; o < 16 * (L.zs_stride - a.rv); o += 64) {
      const int rr = o / (L.zs_stride - a.rv), cc = a.rv + o % (L.zs_stride - a.rv);
      Zs[rr * L.zs_stride + cc] = from_f32<T>(0.f);
    }
    wave_lds_sync();

    // ---- R = K E - z_s (P E) ----
    for (int nt = 0; nt < a.rq / 16; ++nt) {
      floatx4 acc_k = {0.f, 0.f, 0.f, 0.f}, acc_z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const int k = ks * MF::KS + qg * MF::KPL;
        frag bfr;
        if constexpr (kBf)
          bfr = bits_to_frag(*reinterpret_cast<const uint4 *>(Et + (nt * 16 + i) * fs + k));
        else
          bfr = reinterpret_cast<const float *>(Et)[(nt * 16 + i) * fs + k];
        acc_k = MF::mma(ka[ks], bfr, acc_k);
      }
      for (int ks = 0; ks < a.rb_pad / MF::KS; ++ks) {
        const int k = ks * MF::KS + qg * MF::KPL;  // latent dims past r_b meet zero rows of P E
        if constexpr (kBf) {
          const frag af = bits_to_frag(*reinterpret_cast<const uint4 *>(Zs + i * L.zs_stride + k));
          const frag bh = bits_to_frag(*reinterpret_cast<const uint4 *>(PEh + (nt * 16 + i) * ps + k));
          const frag bl = bits_to_frag(*reinterpret_cast<const uint4 *>(PEl + (nt * 16 + i) * ps + k));
          acc_z = MF::mma(af, bh, acc_z);
          acc_z = MF::mma(af, bl, acc_z);
        } else {
          const frag af = reinterpret_cast<const float *>(Zs)[i * L.zs_stride + k];
          acc_z = MF::mma(af, reinterpret_cast<const float *>(PEh)[(nt * 16 + i) * ps + k],
                          acc_z);
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r)
        Rs[(qg * 4 + r) * a.rq + nt * 16 + i] = stored(acc_k[r] - acc_z[r]);
    }
    wave_lds_sync();

    // ---- page stores: latent and residual chunks from LDS, Key chunks from the fragments ----
    const int64_t hp_own = (int64_t)g * a.num_phys + phys;
    // tile chunk c goes to page chunk first + (c < split ? c : c + shift) of a
    // pool page of page_chunks chunks
    auto store_tile = [&](const T *tile, int stride, int n_chunks, C *pool, int page_chunks,
                          int first, int split, int shift) {
      for (int it = 0; it < (16 * n_chunks + 63) / 64; ++it) {
        const int o = it * 64 + lane;
        const int rr = o < 16 * n_chunks ? o / n_chunks : 0, c = o - rr * n_chunks;
        const int ph = __shfl(phys, rr), sl = __shfl(slot, rr);
        if (o < 16 * n_chunks && ph >= 0) {
          const int64_t hp = (int64_t)g * a.num_phys + ph;
          uint4 val;
          if constexpr (kFp8) {  // 16 tile values (already E4M3 values) -> 16 codes
            float x[16];
            unpack_chunk<T>(*reinterpret_cast<const uint4 *>(tile + rr * stride + c * CC), x);
            unpack_chunk<T>(*reinterpret_cast<const uint4 *>(tile + rr * stride + c * CC + 8), x + 8);
            val = make_uint4(f32x4_to_fp8x4(x[0], x[1], x[2], x[3]),
                             f32x4_to_fp8x4(x[4], x[5], x[6], x[7]),
                             f32x4_to_fp8x4(x[8], x[9], x[10], x[11]),
                             f32x4_to_fp8x4(x[12], x[13], x[14], x[15]));
          } else {
            val = *reinterpret_cast<const uint4 *>(tile + rr * stride + c * CC);
          }
          const int pc = first + (c < split ? c : c + shift);
          *reinterpret_cast<uint4 *>(reinterpret_cast<char *>(pool) +
                                     ((hp * page_chunks + pc) * a.page_size + sl) * 16) = val;
        }
      }
    };
    store_tile(Zs, L.zs_stride, zc_total, zpool, a.geom.z_page_chunks, 0, a.geom.z_split,
               a.geom.z_shift);
    store_tile(Rs, a.rq, rc_total, rpool, a.geom.r_page_chunks, a.geom.r_first, rc_total, 0);
    if (phys >= 0) {
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const int k = ks * MF::KS + qg * MF::KPL;  // element k of this lane's row
        char *base = reinterpret_cast<char *>(kpool) +
                     ((hp_own * kc_total + k / CC) * a.page_size + slot) * 16;
        if constexpr (kFp8) {  // 8 Key elements -> 8 codes, half a chunk
          float x[8];
          unpack_chunk<T>(__builtin_bit_cast(uint4, ka[ks]), x);
          *reinterpret_cast<uint2 *>(base + k % CC) =
              make_uint2(f32x4_to_fp8x4(x[0], x[1], x[2], x[3]), f32x4_to_fp8x4(x[4], x[5], x[6], x[7]));
        } else if constexpr (kBf) {
          *reinterpret_cast<uint4 *>(base) = __builtin_bit_cast(uint4, ka[ks]);
        } else {
          reinterpret_cast<float *>(base)[k % CE] = ka[ks];
        }
      }
    }
    wave_lds_sync();  // the tiles are read before the next block overwrites them
    if constexpr (kBf) {
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        va[ks] = vn[ks];
        ka[ks] = kn[ks];
      }
    } else {
      load_rows(blk + n_waves, va, ka);
    }
  }
}

template <typename T>
static size_t compress_lds_bytes(const basiskv_dims &d, int rb_pad) {
  return (size_t)CompressLds<T>(d.r_v, d.r_q, rb_pad).total;
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
  // up to 4 row tiles per workgroup; larger batches take more row-tile groups
  dim3 grid((N + 15) / 16, rt <= 4 ? 1 : (rt + 3) / 4), block(64 * kReconWaves);
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
  return act_bf16(d) ? recon_t<uint16_t>(d, u, u_tiles, M, y, s)
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
  return act_bf16(d) ? fuse_t<uint16_t>(d, Bf, W_O, M, s) : fuse_t<float>(d, Bf, W_O, M, s);
}

template <typename T>
static hipError_t pack_t(const basiskv_dims &d, const void *Mp, void *M, hipStream_t s) {
  const int K = d.n_q_heads * d.r_v, N = d.hidden;
  hipLaunchKernelGGL(pack_kernel<T>, dim3((N + 63) / 64, (K + 63) / 64), dim3(256), 0, s,
                     (const T *)Mp, (T *)M, K, N);
  return hipGetLastError();
}

hipError_t launch_pack_output(const basiskv_dims &d, const void *M_plain, void *M, hipStream_t s) {
  return act_bf16(d) ? pack_t<uint16_t>(d, M_plain, M, s) : pack_t<float>(d, M_plain, M, s);
}

#ifndef BKV_COMPRESS_WGS
#define BKV_COMPRESS_WGS 96
#endif
constexpr int kCompressWgsPerHead = BKV_COMPRESS_WGS;

template <typename T, typename C>
static hipError_t compress_t(const basiskv_dims &d, const void *k, const void *v,
                             const int32_t *start_pos, int32_t n_tokens, const void *A,
                             const void *P, const void *E, const basiskv_cache &c, hipStream_t s) {
  const int pad = sizeof(T) == 2 ? 32 : 16;  // a whole number of k steps and of 16-row tiles
  CompressArgs a;
  a.batch = d.batch;
  a.n_tokens = n_tokens;
  a.n_kv = d.n_kv_heads;
  a.rv = d.r_v;
  a.rb = d.r_b;
  a.rq = d.r_q;
  a.rb_pad = (d.r_b + pad - 1) / pad * pad;
  a.max_pages = d.max_pages_per_seq;
  a.num_phys = d.num_phys_pages;
  a.page_size = d.page_size;
  a.cap = d.max_pages_per_seq * d.page_size;
  a.geom = pool_geom(d);
  const size_t lds = compress_lds_bytes<T>(d, a.rb_pad);
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&compress_kernel<T, C>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  const int rows = d.batch * n_tokens;
  const int n_blocks = (rows + 15) / 16;
  int wgs = (n_blocks + 3) / 4;
  if (wgs > kCompressWgsPerHead) wgs = kCompressWgsPerHead;  // persistent: factors staged once each
  hipLaunchKernelGGL((compress_kernel<T, C>), dim3(wgs, d.n_kv_heads), dim3(256), lds, s,
                     (const T *)k, (const T *)v, start_pos, (const T *)A, (const T *)P,
                     (const T *)E, (C *)c.z_pages, (C *)residual_pool(d, c), (C *)c.k_pages,
                     c.block_table, a);
  return hipGetLastError();
}

// One token per sequence (the decode append, at any batch: the same kernel
// body as the one-call decode step's, so both give the same bits) or few rows
// per head: matrix-vector kernel; otherwise MFMA.
constexpr int kAppendMaxRows = 64;

hipError_t launch_compress(const basiskv_dims &d, const void *k, const void *v,
                           const int32_t *start_pos, int32_t n_tokens, const void *A,
                           const void *P, const void *E, const basiskv_cache &c, hipStream_t s) {
  const bool few = n_tokens == 1 || (int64_t)d.batch * n_tokens <= kAppendMaxRows;
  if (few && d.r_v <= kHeadDim && d.r_q <= kHeadDim)
    return launch_append(d, k, v, start_pos, n_tokens, A, P, E, c, s);
  if (cache_fp8(d))
    return compress_t<uint16_t, uint8_t>(d, k, v, start_pos, n_tokens, A, P, E, c, s);
  return act_bf16(d) ? compress_t<uint16_t, uint16_t>(d, k, v, start_pos, n_tokens, A, P, E, c, s)
                     : compress_t<float, float>(d, k, v, start_pos, n_tokens, A, P, E, c, s);
}

size_t compress_lds(const basiskv_dims &d) {
  const int pad = act_bf16(d) ? 32 : 16;
  const int rb_pad = (d.r_b + pad - 1) / pad * pad;
  return act_bf16(d) ? compress_lds_bytes<uint16_t>(d, rb_pad)
                     : compress_lds_bytes<float>(d, rb_pad);
}

}  // namespace bkv_host
