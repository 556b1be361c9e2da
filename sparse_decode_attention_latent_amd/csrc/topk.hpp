// Exact top-k of one score row per workgroup (or wavefront): the selection
// step of BasisKV's routing (arXiv 2611.02583, Table 9's caption: pages are
// chosen by score under a page budget).
//
// Scores become order-preserving 32-bit keys held in registers, up to KPT per
// lane.  The k-th largest key tau is built from the top.  Bits that every
// valid key shares -- above the highest bit in which the largest and smallest
// keys differ -- are taken as given.  A row held by one wavefront resolves
// one bit per round (a candidate is kept when at least k keys reach it;
// counts by ballots); a row held by several wavefronts resolves 8 bits per
// round (a histogram of the next digit over the keys that share the decided
// bits, by LDS atomics, and a suffix scan over its 256 bins), paying one
// barrier pair per digit instead of one per bit.  For rows held by 16
// wavefronts (over 4096 pages) the first digit is
// not a bit field but one of 256 equal-width buckets of the score range
// [min, max]: a bucket index is a monotone function of the score, so the k-th
// largest key lies in one bucket T, every key of a higher bucket is taken and
// the search goes on over T's keys only: while they are at most 1024, each is
// ranked against the others in LDS (the k-th largest is the key with fewer
// than the remaining rank above it and at least that many at or above it),
// otherwise by bit digits from the highest bit in which they differ.  (The
// leading bits of a row's keys are sign and exponent: as a first digit they
// fall in a handful of bins -- most keys in one, its LDS atomics serialised --
// when a row holds scores of both signs.  On rows held by four wavefronts the
// extra phase measured slower.)  Rows whose range is not a finite positive
// number, or so small that 256 / range overflows, start with the bit digits.
// Either way the search stops as soon as exactly k keys share the decided
// bits (the top-k set is then
// decided, whatever the lower bits of the k-th key).  The compaction
// then hands out, in page order, every page whose key exceeds tau and the
// lowest-index pages equal to it; positions come from ballot popcounts.
#pragma once
#include "common.hpp"

namespace bkv {

#ifndef BKV_TOPK_RADIX_WAVES
#define BKV_TOPK_RADIX_WAVES 4
#endif
constexpr int kTopkRadixWaves = BKV_TOPK_RADIX_WAVES;  // rows this wide search by digits
#ifndef BKV_TOPK_BUCKET_WAVES
#define BKV_TOPK_BUCKET_WAVES 16
#endif
constexpr int kTopkBucketWaves = BKV_TOPK_BUCKET_WAVES;  // rows this wide start with value buckets

// Order-preserving key of a score: larger score, larger key.  -0 and +0 are
// one key; NaN ranks below every number; 0 is left for lanes past the row.
__device__ __forceinline__ uint32_t order_key(float f) {
  if (f != f) return 1u;
  uint32_t u = __float_as_uint(f == 0.f ? 0.f : f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// The score of an order key (inverse of order_key; NaN for key 1).
__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_move_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

// Wavefront-uniform maximum and minimum of unsigned values.
__device__ __forceinline__ void wave_max_min_u32(uint32_t &mx, uint32_t &mn) {
#define BKV_STEP(C)                            \
  mx = max(mx, dpp_move_u32<C>(mx));           \
  mn = min(mn, dpp_move_u32<C>(mn));
  BKV_STEP(0xB1) BKV_STEP(0x4E) BKV_STEP(0x141) BKV_STEP(0x140)
#undef BKV_STEP
  uint32_t a = 0, b = ~0u;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    a = max(a, (uint32_t)__builtin_amdgcn_readlane((int)mx, 16 * r));
    b = min(b, (uint32_t)__builtin_amdgcn_readlane((int)mn, 16 * r));
  }
  mx = a;
  mn = b;
}

// Top-k of one score row, run by NWV whole wavefronts (threads 0 .. 64 NWV - 1).
// Page i = 64 (kpt w + j) + l is held by lane l of wavefront w as key j, for
// j < kpt <= KPT (kpt is uniform; a wavefront loads 64 consecutive scores per
// instruction); v[j] is its score (any value past the row).  Requires
// NP <= 64 NWV kpt and 1 <= k < NP.  emit(pos, j) is called by the lane
// holding the selected page 64 (kpt w + j) + l at position pos (page order).
template <int KPT, int NWV, typename Emit>
__device__ __forceinline__ void topk_row(const float (&v)[KPT], int kpt, int NP, int k,
                                         Emit &&emit) {
  __shared__ int xch[2][NWV > 1 ? NWV : 1][2];
  // several wavefronts: radix digits (one barrier pair per 8 bits); one: bits
  constexpr bool kRadix = NWV >= kTopkRadixWaves;
  __shared__ int hist[kRadix ? 256 : 1];
  __shared__ int found[kRadix ? 3 : 1];
  // bucket rows: bucket T's keys, ranked directly when they are few
  constexpr bool kBucket = NWV >= kTopkBucketWaves;
  constexpr int kMaxCand = 1024;
  __shared__ uint32_t cand[kBucket ? kMaxCand : 1];
  __shared__ int n_cand;
  __shared__ uint32_t tau_found;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int base = wave * 64 * kpt + lane;
  const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  uint32_t key[KPT];
  uint32_t kmax = 0u, kmin = ~0u;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const bool ok = j < kpt && base + 64 * j < NP;
    key[j] = ok ? order_key(v[j]) : 0u;
    kmax = ok ? max(kmax, key[j]) : kmax;
    kmin = ok ? min(kmin, key[j]) : kmin;
  }
  // ---- leading bits shared by every valid key ----
  wave_max_min_u32(kmax, kmin);
  if (NWV > 1) {
    if (lane == 0) {
      xch[0][wave][0] = (int)kmax;
      xch[0][wave][1] = (int)kmin;
    }
    if constexpr (kRadix) {  // the first histogram's bins cleared under the same barrier
      for (int i = threadIdx.x; i < 256; i += 64 * NWV) hist[i] = 0;
      if (threadIdx.x == 0) n_cand = 0;
    }
    __syncthreads();
    kmax = 0u;
    kmin = ~0u;
#pragma unroll
    for (int w = 0; w < NWV; ++w) {
      kmax = max(kmax, (uint32_t)xch[0][w][0]);
      kmin = min(kmin, (uint32_t)xch[0][w][1]);
    }
    // the bit search below rewrites xch at once; the digit search touches xch[0]
    // again only in the compaction, barriers later
    if constexpr (!kRadix) __syncthreads();
  }
  const uint32_t diff = kmax ^ kmin;
  const int top = diff ? 31 - __clz(diff) : -1;  // -1: every valid key is equal
  uint32_t tau = top < 0 ? kmax : top == 31 ? 0u : kmax & ~((2u << top) - 1u);
  if constexpr (kRadix) {
    // ---- tau, 8 bits at a time: histogram of the next digit of the keys that
    // share the bits decided so far (LDS atomics), then one wavefront finds the
    // digit holding the k-th largest key by a suffix scan over the bins ----
    const int tid = threadIdx.x;
    constexpr int NT = 64 * NWV;
    int krem = k;  // rank of the k-th largest key among the keys still searched
    uint32_t live = 0u;  // bit j: key j takes part in the search
#pragma unroll
    for (int j = 0; j < KPT; ++j)
      if (j < kpt && base + 64 * j < NP) live |= 1u << j;
    // wavefront 0 finds the bin holding the krem-th largest key; all read found[]
    auto find_bin = [&]() {
      if (wave == 0) {
        int c[4], s = 0;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          c[t] = hist[4 * lane + t];
          s += c[t];
        }
        int suf = s;  // inclusive suffix sum over lanes >= this one
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const int o = __shfl_down(suf, off);
          if (lane + off < 64) suf += o;
        }
        int above = suf - s;  // keys in the bins of higher lanes
#pragma unroll
        for (int t = 3; t >= 0; --t) {
          if (above < krem && above + c[t] >= krem) {
            found[0] = 4 * lane + t;
            found[1] = above;
            found[2] = c[t];
          }
          above += c[t];
        }
      }
      __syncthreads();
    };
    int hi = top;
    bool hist_clear = true;  // hist holds zeros
    // ---- first digit: equal-width buckets of the score range ----
    const float smax = key_value(kmax), smin = key_value(kmin);
    const float range = smax - smin;
    // the bucket index (x - smin) * 256 / range needs a finite, positive range
    // whose reciprocal scale is finite too (a range below 256 / FLT_MAX, about
    // 7.5e-37, would give an infinite scale): other rows take the bit digits
    const float scale = range > 0.f ? 256.f / range : 0.f;
    if (NWV >= kTopkBucketWaves && top >= 0 && __builtin_isfinite(range) &&
        range > 0.f && __builtin_isfinite(scale)) {  // smin, smax finite too
      auto bucket = [&](float x) { return min(255, (int)((x - smin) * scale)); };
#pragma unroll
      for (int j = 0; j < KPT; ++j)
        if ((live >> j) & 1u) atomicAdd(&hist[bucket(v[j])], 1);
      __syncthreads();
      find_bin();
      hist_clear = false;
      const int T = found[0];
      krem -= found[1];
      // bucket T's keys: gathered into cand[] (while they fit), and their
      // largest and smallest for the bit digits otherwise
      uint32_t mx = 0u, mn = ~0u;
#pragma unroll
      for (int j = 0; j < KPT; ++j) {
        if (((live >> j) & 1u) && bucket(v[j]) == T) {
          mx = max(mx, key[j]);
          mn = min(mn, key[j]);
          const int pos = atomicAdd(&n_cand, 1);
          if (pos < kMaxCand) cand[pos] = key[j];
        } else {
          live &= ~(1u << j);
        }
      }
      __syncthreads();
      const int nc = n_cand;  // uniform
      if (nc <= kMaxCand) {
        // tau is the krem-th largest of the nc candidates: the key with fewer
        // than krem candidates above it and at least krem at or above it (any
        // thread holding that value writes it)
        for (int i = tid; i < nc; i += NT) {
          const uint32_t ki = cand[i];
          int gt = 0, ge = 0;
          for (int j2 = 0; j2 < nc; ++j2) {
            const uint32_t kj = cand[j2];
            gt += kj > ki;
            ge += kj >= ki;
          }
          if (gt < krem && krem <= ge) tau_found = ki;
        }
        __syncthreads();
        tau = tau_found;
        hi = -1;
      } else {
        wave_max_min_u32(mx, mn);
        if (lane == 0) {
          xch[1][wave][0] = (int)mx;
          xch[1][wave][1] = (int)mn;
        }
        __syncthreads();
        mx = 0u;
        mn = ~0u;
#pragma unroll
        for (int w = 0; w < NWV; ++w) {
          mx = max(mx, (uint32_t)xch[1][w][0]);
          mn = min(mn, (uint32_t)xch[1][w][1]);
        }
        const uint32_t d2 = mx ^ mn;
        hi = d2 ? 31 - __clz(d2) : -1;
        tau = hi < 0 ? mx : hi == 31 ? 0u : mx & ~((2u << hi) - 1u);
        if (found[2] == krem) {  // every key of bucket T is taken: tau is its least
          tau = mn;
          hi = -1;
        }
      }
      // (found[] and hist are rewritten only after the next barrier)
    }
    for (; hi >= 0;) {
      const int lo = hi >= 7 ? hi - 7 : 0;
      const uint32_t dmask = (2u << (hi - lo)) - 1u;
      // (after find_bin's barrier wavefront 0 has read the previous counts, and
      // found[] is rewritten only after the two barriers below)
      if (!hist_clear) {
        for (int i = tid; i < 256; i += NT) hist[i] = 0;
        __syncthreads();
      }
      hist_clear = false;
#pragma unroll
      for (int j = 0; j < KPT; ++j) {
        const bool match = hi == 31 || (key[j] >> (hi + 1)) == (tau >> (hi + 1));
        if (((live >> j) & 1u) && match) atomicAdd(&hist[(key[j] >> lo) & dmask], 1);
      }
      __syncthreads();
      find_bin();
      const int digit = found[0];
      krem -= found[1];
      tau |= (uint32_t)digit << lo;
      if (found[2] == krem) break;  // every key sharing these bits is taken
      hi = lo - 1;
    }
  } else {
  // ---- tau, bit by bit (keys past the row are 0 and reach no candidate) ----
  for (int bit = top; bit >= 0; --bit) {
    const uint32_t cand = tau | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < KPT; ++j)
      if (j < kpt) cnt += __popcll(__ballot(key[j] >= cand));
    if (NWV > 1) {
      if (lane == 0) xch[bit & 1][wave][0] = cnt;
      __syncthreads();
      cnt = 0;
#pragma unroll
      for (int w = 0; w < NWV; ++w) cnt += xch[bit & 1][w][0];
    }
    if (cnt >= k) tau = cand;
    if (cnt == k) break;  // exactly k keys reach tau: the set is decided (uniform)
  }
  }
  // ---- compaction in page order: every key above tau, then the lowest-index
  // keys equal to tau up to k in all (tau >= 1: keys past the row never take part;
  // after an early stop every key reaching tau is taken) ----
  int gt_run = 0, eq_run = 0, total_gt = 0;
  if (NWV > 1) {
    int gt_w = 0, eq_w = 0;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      if (j < kpt) {
        gt_w += __popcll(__ballot(key[j] > tau));
        eq_w += __popcll(__ballot(key[j] == tau));
      }
    }
    // the last reads of xch[0] (the bit search's, or the range exchange's when
    // every key is equal and the digit search took no barrier) are complete
    if (!kRadix || top < 0) __syncthreads();
    if (lane == 0) {
      xch[0][wave][0] = gt_w;
      xch[0][wave][1] = eq_w;
    }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < NWV; ++w) {
      const int g = xch[0][w][0], e = xch[0][w][1];
      total_gt += g;
      if (w < wave) {
        gt_run += g;
        eq_run += e;
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < KPT; ++j)
      if (j < kpt) total_gt += __popcll(__ballot(key[j] > tau));
  }
  const int need = k - total_gt;  // keys equal to tau to take (>= 1)
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    if (j < kpt) {
      const uint64_t m_gt = __ballot(key[j] > tau);
      const uint64_t m_eq = __ballot(key[j] == tau);
      const int eq_pos = eq_run + __popcll(m_eq & below);
      const bool take = key[j] > tau || (key[j] == tau && eq_pos < need);
      if (take) emit(gt_run + __popcll(m_gt & below) + min(eq_pos, need), j);
      gt_run += __popcll(m_gt);
      eq_run += __popcll(m_eq);
    }
  }
}

}  // namespace bkv
