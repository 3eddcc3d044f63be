// Workgroup scans and the radix k-th-largest search shared by the selection
// kernels (device code, included by the .hip sources that select).
#pragma once

#include "common.h"

namespace sa {

// Inclusive prefix sum within a wave (64 lanes, all active).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t x = __shfl_up(v, off);
    if (lane >= off) v += x;
  }
  return v;
}

// Exclusive prefix sum over the workgroup (wave scans, then the wave totals).
template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* tmp, uint32_t& total) {
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x, wv = tid >> 6;
  const uint32_t incl = wave_incl_scan(v);
  if ((tid & 63) == 63) tmp[wv] = incl;
  __syncthreads();
  uint32_t before = 0u, all = 0u;
#pragma unroll
  for (int j = 0; j < NW; ++j) {
    const uint32_t x = tmp[j];
    before += j < wv ? x : 0u;
    all += x;
  }
  total = all;
  __syncthreads();
  return before + incl - v;
}

// k-th largest key (1 <= k <= e-b) of key_at(b..e-1): MSB-first radix select
// with 8-bit digits and LDS histograms.  Returns T and how many keys equal to
// T belong to the top k.  Called by every thread of the workgroup.
// With top_shift < 24 the caller guarantees that all keys share their bits
// above top_shift + 8 with `known` (e.g. keys inside a bracket [lo, hi]); those
// digits are not counted again.
template <int NT, class KeyAt>
__device__ void radix_kth(KeyAt key_at, int64_t b, int64_t e, int64_t k, uint32_t* hist, uint32_t* tmp,
                          uint32_t* shv, uint32_t& T, int64_t& need, int top_shift = 24, uint32_t known = 0u) {
  const int tid = threadIdx.x;
  uint32_t pmask = top_shift >= 24 ? 0u : ~((1u << (top_shift + 8)) - 1u);
  uint32_t prefix = known & pmask;
  int64_t remaining = k;
  for (int shift = top_shift; shift >= 0; shift -= 8) {
    for (int d = tid; d < 256; d += NT) hist[d] = 0u;
    __syncthreads();
    for (int64_t i = b + tid; i < e; i += NT) {
      const uint32_t kk = key_at(i);
      if ((kk & pmask) == prefix) atomicAdd(&hist[(kk >> shift) & 255u], 1u);
    }
    __syncthreads();
    // suffix sums over the 256 digits (thread t: keys with digit >= 255-t),
    // by the first four waves
    uint32_t v = 0u, incl = 0u;
    if (tid < 256) {
      v = hist[255 - tid];
      incl = wave_incl_scan(v);
      if ((tid & 63) == 63) tmp[tid >> 6] = incl;
    }
    __syncthreads();
    if (tid < 256) {
      uint32_t before = 0u;
      for (int j = 0; j < (tid >> 6); ++j) before += tmp[j];
      const uint32_t ge = before + incl;
      const uint32_t gt = ge - v;
      if (gt < (uint32_t)remaining && (uint32_t)remaining <= ge) {
        shv[0] = 255u - tid;
        shv[1] = gt;
      }
    }
    __syncthreads();
    remaining -= shv[1];
    prefix |= shv[0] << shift;
    pmask |= 255u << shift;
    __syncthreads();
  }
  T = prefix;
  need = remaining;
}

// The k1-th and k2-th largest keys of [b, e) at once: the same digit search as
// radix_kth for each rank, with both ranks' histograms built in one sweep per
// pass (hist holds 512 bins, tmp 8 entries), so the two searches share their
// barriers.  Needs NT >= 512.
template <int NT, typename KeyAt>
__device__ void radix_kth2(KeyAt key_at, int64_t b, int64_t e, int64_t k1, int64_t k2, uint32_t* hist, uint32_t* tmp,
                           uint32_t* shv, uint32_t& T1, uint32_t& T2) {
  static_assert(NT >= 512, "two 256-digit scans run side by side");
  const int tid = threadIdx.x;
  uint32_t pmask = 0u, prefix1 = 0u, prefix2 = 0u;
  int64_t rem1 = k1, rem2 = k2;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int d = tid; d < 512; d += NT) hist[d] = 0u;
    __syncthreads();
    for (int64_t i = b + tid; i < e; i += NT) {
      const uint32_t kk = key_at(i);
      const uint32_t dg = (kk >> shift) & 255u;
      if ((kk & pmask) == prefix1) atomicAdd(&hist[dg], 1u);
      if ((kk & pmask) == prefix2) atomicAdd(&hist[256 + dg], 1u);
    }
    __syncthreads();
    // threads 0..255 scan rank 1's digits, 256..511 rank 2's (keys with digit >= 255 - t)
    const int r = tid >> 8, t = tid & 255;
    uint32_t v = 0u, incl = 0u;
    if (tid < 512) {
      v = hist[256 * r + 255 - t];
      incl = wave_incl_scan(v);
      if ((tid & 63) == 63) tmp[tid >> 6] = incl;
    }
    __syncthreads();
    if (tid < 512) {
      uint32_t before = 0u;
      for (int j = 4 * r; j < (tid >> 6); ++j) before += tmp[j];
      const uint32_t ge = before + incl;
      const uint32_t gt = ge - v;
      const int64_t rem = r == 0 ? rem1 : rem2;
      if (gt < (uint32_t)rem && (uint32_t)rem <= ge) {
        shv[2 * r] = 255u - t;
        shv[2 * r + 1] = gt;
      }
    }
    __syncthreads();
    rem1 -= shv[1];
    rem2 -= shv[3];
    prefix1 |= shv[0] << shift;
    prefix2 |= shv[2] << shift;
    pmask |= 255u << shift;
    __syncthreads();
  }
  T1 = prefix1;
  T2 = prefix2;
}

__device__ __forceinline__ float key_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k ^ 0x80000000u) : ~k);
}

__device__ __forceinline__ uint64_t wave_incl_scan_u64(uint64_t v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint64_t x = __shfl_up(v, off);
    if (lane >= off) v += x;
  }
  return v;
}

// Adaptive-budget selection of one row: the shortest prefix of the selection
// order (higher score first, lower index on ties) that holds `mass` of the
// row's softmax weight, clamped to [k_min, min(k_max, n)].  kv[0 .. P) holds
// (order key << 32 | ~index) for the n candidates and 0 for the padding up to
// P, a power of two >= 64; the caller has filled it and synchronised.
// Candidate j weighs exp(s_j - m), m the row maximum, and an entry equal to m
// weighs exactly 1.  kv is sorted by a bitonic network, a block scan sums the
// weights along that order, and a position is kept while the weight ahead of
// it is below mass * total.  The kept indices are marked in the bitmap bm
// (cleared here) and written in index order to out[0 .. count), then -1 up to
// kmax; *cnt_out = count.  Weights are fp32 exponentials rounded to multiples
// of 2^-40 and summed as 64-bit integers (4096 * 2^40 < 2^53), so every prefix
// is exact, the prefixes never decrease, and the last one is the total
// whatever the thread layout; the comparison with mass * total is made in
// double.  Called by all NT threads; n <= 32 * NT.
template <int NT>
__device__ void mass_select_lds(uint64_t* kv, uint32_t* bm, uint64_t* wtmp, uint32_t* utmp, int n, int P, float mass,
                                int k_min, int k_max, int32_t* out, int kmax, int32_t* cnt_out) {
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x, wv = tid >> 6;
  const int nw = (n + 31) >> 5;
  for (int w = tid; w < nw; w += NT) bm[w] = 0u;
  // bitonic network, descending: runs of length kk alternate direction until the last merge
  for (int kk = 2; kk <= P; kk <<= 1) {
    for (int j = kk >> 1; j > 0; j >>= 1) {
      for (int i = tid; i < P / 2; i += NT) {
        const int lo = ((i & ~(j - 1)) << 1) | (i & (j - 1)), hi = lo + j;
        const uint64_t a = kv[lo], b = kv[hi];
        if ((a < b) == ((lo & kk) == 0)) {
          kv[lo] = b;
          kv[hi] = a;
        }
      }
      __syncthreads();
    }
  }
  // weights along the sorted order: thread t owns positions [t*E, t*E + E)
  const float m = key_float((uint32_t)(kv[0] >> 32));
  const int E = P >= NT ? P / NT : 1;
  const int j0 = tid * E, j1 = min(n, j0 + E);
  auto weight = [&](int j) -> uint64_t {  // in units of 2^-40
    const float s = key_float((uint32_t)(kv[j] >> 32));
    const float w = s == m ? 1.f : expf(s - m);
    return __double2ull_rn((double)w * 1099511627776.0);
  };
  uint64_t part = 0ull;
  for (int j = j0; j < j1; ++j) part += weight(j);
  const uint64_t incl = wave_incl_scan_u64(part);
  if ((tid & 63) == 63) wtmp[wv] = incl;
  __syncthreads();
  uint64_t ahead = incl - part, total = 0ull;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const uint64_t x = wtmp[w];
    ahead += w < wv ? x : 0ull;
    total += x;
  }
  const double thr = (double)mass * (double)total;
  uint32_t kept_here = 0u;
  for (int j = j0; j < j1; ++j) {
    kept_here += (double)ahead < thr ? 1u : 0u;
    ahead += weight(j);
  }
  uint32_t c_raw;
  block_excl_scan<NT>(kept_here, utmp, c_raw);
  int c = max((int)c_raw, k_min);
  c = min(c, min(k_max, n));
  for (int j = tid; j < c; j += NT) {
    const uint32_t i = ~(uint32_t)kv[j];
    atomicOr(&bm[i >> 5], 1u << (i & 31u));
  }
  __syncthreads();
  // emission in index order: thread t owns bitmap word t (nw <= NT)
  const uint32_t word = tid < nw ? bm[tid] : 0u;
  uint32_t tot;
  uint32_t at = block_excl_scan<NT>((uint32_t)__popc(word), utmp, tot);
  uint32_t bits = word;
  while (bits) {
    const int b = __builtin_ctz(bits);
    bits &= bits - 1u;
    out[at++] = 32 * tid + b;
  }
  for (int j = c + tid; j < kmax; j += NT) out[j] = -1;
  if (tid == 0) *cnt_out = c;
}

}  // namespace sa
