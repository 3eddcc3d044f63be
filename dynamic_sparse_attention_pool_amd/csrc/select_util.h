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

}  // namespace sa
