// Exact per-row top-k with forced members, and the vertical-slash table build.
//
// Selection keeps the best-scoring subset ("MInference 1.0" article,
// §方法介紹; Squeezed Attention page, §技术方案; IndexCache article,
// §长文本的算力困境); the leading (sink) and trailing (local) candidates are
// always kept ("稀疏注意力机制解析" explainer, §1.2).  Because the forced
// members are a prefix and a suffix of the causal range, the ranked pool is one
// contiguous range [pb, pe).
//
// Method: scores become order-preserving 32-bit keys; a radix select finds the
// k-th largest key T and how many keys equal to T must be taken; one more pass
// emits, in index order, the forced members, every pool key > T and the
// lowest-index keys == T.  The emission order makes the output ascending and
// breaks ties toward the lower index, which is the required total order.
// Rows of up to 4096 candidates are staged in LDS once; rows of up to 131072
// are read once (k_select_long: sampled bracket, selection bitmaps in LDS);
// longer rows are read twice (bracketing pass + emission) when the sampled
// bracket holds.
#include <climits>

#include "common.h"
#include "launch.h"
#include "select_util.h"

namespace sa {
namespace {

// Row-wise selection.  IN_LDS: the row (<= 4096 candidates) is staged in LDS
// and ranked there.  Otherwise the threshold comes from a sample: 4096 evenly
// spaced pool keys bracket the k-th key between two sample ranks, one pass
// over the row counts the keys above the bracket and gathers the keys inside
// it into LDS, and the exact threshold is ranked among those.  When the
// bracket misses (or holds too many keys) a full radix select over the row
// runs instead, so the result never depends on the sample.
template <int NT, bool IN_LDS>
__global__ __launch_bounds__(NT) void k_select(SelectParams p) {
  constexpr int kLdsMax = 4096;
  constexpr int kSample = 4096;
  constexpr int kBand = 8192;
  __shared__ uint32_t keys[IN_LDS ? kLdsMax : kSample];
  __shared__ uint32_t band[IN_LDS ? 1 : kBand];
  __shared__ uint32_t hist[256];
  __shared__ uint32_t tmp[NT];
  __shared__ uint32_t shv[4];

  const int tid = threadIdx.x;
  const int64_t r = blockIdx.x;
  const float* row = p.scores + r * p.ld;
  const int64_t n = p.causal ? min(p.ncand, (r % p.period) + p.offset + 1) : p.ncand;
  const int64_t pb = min((int64_t)p.n_sink, n);
  const int64_t pe = max(pb, n - (int64_t)p.n_local);
  const int64_t npool = pe - pb;
  int64_t kr = p.rden > 0 ? ((int64_t)p.rnum * n + p.rden - 1) / p.rden : (int64_t)p.k;
  kr = max((int64_t)0, min(kr, npool));
  const bool take_all = (kr == npool);

  if (tid < 4) shv[tid] = 0u;
  __syncthreads();
  uint32_t T = 0xffffffffu;
  int64_t need = 0;  // keys equal to T that are taken
  if (IN_LDS) {
    bool nan_seen = false;
    for (int64_t i = tid; i < n; i += NT) {
      const float f = row[i];
      nan_seen |= is_nan(f);
      keys[i] = order_key(f);
    }
    if (nan_seen) atomicOr(&shv[2], 1u);
    __syncthreads();
    if (kr > 0 && !take_all)
      radix_kth<NT>([&](int64_t i) { return keys[i]; }, pb, pe, kr, hist, tmp, shv, T, need);
  } else {
    bool nan_seen = false;
    if (kr > 0 && !take_all) {
      // ---- bracket the threshold with a sample of the pool
      const int ns = (int)min((int64_t)kSample, npool);
      for (int s = tid; s < ns; s += NT) keys[s] = order_key(row[pb + ((int64_t)s * npool) / ns]);
      __syncthreads();
      const double frac = (double)kr * ns / (double)npool;
      const int margin = (int)(3.0 * sqrt(frac)) + 8;
      const int64_t rk_hi = max((int64_t)1, (int64_t)frac - margin);
      const int64_t rk_lo = min((int64_t)ns, (int64_t)ceil(frac) + margin);
      uint32_t hi, lo;
      int64_t dummy;
      radix_kth<NT>([&](int64_t i) { return keys[i]; }, 0, ns, rk_hi, hist, tmp, shv, hi, dummy);
      radix_kth<NT>([&](int64_t i) { return keys[i]; }, 0, ns, rk_lo, hist, tmp, shv, lo, dummy);
      // ---- one pass: keys above the bracket are counted, keys inside are gathered
      if (tid == 0) {
        shv[0] = 0u;  // keys > hi
        shv[1] = 0u;  // keys in [lo, hi]
      }
      __syncthreads();
      uint32_t above = 0u;
      for (int64_t i = pb + tid; i < pe; i += NT) {
        const float f = row[i];
        nan_seen |= is_nan(f);
        const uint32_t kk = order_key(f);
        if (kk > hi) ++above;
        else if (kk >= lo) {
          const uint32_t pos = atomicAdd(&shv[1], 1u);
          if (pos < (uint32_t)kBand) band[pos] = kk;
        }
      }
      atomicAdd(&shv[0], above);
      __syncthreads();
      const int64_t c_hi = shv[0], c_mid = shv[1];
      __syncthreads();
      if (c_hi < kr && kr <= c_hi + c_mid && c_mid <= kBand) {
        radix_kth<NT>([&](int64_t i) { return band[i]; }, 0, c_mid, kr - c_hi, hist, tmp, shv, T, need);
      } else {
        radix_kth<NT>([&](int64_t i) { return order_key(row[i]); }, pb, pe, kr, hist, tmp, shv, T, need);
      }
    }
    // NaN check over the forced members (and over the pool when it was not read)
    const bool pool_read = kr > 0 && !take_all;
    for (int64_t i = tid; i < n; i += NT)
      if (!pool_read || i < pb || i >= pe) nan_seen |= is_nan(row[i]);
    if (nan_seen) atomicOr(&shv[2], 1u);
    __syncthreads();
  }
  if (shv[2] && tid == 0 && p.err != nullptr) atomicOr(reinterpret_cast<unsigned int*>(p.err), 1u);

  auto key_at = [&](int64_t i) -> uint32_t { return IN_LDS ? keys[i] : order_key(row[i]); };

  // ---- emission in index order, tiles of NT*4 candidates
  int32_t* out = p.idx + r * p.kmax;
  uint32_t gtf_run = 0u, eq_run = 0u;  // selected-by-rank and tie counts before this tile
  for (int64_t t0 = 0; t0 < n; t0 += (int64_t)NT * 4) {
    const int64_t i0 = t0 + (int64_t)tid * 4;
    uint32_t f[4];
    uint32_t c_gtf = 0u, c_eq = 0u;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t i = i0 + e;
      uint32_t cls = 0u;  // 0 not taken, 1 taken, 2 tie candidate
      if (i < n) {
        if (i < pb || i >= pe) cls = 1u;
        else if (kr > 0) {
          if (take_all) cls = 1u;
          else {
            const uint32_t kk = key_at(i);
            cls = kk > T ? 1u : (kk == T ? 2u : 0u);
          }
        }
      }
      f[e] = cls;
      c_gtf += cls == 1u;
      c_eq += cls == 2u;
    }
    uint32_t tot;
    const uint32_t ex = block_excl_scan<NT>((c_eq << 16) | c_gtf, tmp, tot);
    uint32_t g_before = gtf_run + (ex & 0xffffu);
    uint32_t e_before = eq_run + (ex >> 16);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t i = i0 + e;
      if (f[e] == 1u) {
        const uint32_t pos = g_before + (uint32_t)min((int64_t)e_before, need);
        out[pos] = (int32_t)i;
        ++g_before;
      } else if (f[e] == 2u) {
        if ((int64_t)e_before < need) {
          const uint32_t pos = g_before + e_before;
          out[pos] = (int32_t)i;
        }
        ++e_before;
      }
    }
    gtf_run += tot & 0xffffu;
    eq_run += tot >> 16;
  }
  const int64_t total = (int64_t)gtf_run + min((int64_t)eq_run, need);
  for (int64_t j = total + tid; j < p.kmax; j += NT) out[j] = -1;
  if (tid == 0) p.cnt[r] = (int32_t)total;
}

// Exclusive prefix sums of two counters over the workgroup: wave scans by
// lane shuffles, then one pass over the wave totals.
template <int NT>
__device__ __forceinline__ void block_excl_scan2(uint32_t a, uint32_t b, uint32_t* wsum, uint32_t& ea, uint32_t& eb,
                                                 uint32_t& ta, uint32_t& tb) {
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  uint32_t ia = a, ib = b;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t xa = __shfl_up(ia, off), xb = __shfl_up(ib, off);
    if (lane >= off) {
      ia += xa;
      ib += xb;
    }
  }
  if (lane == 63) {
    wsum[2 * wv] = ia;
    wsum[2 * wv + 1] = ib;
  }
  __syncthreads();
  uint32_t pa = 0u, pb = 0u, sa = 0u, sb = 0u;
  for (int j = 0; j < NW; ++j) {
    const uint32_t va = wsum[2 * j], vb = wsum[2 * j + 1];
    if (j < wv) {
      pa += va;
      pb += vb;
    }
    sa += va;
    sb += vb;
  }
  ea = pa + ia - a;
  eb = pb + ib - b;
  ta = sa;
  tb = sb;
  __syncthreads();
}

// Long rows (4096 < candidates <= kBmMax), read once.  A sample of 256 runs of
// 16 consecutive pool keys (a few cache lines, not the whole row) brackets the
// k-th key; one pass over the row marks the keys above the bracket in an LDS
// bitmap and gathers (key, index) of the keys inside it; the exact threshold T
// is ranked among those, keys > T join the bitmap and keys == T go to a tie
// bitmap.  Emission walks the bitmaps in index order with one prefix sum, so
// the row is not read again.  When the bracket misses, the threshold comes
// from a radix select over the row and one more pass fills the bitmaps.
constexpr int kBmMax = 131072;

template <int NT>
__global__ __launch_bounds__(NT) void k_select_long(SelectParams p) {
  constexpr int kSample = 4096, kRun = 16, kBand = 4096, kWords = kBmMax / 32;
  // ~69 KB of LDS: two workgroups per CU, so one's ranking overlaps the other's pass
  __shared__ uint32_t keys[kSample];  // the sample, then the band's keys
  uint32_t* bk = keys;
  __shared__ int32_t bi[kBand];
  __shared__ uint32_t selbm[kWords];
  __shared__ uint32_t tiebm[kWords];
  __shared__ uint32_t hist[512];
  __shared__ uint32_t tmp[NT];
  __shared__ uint32_t shv[4];

  const int tid = threadIdx.x;
  const int64_t r = blockIdx.x;
  const float* row = p.scores + r * p.ld;
  const int n = (int)(p.causal ? min(p.ncand, (r % p.period) + p.offset + 1) : p.ncand);
  const int pb = min(p.n_sink, n);
  const int pe = max(pb, n - p.n_local);
  const int npool = pe - pb;
  int64_t kr = p.rden > 0 ? ((int64_t)p.rnum * n + p.rden - 1) / p.rden : (int64_t)p.k;
  kr = max((int64_t)0, min(kr, (int64_t)npool));
  const bool take_all = (kr == npool);
  const int nw = (n + 31) / 32;
  const bool aligned = (p.ld % 4) == 0 && (reinterpret_cast<uintptr_t>(p.scores) & 15) == 0;

  for (int w = tid; w < nw; w += NT) {
    selbm[w] = 0u;
    tiebm[w] = 0u;
  }
  if (tid < 4) shv[tid] = 0u;
  __syncthreads();

  bool nan_seen = false;
  uint32_t T = 0xffffffffu;
  int64_t need = 0;  // keys equal to T that are taken
  if (kr > 0 && !take_all) {
    // ---- bracket the threshold with a sample of the pool
    int ns;
    if (npool >= 2 * kSample) {
      ns = kSample;
      constexpr int nrun = kSample / kRun;
      for (int s = tid; s < ns; s += NT) {
        const int c = s / kRun;
        const int at = pb + (int)(((int64_t)c * (npool - kRun)) / (nrun - 1)) + s % kRun;
        keys[s] = order_key(row[at]);
      }
    } else {
      ns = min(kSample, npool);
      for (int s = tid; s < ns; s += NT) keys[s] = order_key(row[pb + ((int64_t)s * npool) / ns]);
    }
    __syncthreads();
    const double frac = (double)kr * ns / (double)npool;
    const int margin = (int)(3.0 * sqrt(frac)) + 8;
    const int64_t rk_hi = max((int64_t)1, (int64_t)frac - margin);
    const int64_t rk_lo = min((int64_t)ns, (int64_t)ceil(frac) + margin);
    uint32_t hi, lo;
    radix_kth2<NT>([&](int64_t i) { return keys[i]; }, 0, ns, rk_hi, rk_lo, hist, tmp, shv, hi, lo);
    if (tid == 0) {
      shv[0] = 0u;  // keys > hi
      shv[1] = 0u;  // keys in [lo, hi]
      shv[2] = 0u;  // the NaN flag below (the bracket search used it)
      shv[3] = 0u;
    }
    __syncthreads();
    // ---- the one pass over the pool.  Per key: its order key, a running
    // min / max of the keys (a NaN maps outside [key(-inf), key(+inf)]) and one
    // compare; only keys >= lo (a few percent) take the slow branch.
    uint32_t above = 0u, kmin = 0xffffffffu, kmax_ = 0u;
    auto slow = [&](int i, uint32_t kk) {
      if (kk > hi) {
        ++above;
        atomicOr(&selbm[i >> 5], 1u << (i & 31));
      } else {
        const uint32_t pos = atomicAdd(&shv[1], 1u);
        if (pos < (uint32_t)kBand) {
          bk[pos] = kk;
          bi[pos] = i;
        }
      }
    };
    if (aligned) {
      // 16-byte loads, 4 per thread in flight; the 4-aligned chunks covering
      // [pb, pe) stay inside the row's ld (a multiple of 4)
      const int c0 = pb >> 2, c1 = (pe + 3) >> 2;
      const f32x4* row4 = reinterpret_cast<const f32x4*>(row);
      for (int cb = c0 + tid; cb < c1; cb += 4 * NT) {
        f32x4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int c = cb + u * NT;
          if (c < c1) v[u] = row4[c];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int c = cb + u * NT;
          if (c < c1) {
            const bool inner = 4 * c >= pb && 4 * c + 3 < pe;
            uint32_t kk[4];
            bool hit = false;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              kk[e] = order_key(v[u][e]);
              const bool in = inner || (4 * c + e >= pb && 4 * c + e < pe);
              if (in) {
                kmin = min(kmin, kk[e]);
                kmax_ = max(kmax_, kk[e]);
                hit |= kk[e] >= lo;
              }
            }
            if (hit) {
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int i = 4 * c + e;
                if (kk[e] >= lo && i >= pb && i < pe) slow(i, kk[e]);
              }
            }
          }
        }
      }
    } else {
      for (int ib = pb + tid; ib < pe; ib += 8 * NT) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int i = ib + u * NT;
          if (i < pe) v[u] = row[i];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int i = ib + u * NT;
          if (i < pe) {
            const uint32_t kk = order_key(v[u]);
            kmin = min(kmin, kk);
            kmax_ = max(kmax_, kk);
            if (kk >= lo) slow(i, kk);
          }
        }
      }
    }
    // order keys of -inf and +inf: anything outside is a NaN
    nan_seen |= kmin < 0x007fffffu || kmax_ > 0xff800000u;
    atomicAdd(&shv[0], above);
    __syncthreads();
    const int64_t c_hi = shv[0], c_mid = shv[1];
    __syncthreads();
    if (c_hi < kr && kr <= c_hi + c_mid && c_mid <= kBand) {
      // band keys lie in [lo, hi]: they share every bit above the first one where lo and hi differ
      const int top = lo == hi ? 0 : ((31 - __builtin_clz(lo ^ hi)) / 8) * 8;
      radix_kth<NT>([&](int64_t i) { return bk[i]; }, 0, c_mid, kr - c_hi, hist, tmp, shv, T, need, top, lo);
      for (int j = tid; j < (int)c_mid; j += NT) {
        const int i = bi[j];
        if (bk[j] > T) atomicOr(&selbm[i >> 5], 1u << (i & 31));
        else if (bk[j] == T) atomicOr(&tiebm[i >> 5], 1u << (i & 31));
      }
    } else {
      // bracket missed: exact threshold over the whole pool, then the bitmaps afresh
      radix_kth<NT>([&](int64_t i) { return order_key(row[i]); }, pb, pe, kr, hist, tmp, shv, T, need);
      for (int w = tid; w < nw; w += NT) selbm[w] = 0u;
      __syncthreads();
      for (int i = pb + tid; i < pe; i += NT) {
        const uint32_t kk = order_key(row[i]);
        if (kk > T) atomicOr(&selbm[i >> 5], 1u << (i & 31));
        else if (kk == T) atomicOr(&tiebm[i >> 5], 1u << (i & 31));
      }
    }
  } else if (take_all) {
    for (int i = pb + tid; i < pe; i += NT) atomicOr(&selbm[i >> 5], 1u << (i & 31));
  }
  // forced members (and the NaN check over everything the pass did not read)
  const bool pool_read = kr > 0 && !take_all;
  for (int i = tid; i < pb; i += NT) {
    atomicOr(&selbm[i >> 5], 1u << (i & 31));
    nan_seen |= is_nan(row[i]);
  }
  for (int i = pe + tid; i < n; i += NT) {
    atomicOr(&selbm[i >> 5], 1u << (i & 31));
    nan_seen |= is_nan(row[i]);
  }
  if (!pool_read)
    for (int i = pb + tid; i < pe; i += NT) nan_seen |= is_nan(row[i]);
  if (nan_seen) atomicOr(&shv[2], 1u);
  __syncthreads();
  if (shv[2] && tid == 0 && p.err != nullptr) atomicOr(reinterpret_cast<unsigned int*>(p.err), 1u);

  // ---- emission in index order: thread t owns words [t*wpt, (t+1)*wpt)
  const int wpt = (nw + NT - 1) / NT;
  const int w0 = min(nw, tid * wpt), w1 = min(nw, w0 + wpt);
  uint32_t cs = 0u, ce = 0u;
  for (int w = w0; w < w1; ++w) {
    cs += __popc(selbm[w]);
    ce += __popc(tiebm[w]);
  }
  uint32_t g_before, e_before, tot_s, tot_e;
  block_excl_scan2<NT>(cs, ce, tmp, g_before, e_before, tot_s, tot_e);
  int32_t* out = p.idx + r * p.kmax;
  for (int w = w0; w < w1; ++w) {
    const uint32_t sw = selbm[w], tw = tiebm[w];
    uint32_t mbits = sw | tw;
    while (mbits) {
      const int bit = __builtin_ctz(mbits);
      mbits &= mbits - 1u;
      const int i = 32 * w + bit;
      if ((sw >> bit) & 1u) {
        out[g_before + (uint32_t)min((int64_t)e_before, need)] = i;
        ++g_before;
      } else {
        if ((int64_t)e_before < need) out[g_before + e_before] = i;
        ++e_before;
      }
    }
  }
  const int64_t total = (int64_t)tot_s + min((int64_t)tot_e, need);
  for (int64_t j = total + tid; j < p.kmax; j += NT) out[j] = -1;
  if (tid == 0) p.cnt[r] = (int32_t)total;
}

// Rows of 257 .. 2048 candidates (block-sparse rows up to 128K tokens): one
// wave per row and no workgroup barriers.  Lane l keeps candidates 64u + l of
// the row as keys in registers (all loads in flight together); a radix select
// over a per-wave LDS histogram (8-bit digits, lane l owning digits
// 255-4l .. 252-4l) finds the k-th pool key T and the number of keys equal to
// T that are taken; the emission walks the row in chunks of 64 in index order
// and places every kept candidate with two ballots.  Same result as k_select.
constexpr int kSwWaves = 4;
constexpr int kSwPer = 32;  // keys per lane
constexpr int kSwMax = 64 * kSwPer;

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__global__ __launch_bounds__(64 * kSwWaves) __attribute__((amdgpu_waves_per_eu(7))) void k_select_wave(SelectParams p) {
  __shared__ uint32_t hist_s[kSwWaves][256];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t r = (int64_t)blockIdx.x * kSwWaves + wv;
  if (r >= p.rows) return;  // the whole wave leaves; nothing below waits for other waves
  uint32_t* hist = hist_s[wv];
  const float* row = p.scores + r * p.ld;
  const int n = (int)(p.causal ? min(p.ncand, (r % p.period) + p.offset + 1) : p.ncand);
  const int pb = min(p.n_sink, n);
  const int pe = max(pb, n - p.n_local);
  const int npool = pe - pb;
  int64_t kr64 = p.rden > 0 ? ((int64_t)p.rnum * n + p.rden - 1) / p.rden : (int64_t)p.k;
  const int kr = (int)max((int64_t)0, min(kr64, (int64_t)npool));
  const bool take_all = (kr == npool);

  // keys straight from the loads (no float copies kept: fewer registers, more
  // waves per SIMD); a NaN's key lies outside [key(-inf), key(+inf)]
  uint32_t key[kSwPer];
#pragma unroll
  for (int u = 0; u < kSwPer; ++u) {
    const int i = 64 * u + lane;
    key[u] = order_key(i < n ? row[i] : 0.f);
  }
  bool nan_seen = false;
#pragma unroll
  for (int u = 0; u < kSwPer; ++u) nan_seen |= (64 * u + lane < n) && (key[u] > 0xff800000u || key[u] < 0x007fffffu);

  uint32_t T = 0xffffffffu;
  int need = 0;  // keys equal to T that are taken
  if (kr > 0 && !take_all) {
    uint32_t prefix = 0u, pmask = 0u;
    uint32_t remaining = (uint32_t)kr;
#pragma unroll 1
    for (int shift = 24; shift >= 0; shift -= 8) {
      wave_lds_sync();
#pragma unroll
      for (int x = 0; x < 4; ++x) hist[4 * lane + x] = 0u;
      wave_lds_sync();
#pragma unroll
      for (int u = 0; u < kSwPer; ++u) {
        const int i = 64 * u + lane;
        if (i >= pb && i < pe && (key[u] & pmask) == prefix) atomicAdd(&hist[(key[u] >> shift) & 255u], 1u);
      }
      wave_lds_sync();
      uint32_t c[4], loc = 0u;
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        c[x] = hist[255 - 4 * lane - x];
        loc += c[x];
      }
      const uint32_t incl = wave_incl_scan(loc);  // keys with a digit >= 252 - 4*lane
      const uint32_t above = incl - loc;
      const bool mine = above < remaining && remaining <= incl;
      uint32_t dsel = 0u, gt = 0u;
      if (mine) {
        uint32_t acc = above;
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          if (acc + c[x] >= remaining) {
            dsel = (uint32_t)(255 - 4 * lane - x);
            gt = acc;
            break;
          }
          acc += c[x];
        }
      }
      const int src = __ffsll((unsigned long long)__ballot(mine)) - 1;
      dsel = (uint32_t)__shfl((int)dsel, src);
      gt = (uint32_t)__shfl((int)gt, src);
      remaining -= gt;
      prefix |= dsel << shift;
      pmask |= 255u << shift;
    }
    T = prefix;
    need = (int)remaining;
  }

  // ---- emission in index order
  int32_t* out = p.idx + r * p.kmax;
  const uint64_t below = (1ull << lane) - 1ull;
  uint32_t g_run = 0u, e_run = 0u;  // taken-for-sure and tie counts before this chunk
#pragma unroll
  for (int u = 0; u < kSwPer; ++u) {
    const int i = 64 * u + lane;
    bool tk = false, tie = false;
    if (i < n) {
      if (i < pb || i >= pe) tk = true;
      else if (kr > 0) {
        if (take_all) tk = true;
        else {
          tk = key[u] > T;
          tie = key[u] == T;
        }
      }
    }
    const uint64_t bt = __ballot(tk), be = __ballot(tie);
    const uint32_t gb = g_run + (uint32_t)__popcll(bt & below);
    const uint32_t eb = e_run + (uint32_t)__popcll(be & below);
    if (tk) out[gb + min(eb, (uint32_t)need)] = i;
    else if (tie && eb < (uint32_t)need) out[gb + eb] = i;
    g_run += (uint32_t)__popcll(bt);
    e_run += (uint32_t)__popcll(be);
  }
  const int total = (int)g_run + min((int)e_run, need);
  for (int j = total + lane; j < p.kmax; j += 64) out[j] = -1;
  const bool any_nan = __any(nan_seen);
  if (lane == 0) {
    p.cnt[r] = total;
    if (any_nan && p.err != nullptr) atomicOr(reinterpret_cast<unsigned int*>(p.err), 1u);
  }
}

// Rows of at most 256 candidates (cluster selection): one thread per
// candidate computes its rank under the total order (higher score first, lower
// index first on ties) by sweeping the row in LDS; candidates with rank < k are
// kept and written in index order through a wave-ballot prefix count.
__global__ __launch_bounds__(256) void k_select_small(SelectParams p) {
  __shared__ uint32_t keys[256];
  __shared__ uint32_t wave_cnt[4];
  __shared__ uint32_t shnan;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t r = blockIdx.x;
  const float* row = p.scores + r * p.ld;
  const int n = (int)(p.causal ? min(p.ncand, (r % p.period) + p.offset + 1) : p.ncand);
  const int pb = min(p.n_sink, n);
  const int pe = max(pb, n - p.n_local);
  const int npool = pe - pb;
  int64_t kr = p.rden > 0 ? ((int64_t)p.rnum * n + p.rden - 1) / p.rden : (int64_t)p.k;
  kr = max((int64_t)0, min(kr, (int64_t)npool));
  if (tid == 0) shnan = 0u;
  float f = 0.f;
  if (tid < n) {
    f = row[tid];
    keys[tid] = order_key(f);
  }
  __syncthreads();
  if (tid < n && is_nan(f)) atomicOr(&shnan, 1u);
  bool take = false;
  if (tid < n) {
    if (tid < pb || tid >= pe) {
      take = true;
    } else if (kr > 0) {
      const uint32_t mine = keys[tid];
      int rank = 0;
      for (int j = pb; j < pe; ++j) {
        const uint32_t kj = keys[j];
        rank += (kj > mine) | ((kj == mine) & (j < tid));
      }
      take = rank < kr;
    }
  }
  const uint64_t bal = __ballot(take);
  if (lane == 0) wave_cnt[wv] = (uint32_t)__popcll(bal);
  __syncthreads();
  uint32_t base = 0;
  for (int w = 0; w < wv; ++w) base += wave_cnt[w];
  const uint32_t total = wave_cnt[0] + wave_cnt[1] + wave_cnt[2] + wave_cnt[3];
  int32_t* out = p.idx + r * p.kmax;
  if (take) out[base + __popcll(bal & ((1ull << lane) - 1ull))] = tid;
  for (int j = (int)total + tid; j < p.kmax; j += 256) out[j] = -1;
  if (tid == 0) {
    p.cnt[r] = (int32_t)total;
    if (shnan && p.err != nullptr) atomicOr(reinterpret_cast<unsigned int*>(p.err), 1u);
  }
}

// ---------------------------------------------------------------- adaptive budget
// The shortest prefix of the selection order (higher score first, lower index
// on ties) that holds a given share of the row's softmax weight (Squeezed
// Attention page, §技术方案: the number of clusters kept follows the
// distribution of the centroid similarities).  Candidate j weighs
// exp(s_j - m), m the row maximum, and an entry equal to m weighs exactly 1.
// One workgroup per row of at most 4096 candidates: (key, ~index) pairs are
// sorted in LDS by a bitonic network, a block scan sums the weights along that
// order, and a position is kept while the weight ahead of it is below
// mass * total.  The kept indices are marked in an LDS bitmap and written in
// index order.  Weights are fp32 exponentials rounded to multiples of 2^-40
// and summed as 64-bit integers (4096 * 2^40 < 2^53), so every prefix is exact,
// the prefixes never decrease, and the last one is the total whatever the
// thread layout; the comparison with mass * total is made in double.
constexpr int kMassNT = 256;

__global__ __launch_bounds__(kMassNT) void k_select_mass(MassParams p) {
  constexpr int NT = kMassNT;
  __shared__ uint64_t kv[kMassMax];
  __shared__ uint32_t bm[kMassMax / 32];
  __shared__ uint64_t wtmp[NT / 64];
  __shared__ uint32_t utmp[NT / 64];
  __shared__ uint32_t shnan;
  const int tid = threadIdx.x;
  const int64_t r = blockIdx.x;
  const float* row = p.scores + r * p.ld;
  const int n = (int)p.ncand;
  int P = 64;
  while (P < n) P <<= 1;
  bool nan_seen = false;
  for (int i = tid; i < P; i += NT) {
    uint64_t e = 0ull;  // padding sorts last: every real key is above 0
    if (i < n) {
      const float f = row[i];
      nan_seen |= is_nan(f);
      e = ((uint64_t)order_key(f) << 32) | (uint64_t)(~(uint32_t)i);
    }
    kv[i] = e;
  }
  if (tid == 0) shnan = 0u;
  __syncthreads();
  if (nan_seen) atomicOr(&shnan, 1u);
  mass_select_lds<NT>(kv, bm, wtmp, utmp, n, P, p.mass, p.k_min, p.k_max, p.idx + r * p.kmax, p.kmax, p.cnt + r);
  if (tid == 0 && shnan && p.err != nullptr) atomicOr(reinterpret_cast<unsigned int*>(p.err), 1u);
}

// ---------------------------------------------------------------- vertical-slash tables
// One thread per (row, query block).  Offsets arrive ascending, so walking
// them backwards yields tile starts 64i-o in ascending order; overlapping or
// touching tiles merge into one interval.  Columns arrive ascending; those not
// covered by an interval and not beyond the block's last row are kept.
__global__ __launch_bounds__(64) void k_vs_build(VsBuildParams p) {
  const int64_t nqb = p.seq / p.bs;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= p.rows * nqb) return;
  const int64_t r = gid / nqb;
  const int i = (int)(gid % nqb);
  const int32_t* offs = p.slash + r * p.n_slash;
  const int32_t* cols = p.vert + r * p.n_vert;
  // counts beyond the capacities, negative offsets and columns outside
  // [0, seq) are ignored, so every table entry names keys that exist
  const int ns = max(0, min(p.slash_cnt[r], p.n_slash)), nv = max(0, min(p.vert_cnt[r], p.n_vert));
  int32_t* iv = p.iv + gid * p.n_slash * 2;
  int32_t* col = p.col + gid * p.n_vert;
  const int64_t q0 = (int64_t)i * p.bs;
  int niv = 0;
  for (int s = ns - 1; s >= 0; --s) {
    const int64_t o = offs[s];
    const int64_t e = q0 - o + p.bs;
    if (o < 0 || e <= 0) continue;
    const int64_t b = max((int64_t)0, q0 - o);
    if (niv > 0 && b <= iv[2 * niv - 1]) {
      if (e > iv[2 * niv - 1]) iv[2 * niv - 1] = (int32_t)e;
    } else {
      iv[2 * niv] = (int32_t)b;
      iv[2 * niv + 1] = (int32_t)e;
      ++niv;
    }
  }
  const int64_t last = q0 + p.bs - 1;
  int nc = 0, w = 0;
  for (int c = 0; c < nv; ++c) {
    const int64_t x = cols[c];
    if (x > last) break;
    if (x < 0) continue;
    while (w < niv && iv[2 * w + 1] <= x) ++w;
    if (w < niv && iv[2 * w] <= x) continue;
    col[nc++] = (int32_t)x;
  }
  p.iv_cnt[gid] = niv;
  p.col_cnt[gid] = nc;
}

// The same tables with one wave per (row, query block), for n_slash <= 64.
// Lane j takes offset index ns-1-j: tile ends 64i-o+64 then ascend with the
// lane, so a tile starts a new interval exactly when it begins after the
// previous lane's end; a ballot numbers the intervals.  Columns are taken 64
// at a time: each lane finds the interval around its column by binary search
// and a ballot compacts the kept ones in order.
constexpr int kVbWaves = 4;

__global__ __launch_bounds__(64 * kVbWaves) void k_vs_build_wave(VsBuildParams p) {
  __shared__ int32_t sb[kVbWaves][64];
  __shared__ int32_t se[kVbWaves][64];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t nqb = p.seq / p.bs;
  const int64_t gid = (int64_t)blockIdx.x * kVbWaves + wv;
  if (gid >= p.rows * nqb) return;  // whole waves only; no workgroup barrier below
  const int64_t r = gid / nqb;
  const int i = (int)(gid % nqb);
  const int32_t* offs = p.slash + r * p.n_slash;
  const int32_t* cols = p.vert + r * p.n_vert;
  // the same clipping as k_vs_build
  const int ns = max(0, min(p.slash_cnt[r], min(p.n_slash, 64))), nv = max(0, min(p.vert_cnt[r], p.n_vert));
  int32_t* iv = p.iv + gid * p.n_slash * 2;
  int32_t* col = p.col + gid * p.n_vert;
  const int q0 = i * p.bs;
  const uint64_t lt = (1ull << lane) - 1ull;
  // ---- slash tiles -> disjoint intervals
  int b = 0, e = 0;
  bool valid = false;
  if (lane < ns) {
    const int o = offs[ns - 1 - lane];
    e = q0 - o + p.bs;
    valid = o >= 0 && e > 0;
    b = max(0, q0 - o);
  }
  const int prev_e = __shfl_up(e, 1);  // every lane takes part in the exchanges
  const int prev_v = __shfl_up((int)valid, 1);
  const bool prev_valid = lane > 0 && prev_v != 0;
  const bool starts = valid && (!prev_valid || b > prev_e);
  const uint64_t ms = __ballot(starts);
  const int next_s = __shfl_down((int)starts, 1);
  const int next_v = __shfl_down((int)valid, 1);
  const bool next_starts = lane < 63 && next_s != 0;
  const bool next_valid = lane < 63 && lane + 1 < ns && next_v != 0;
  const bool ends = valid && (!next_valid || next_starts);
  const int k_here = (int)__popcll(ms & (lt | (1ull << lane))) - 1;  // interval of this lane
  if (starts) {
    iv[2 * k_here] = b;
    sb[wv][k_here] = b;
  }
  if (ends) {
    iv[2 * k_here + 1] = e;
    se[wv][k_here] = e;
  }
  const int niv = (int)__popcll(ms);
  __builtin_amdgcn_wave_barrier();
  // ---- kept columns: <= the block's last row and outside every interval
  const int last = q0 + p.bs - 1;
  int nc = 0;
  for (int c0 = 0; c0 < nv; c0 += 64) {
    const int x = c0 + lane < nv ? cols[c0 + lane] : INT_MAX;
    const bool in_range = x <= last;
    int lo = 0, hi = niv;  // intervals with start <= x: [0, lo)
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (sb[wv][mid] <= x) lo = mid + 1;
      else hi = mid;
    }
    const bool inside = lo > 0 && x < se[wv][lo - 1];
    const bool keep = x >= 0 && in_range && !inside;
    const uint64_t mk = __ballot(keep);
    if (keep) col[nc + (int)__popcll(mk & lt)] = x;
    nc += (int)__popcll(mk);
    if (__any(!in_range)) break;  // columns ascend: nothing later is kept
  }
  if (lane == 0) {
    p.iv_cnt[gid] = niv;
    p.col_cnt[gid] = nc;
  }
}

}  // namespace

hipError_t launch_select(const SelectParams& p, hipStream_t stream) {
  if (p.rows == 0) return hipSuccess;
  const dim3 grid((unsigned)p.rows);
  if (p.ncand <= 256)
    hipLaunchKernelGGL(k_select_small, grid, dim3(256), 0, stream, p);
  else if (p.ncand <= kSwMax)
    hipLaunchKernelGGL(k_select_wave, dim3((unsigned)((p.rows + kSwWaves - 1) / kSwWaves)), dim3(64 * kSwWaves), 0,
                       stream, p);
  else if (p.ncand <= 4096)
    hipLaunchKernelGGL((k_select<256, true>), grid, dim3(256), 0, stream, p);
  else if (p.ncand <= kBmMax)
    hipLaunchKernelGGL((k_select_long<1024>), grid, dim3(1024), 0, stream, p);
  else
    hipLaunchKernelGGL((k_select<1024, false>), grid, dim3(1024), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_select_mass(const MassParams& p, hipStream_t stream) {
  if (p.rows == 0) return hipSuccess;
  hipLaunchKernelGGL(k_select_mass, dim3((unsigned)p.rows), dim3(kMassNT), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_vs_build(const VsBuildParams& p, hipStream_t stream) {
  const int64_t n = p.rows * (p.seq / p.bs);
  if (n == 0) return hipSuccess;
  if (p.n_slash <= 64)
    hipLaunchKernelGGL(k_vs_build_wave, dim3((unsigned)((n + kVbWaves - 1) / kVbWaves)), dim3(64 * kVbWaves), 0,
                       stream, p);
  else
    hipLaunchKernelGGL(k_vs_build, dim3((unsigned)((n + 63) / 64)), dim3(64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace sa
