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
// Rows of up to 4096 candidates are staged in LDS once; longer rows are read
// twice (bracketing pass + emission) when the sampled bracket holds.
#include "common.h"
#include "launch.h"

namespace sa {
namespace {

template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* tmp, uint32_t& total) {
  const int tid = threadIdx.x;
  tmp[tid] = v;
  __syncthreads();
  for (int off = 1; off < NT; off <<= 1) {
    const uint32_t a = tid >= off ? tmp[tid - off] : 0u;
    __syncthreads();
    tmp[tid] += a;
    __syncthreads();
  }
  const uint32_t incl = tmp[tid];
  total = tmp[NT - 1];
  __syncthreads();
  return incl - v;
}

// k-th largest key (1 <= k <= e-b) of key_at(b..e-1): MSB-first radix select
// with 8-bit digits and LDS histograms.  Returns T and how many keys equal to
// T belong to the top k.  Called by every thread of the workgroup.
template <int NT, class KeyAt>
__device__ void radix_kth(KeyAt key_at, int64_t b, int64_t e, int64_t k, uint32_t* hist, uint32_t* tmp,
                          uint32_t* shv, uint32_t& T, int64_t& need) {
  const int tid = threadIdx.x;
  uint32_t prefix = 0u, pmask = 0u;
  int64_t remaining = k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int d = tid; d < 256; d += NT) hist[d] = 0u;
    __syncthreads();
    for (int64_t i = b + tid; i < e; i += NT) {
      const uint32_t kk = key_at(i);
      if ((kk & pmask) == prefix) atomicAdd(&hist[(kk >> shift) & 255u], 1u);
    }
    __syncthreads();
    // suffix sums over the 256 digits: tmp[t] = keys with digit >= 255-t
    if (tid < 256) tmp[tid] = hist[255 - tid];
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
      uint32_t a = 0u;
      if (tid < 256 && tid >= off) a = tmp[tid - off];
      __syncthreads();
      if (tid < 256) tmp[tid] += a;
      __syncthreads();
    }
    if (tid < 256) {
      const uint32_t ge = tmp[tid];
      const uint32_t gt = tid > 0 ? tmp[tid - 1] : 0u;
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
  const int ns = p.slash_cnt[r], nv = p.vert_cnt[r];
  int32_t* iv = p.iv + gid * p.n_slash * 2;
  int32_t* col = p.col + gid * p.n_vert;
  const int64_t q0 = (int64_t)i * p.bs;
  int niv = 0;
  for (int s = ns - 1; s >= 0; --s) {
    const int64_t o = offs[s];
    const int64_t e = q0 - o + p.bs;
    if (e <= 0) continue;
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
    while (w < niv && iv[2 * w + 1] <= x) ++w;
    if (w < niv && iv[2 * w] <= x) continue;
    col[nc++] = (int32_t)x;
  }
  p.iv_cnt[gid] = niv;
  p.col_cnt[gid] = nc;
}

}  // namespace

hipError_t launch_select(const SelectParams& p, hipStream_t stream) {
  if (p.rows == 0) return hipSuccess;
  const dim3 grid((unsigned)p.rows);
  if (p.ncand <= 256)
    hipLaunchKernelGGL(k_select_small, grid, dim3(256), 0, stream, p);
  else if (p.ncand <= 4096)
    hipLaunchKernelGGL((k_select<256, true>), grid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((k_select<1024, false>), grid, dim3(1024), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_vs_build(const VsBuildParams& p, hipStream_t stream) {
  const int64_t n = p.rows * (p.seq / p.bs);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_vs_build, dim3((unsigned)((n + 63) / 64)), dim3(64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace sa
