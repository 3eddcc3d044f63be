// Exact per-row top-k with forced members, and the vertical-slash table build.
//
// Selection keeps the best-scoring subset ("MInference 1.0" article,
// §方法介紹; Squeezed Attention page, §技术方案; IndexCache article,
// §长文本的算力困境); the leading (sink) and trailing (local) candidates are
// always kept ("稀疏注意力机制解析" explainer, §1.2).  Because the forced
// members are a prefix and a suffix of the causal range, the ranked pool is one
// contiguous range [pb, pe).
//
// Method: scores become order-preserving 32-bit keys; an MSB-first radix
// select (4 passes of 8 bits, LDS histograms) finds the k-th largest key T and
// how many keys equal to T must be taken; one more pass emits, in index order,
// the forced members, every pool key > T and the lowest-index keys == T.  The
// emission order makes the output ascending and breaks ties toward the lower
// index, which is the required total order.  Rows of up to 4096 candidates are
// staged in LDS once; longer rows are re-read from memory on every pass.
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

template <int NT, bool IN_LDS>
__global__ __launch_bounds__(NT) void k_select(SelectParams p) {
  constexpr int kLdsMax = 4096;
  __shared__ uint32_t keys[IN_LDS ? kLdsMax : 1];
  __shared__ uint32_t hist[256];
  __shared__ uint32_t tmp[NT];
  __shared__ uint32_t sh_digit, sh_above, sh_nan;

  const int tid = threadIdx.x;
  const int64_t r = blockIdx.x;
  const float* row = p.scores + r * p.ld;
  const int64_t n = p.causal ? min(p.ncand, (r % p.period) + p.offset + 1) : p.ncand;
  const int64_t pb = min((int64_t)p.n_sink, n);
  const int64_t pe = max(pb, n - (int64_t)p.n_local);
  const int64_t npool = pe - pb;
  int64_t kr = p.rden > 0 ? ((int64_t)p.rnum * n + p.rden - 1) / p.rden : (int64_t)p.k;
  kr = max((int64_t)0, min(kr, npool));

  if (tid == 0) sh_nan = 0u;
  __syncthreads();
  bool nan_seen = false;
  if (IN_LDS) {
    for (int64_t i = tid; i < n; i += NT) {
      const float f = row[i];
      nan_seen |= is_nan(f);
      keys[i] = order_key(f);
    }
  } else {
    for (int64_t i = tid; i < n; i += NT) nan_seen |= is_nan(row[i]);
  }
  if (nan_seen) atomicOr(&sh_nan, 1u);
  __syncthreads();
  if (sh_nan && tid == 0 && p.err != nullptr) atomicOr(reinterpret_cast<unsigned int*>(p.err), 1u);

  auto key_at = [&](int64_t i) -> uint32_t { return IN_LDS ? keys[i] : order_key(row[i]); };

  // ---- threshold: the kr-th largest key of the pool
  uint32_t T = 0xffffffffu;
  int64_t need = 0;  // keys equal to T that are taken
  bool take_all = (kr == npool);
  if (kr > 0 && !take_all) {
    uint32_t prefix = 0u, pmask = 0u;
    int64_t remaining = kr;
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int d = tid; d < 256; d += NT) hist[d] = 0u;
      __syncthreads();
      for (int64_t i = pb + tid; i < pe; i += NT) {
        const uint32_t kk = key_at(i);
        if ((kk & pmask) == prefix) atomicAdd(&hist[(kk >> shift) & 255u], 1u);
      }
      __syncthreads();
      // suffix sums over the 256 digits (counts of keys with digit >= d)
      if (tid < 256) tmp[tid] = hist[255 - tid];
      __syncthreads();
      for (int off = 1; off < 256; off <<= 1) {
        uint32_t a = 0u;
        if (tid < 256 && tid >= off) a = tmp[tid - off];
        __syncthreads();
        if (tid < 256) tmp[tid] += a;
        __syncthreads();
      }
      // tmp[t] = number of keys with digit >= 255-t
      if (tid < 256) {
        const uint32_t ge = tmp[tid];
        const uint32_t gt = tid > 0 ? tmp[tid - 1] : 0u;
        if (gt < (uint32_t)remaining && (uint32_t)remaining <= ge) {
          sh_digit = 255u - tid;
          sh_above = gt;
        }
      }
      __syncthreads();
      remaining -= sh_above;
      prefix |= sh_digit << shift;
      pmask |= 255u << shift;
      __syncthreads();
    }
    T = prefix;
    need = remaining;
  }

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
  if (p.ncand <= 4096)
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
