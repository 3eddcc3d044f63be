// Gathered attention: clustered-context decode and token-gathered prefill,
// plus the offline cluster-major packing of a fixed context.
//
// Squeezed Attention page, §技术方案: offline, keys are clustered and each
// key is mapped to its cluster; online, a query attends only the key/value
// pairs of its top-K clusters.  IndexCache article, §长文本的算力困境 and
// §"偷懒"的艺术: every query token attends its indexer-selected token subset,
// and shared layers reuse a full layer's subset.
//
// Cluster decode is bound by HBM bandwidth.  The context is stored cluster by
// cluster, so the union of all selected clusters can be streamed once: each
// workgroup sweeps a contiguous range of packed rows, skips 64-row tiles that
// no query of the KV head selected, and runs all of the head's queries
// (<= 64, here 8 tokens x 4 grouped heads) against each tile with a
// per-(query, row) selection mask.  Partial (max, sum, output) per range are
// merged by a second, fixed-order kernel.
//
// Matrix-core layout (v_mfma_f32_32x32x16_bf16, queries as the N dimension):
//   S^T[key][query] = K . Q^T  — K rows go straight from memory into the A
//   operand (each lane reads 128 contiguous bytes of one key row; Q^T uses
//   the same dimension order), V is transposed through LDS for O^T = V^T P^T.
// The token gather uses v_mfma_f32_16x16x32_bf16 with the 16 query heads of
// one token as the N dimension.
#include <algorithm>
#include <climits>

#include "common.h"
#include "launch.h"

namespace sa {
namespace {

// a + b and max(a, b) with lane l ^ 16 (v_permlane16_swap: rows of 16 lanes trade
// places inside each half of the wave).
__device__ __forceinline__ float xor16_add(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor16_max(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}


constexpr int kBlk = 64;
constexpr int kD = 128;
constexpr int kVS = kBlk + 8;  // V^T row stride (elements)

// ================================================================ cluster pack
constexpr int kSeg = 512;  // tokens per pack segment

__global__ __launch_bounds__(256) void k_pack_count(const int32_t* __restrict__ labels, int64_t n, int C, int nseg,
                                                    int32_t* __restrict__ segcnt, int32_t* err) {
  extern __shared__ int32_t hist[];
  const int g = blockIdx.x / nseg, s = blockIdx.x % nseg;
  for (int c = threadIdx.x; c < C; c += blockDim.x) hist[c] = 0;
  __syncthreads();
  const int64_t t0 = (int64_t)s * kSeg, t1 = min(n, t0 + kSeg);
  bool bad = false;
  for (int64_t t = t0 + threadIdx.x; t < t1; t += blockDim.x) {
    const int c = labels[(int64_t)g * n + t];
    if (c < 0 || c >= C) bad = true;
    else atomicAdd(&hist[c], 1);
  }
  if (bad && err != nullptr) atomicOr(reinterpret_cast<unsigned int*>(err), 1u);
  __syncthreads();
  for (int c = threadIdx.x; c < C; c += blockDim.x) segcnt[((int64_t)g * nseg + s) * C + c] = hist[c];
}

// Exclusive scan in (cluster, segment) order -> per-segment bases and cluster_ptr.
// One workgroup per KV head: thread t owns a run of consecutive (cluster,
// segment) entries, sums it, takes its base from a workgroup scan, then writes
// the running bases; the first entry of every cluster gives cluster_ptr.
constexpr int kScanThreads = 1024;

__global__ __launch_bounds__(kScanThreads) void k_pack_scan(int C, int nseg, int32_t* __restrict__ seg,
                                                            int32_t* __restrict__ ptr) {
  __shared__ int32_t wsum[kScanThreads / 64];
  const int g = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t total = (int64_t)C * nseg;
  const int64_t per = (total + kScanThreads - 1) / kScanThreads;
  const int64_t e0 = min(total, (int64_t)tid * per), e1 = min(total, e0 + per);
  int32_t* sg = seg + (int64_t)g * nseg * C;
  auto at = [&](int64_t e) -> int32_t& {  // entry e = cluster e / nseg, segment e % nseg
    return sg[(e % nseg) * C + e / nseg];
  };
  int32_t run = 0;
  for (int64_t e = e0; e < e1; ++e) run += at(e);
  // workgroup exclusive scan of the per-thread sums
  int32_t incl = run;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int32_t o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  if (lane == 63) wsum[wv] = incl;
  __syncthreads();
  int32_t base = incl - run, all = 0;
#pragma unroll
  for (int x = 0; x < kScanThreads / 64; ++x) {
    const int32_t v = wsum[x];
    base += x < wv ? v : 0;
    all += v;
  }
  for (int64_t e = e0; e < e1; ++e) {
    int32_t& cell = at(e);
    const int32_t x = cell;
    if (e % nseg == 0) ptr[(int64_t)g * (C + 1) + e / nseg] = base;
    cell = base;
    base += x;
  }
  if (tid == 0) ptr[(int64_t)g * (C + 1) + C] = all;
}

// With C <= kScanThreads clusters: thread t takes cluster t % C and the t / C-th
// of Q = kScanThreads / C consecutive ranges of its segments, so for each
// segment the wave reads consecutive clusters (coalesced); the runs are then
// scanned in (cluster, range) order through LDS.
__global__ __launch_bounds__(kScanThreads) void k_pack_scan_cm(int C, int nseg, int32_t* __restrict__ seg,
                                                               int32_t* __restrict__ ptr) {
  __shared__ int32_t buf[kScanThreads];
  __shared__ int32_t wsum[kScanThreads / 64];
  const int g = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int Q = kScanThreads / C;
  const int c = tid % C, q = tid / C;
  const bool act = q < Q;
  const int per = (nseg + Q - 1) / Q;
  const int s0 = act ? min(nseg, q * per) : 0, s1 = act ? min(nseg, s0 + per) : 0;
  int32_t* sg = seg + (int64_t)g * nseg * C;
  int32_t run = 0;
  for (int s = s0; s < s1; ++s) run += sg[(int64_t)s * C + c];
  const int o = act ? c * Q + q : tid;  // position in (cluster, range) order
  buf[o] = run;
  __syncthreads();
  const int32_t v = buf[tid];
  int32_t incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int32_t u = __shfl_up(incl, off);
    if (lane >= off) incl += u;
  }
  if (lane == 63) wsum[wv] = incl;
  __syncthreads();
  int32_t ex = incl - v, all = 0;
#pragma unroll
  for (int x = 0; x < kScanThreads / 64; ++x) {
    const int32_t w = wsum[x];
    ex += x < wv ? w : 0;
    all += w;
  }
  buf[tid] = ex;
  __syncthreads();
  if (act) {
    int32_t base = buf[o];
    if (q == 0) ptr[(int64_t)g * (C + 1) + c] = base;
    for (int s = s0; s < s1; ++s) {
      int32_t& cell = sg[(int64_t)s * C + c];
      const int32_t x = cell;
      cell = base;
      base += x;
    }
  }
  if (tid == 0) ptr[(int64_t)g * (C + 1) + C] = all;
}

// Each thread owns clusters; walking the segment in token order keeps the sort stable.
__global__ __launch_bounds__(256) void k_pack_scatter(const int32_t* __restrict__ labels, int64_t n, int C, int nseg,
                                                      const int32_t* __restrict__ seg, int32_t* __restrict__ perm) {
  __shared__ __attribute__((aligned(16))) int32_t lab[kSeg];
  const int g = blockIdx.x / nseg, s = blockIdx.x % nseg;
  const int64_t t0 = (int64_t)s * kSeg, t1 = min(n, t0 + kSeg);
  const int len = (int)(t1 - t0);
  for (int t = threadIdx.x; t < len; t += blockDim.x) lab[t] = labels[(int64_t)g * n + t0 + t];
  __syncthreads();
  for (int c = threadIdx.x; c < C; c += blockDim.x) {
    int32_t pos = seg[((int64_t)g * nseg + s) * C + c];
    int32_t* pg = perm + (int64_t)g * n;
    int t = 0;
    for (; t + 4 <= len; t += 4) {  // four labels per LDS read
      const int4 l4 = *reinterpret_cast<const int4*>(&lab[t]);
      if (l4.x == c) pg[pos++] = (int32_t)(t0 + t);
      if (l4.y == c) pg[pos++] = (int32_t)(t0 + t + 1);
      if (l4.z == c) pg[pos++] = (int32_t)(t0 + t + 2);
      if (l4.w == c) pg[pos++] = (int32_t)(t0 + t + 3);
    }
    for (; t < len; ++t)
      if (lab[t] == c) pg[pos++] = (int32_t)(t0 + t);
  }
}

__global__ __launch_bounds__(256) void k_pack_copy(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                                   const int32_t* __restrict__ perm, const int32_t* __restrict__ ptr,
                                                   int64_t n, int C, int row_bytes, int64_t total_chunks) {
  const int cpr = row_bytes / 16;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total_chunks;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = e / cpr;  // packed row over all heads
    const int ch = (int)(e % cpr);
    const int64_t g = row / n, p = row % n;
    if (p >= ptr[g * (C + 1) + C]) continue;  // rows dropped for invalid labels
    const int64_t srow = g * n + perm[row];
    stg16(dst + row * row_bytes + ch * 16, ldg16(src + srow * row_bytes + ch * 16));
  }
}

// ================================================================ shared tile helpers
// V tile of 64 rows -> registers (each lane: 4 groups of 4 rows x 16 bytes).
struct VRegs {
  u32x4 v[4][4];
};

__device__ __forceinline__ void v_fetch(VRegs& R, const uint16_t* vb, const int* rows, int lane) {
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int gidx = lane + 64 * n;
    const int kg = gidx % 16, dc = gidx / 16;
#pragma unroll
    for (int e = 0; e < 4; ++e) R.v[n][e] = ldg16(vb + (int64_t)rows[4 * n + e] * kD + 8 * dc);
  }
}

// rows[] for v_fetch: the 16 rows this lane loads (4 groups of 4 consecutive slots)
__device__ __forceinline__ int v_slot(int lane, int n, int e) { return 4 * ((lane + 64 * n) % 16) + e; }

// Store V^T: POS maps a 4-key group index to its LDS position.
template <int LAYOUT>
__device__ __forceinline__ int vt_pos(int kg) {
  if (LAYOUT == 32) {  // 32x32x16 consumers: groups swap 1 <-> 2 inside each 16-key block
    const int q4 = kg & 3;
    return 16 * (kg >> 2) + 4 * ((q4 == 1) ? 2 : (q4 == 2) ? 1 : q4);
  }
  // 16x16x32 consumers: key 32ks + 16a + 4b + c sits at 32ks + 8b + 4a + c
  return 32 * (kg >> 3) + 8 * (kg & 3) + 4 * ((kg & 7) >> 2);
}

template <int LAYOUT>
__device__ __forceinline__ void v_store(uint16_t* vt, const VRegs& R, int lane) {
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int gidx = lane + 64 * n;
    const int kg = gidx % 16, dc = gidx / 16;
    const int pos = vt_pos<LAYOUT>(kg);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int w = e >> 1, sh = (e & 1) * 16;
      u32x2 pk;
      pk[0] = ((R.v[n][0][w] >> sh) & 0xffffu) | (((R.v[n][1][w] >> sh) & 0xffffu) << 16);
      pk[1] = ((R.v[n][2][w] >> sh) & 0xffffu) | (((R.v[n][3][w] >> sh) & 0xffffu) << 16);
      *reinterpret_cast<u32x2*>(&vt[(8 * dc + e) * kVS + pos]) = pk;
    }
  }
}

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ================================================================ cluster decode
constexpr int kDecWaves = 4;
constexpr int kRowsPerSplit = 2048;

int decode_splits(int64_t n_ctx) { return (int)((n_ctx + kRowsPerSplit - 1) / kRowsPerSplit); }

constexpr int kDecRows = 32;      // rows per tile
constexpr int kDecMaxC = 1024;    // clusters whose tables are staged in LDS

struct DecWaveLds {
  uint16_t v[2][kDecRows * kD];   // double-buffered V tiles, row-major, chunk-swizzled
  uint64_t rmask[2][kDecRows];    // per row: which queries selected its cluster
};

// V rows -> LDS: 32 rows x 256 B, chunk c of row r at position c ^ key(r);
// 8 copies of 1 KB.
__device__ __forceinline__ void dec_dma_v(uint16_t* vl, const uint16_t* vb, int64_t base, int len, int lane) {
  const uint32_t vbase = __builtin_amdgcn_readfirstlane(lds_addr(vl));
#pragma unroll
  for (int n = 0; n < 8; ++n) {
    const int r = 4 * n + lane / 16;
    const int c = (lane % 16) ^ swz_key128(r);
    const int64_t row = base + min(r, len - 1);
    dma16(vbase + n * 1024u, vb + row * kD + 8 * c);
  }
}

// One workgroup per (KV head, packed-row range).  Its waves stream disjoint
// 32-row tiles independently.  K rows go straight from memory into the A
// operand registers of the score product; V tiles go through a per-wave,
// double-buffered LDS region by direct copies (the transposing LDS reads need
// them there).  The next tile's K and V are requested right after the current
// tile's scores, so they are in flight during its softmax and P.V; LDS per
// wave is 16.5 KB, so two workgroups of four waves share a CU.
// NQT = query tiles of 32.  CAUSAL: query t only sees packed rows whose
// context position (perm) is at most q_pos[t].
template <int NQT, bool CAUSAL>
__global__ __launch_bounds__(64 * kDecWaves, NQT == 1 ? 2 : 1) void k_decode_split(GatherParams p, float* __restrict__ part, int nsplit) {
  __shared__ __attribute__((aligned(1024))) DecWaveLds L[kDecWaves];
  __shared__ int32_t ptr_s[kDecMaxC + 1];
  __shared__ uint64_t mask_s[kDecMaxC];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, hf = lane >> 5, l32 = lane & 31;
  const int g = blockIdx.x / nsplit, split = blockIdx.x % nsplit;
  const int grp = p.hq / p.hkv;
  const int nq = p.T * grp;
  const int64_t N = p.n_ctx;
  const int C = p.C;
  const uint16_t* kb = p.k + (int64_t)g * N * kD;
  const uint16_t* vb = p.v + (int64_t)g * N * kD;
  const int64_t p0 = (int64_t)split * kRowsPerSplit;
  const int64_t p1 = min(N, p0 + kRowsPerSplit);
  const int ntile = (int)((p1 - p0 + kDecRows - 1) / kDecRows);
  DecWaveLds& W = L[w];
  // K operand of tile t: lane row l32, dims 16s + 8hf .. +7 of step s (ordinary
  // loads: the compiler's wait for them also covers the older V copies)
  bf16x8 kr[8];
  int prow = 0;  // CAUSAL: context position of this lane's row of the fetched tile
  auto fetch = [&](int t, int buf) {
    const int64_t base = p0 + (int64_t)t * kDecRows;
    const int len = (int)min((int64_t)kDecRows, p1 - base);
    dec_dma_v(W.v[buf], vb, base, len, lane);
    const uint16_t* krow = kb + (base + min(l32, len - 1)) * kD + 8 * hf;
#pragma unroll
    for (int s = 0; s < 8; ++s) kr[s] = as_bf16x8(ldg16(krow + 16 * s));
    if (CAUSAL) prow = p.perm[(int64_t)g * N + base + min(l32, len - 1)];
  };
  // This wave's first tile is fetched before the set-up below: at decode sizes
  // nearly every tile is selected, so its copy travels with the set-up loads.
  // If the wave's first selected tile is another one, that fetch refills the
  // same buffer and registers (a wave's loads complete in order, so the later
  // copy lands last).
  const bool spec = w < ntile;
  if (spec) fetch(w, 0);
  // Set-up: the cluster pointers, the selected cluster ids and Q are all
  // requested before the first of them is used, so the workgroup waits for one
  // memory latency instead of one per loop trip.
  constexpr int kNT = 64 * kDecWaves;
  constexpr int kPtrPer = (kDecMaxC + kNT) / kNT;  // covers C + 1 <= kDecMaxC + 1 pointers
  constexpr int kSelPer = 8;
  for (int c = threadIdx.x; c < C; c += kNT) mask_s[c] = 0ull;
  int32_t pv_[kPtrPer];
#pragma unroll
  for (int u = 0; u < kPtrPer; ++u) {
    const int c = threadIdx.x + u * kNT;
    pv_[u] = c <= C ? p.cluster_ptr[(int64_t)g * (C + 1) + c] : 0;
  }
  // mask_s[c] bit j <=> query j of this KV head (token t, head-in-group hh: j = t*grp + hh)
  // selected cluster c; duplicate and out-of-range ids fall out naturally
  const int nsel_all = nq * p.n_sel;
  auto sel_load = [&](int e0, int32_t* cv) {
#pragma unroll
    for (int u = 0; u < kSelPer; ++u) {
      const int e = e0 + u * kNT;
      cv[u] = -1;
      if (e < nsel_all) {
        const int qi = e / p.n_sel, sidx = e % p.n_sel;
        const int t = qi / grp, hh = qi % grp;
        cv[u] = p.sel[((int64_t)t * p.hq + g * grp + hh) * p.n_sel + sidx];
      }
    }
  };
  auto sel_mark = [&](int e0, const int32_t* cv) {
#pragma unroll
    for (int u = 0; u < kSelPer; ++u) {
      const int e = e0 + u * kNT;
      const int c = cv[u];
      if (e < nsel_all && c >= 0 && c < C)
        atomicOr(reinterpret_cast<unsigned long long*>(&mask_s[c]), 1ull << (e / p.n_sel));
    }
  };
  int32_t cv0[kSelPer];
  sel_load(threadIdx.x, cv0);

  // Q^T: lane holds query 32nt+l32, dims 16s + 8hf .. +7 at step s
  bf16x8 qv[NQT][8];
#pragma unroll
  for (int nt = 0; nt < NQT; ++nt) {
    const int qi = min(32 * nt + l32, nq - 1);
    const int t = qi / grp, h = g * grp + qi % grp;
    const uint16_t* qr = p.q + ((int64_t)t * p.hq + h) * kD + 8 * hf;
#pragma unroll
    for (int s = 0; s < 8; ++s) qv[nt][s] = as_bf16x8(ldg16(qr + 16 * s));
  }
  int qlim[NQT];  // causal bound of this lane's query in each query tile
#pragma unroll
  for (int nt = 0; nt < NQT; ++nt) {
    const int qi = 32 * nt + l32;
    qlim[nt] = (CAUSAL && qi < nq) ? p.q_pos[qi / grp] : INT_MAX;
  }
#pragma unroll
  for (int u = 0; u < kPtrPer; ++u) {
    const int c = threadIdx.x + u * kNT;
    if (c <= C) ptr_s[c] = pv_[u];
  }
  __syncthreads();  // mask_s cleared, ptr_s complete
  sel_mark(threadIdx.x, cv0);
  for (int e0 = threadIdx.x + kSelPer * kNT; e0 < nsel_all; e0 += kSelPer * kNT) {
    int32_t cv[kSelPer];
    sel_load(e0, cv);
    sel_mark(e0, cv);
  }
  const float sl2 = p.scale * kLog2e;
  __syncthreads();

  f32x16 o[NQT][4];
  float m[NQT], l[NQT];
#pragma unroll
  for (int nt = 0; nt < NQT; ++nt) {
    m[nt] = -INFINITY;
    l[nt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[nt][dt][r] = 0.f;
  }

  // cluster of this lane's row: last c with ptr[c] <= row.  Rows only grow
  // along a wave's tiles, so after one binary search the cluster index
  // advances incrementally.
  int cl = 0;
  {
    const int64_t row0 = p0 + (int64_t)w * kDecRows + l32;
    int lo = 0, hi = C - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (ptr_s[mid] <= row0) lo = mid;
      else hi = mid - 1;
    }
    cl = lo;
  }
  // next selected tile at or after index t (stride kDecWaves); writes its row masks
  auto find = [&](int t, int buf) -> int {
    for (; t < ntile; t += kDecWaves) {
      const int64_t base = p0 + (int64_t)t * kDecRows;
      const int len = (int)min((int64_t)kDecRows, p1 - base);
      const int64_t row = base + min(l32, len - 1);
      while (cl + 1 < C && ptr_s[cl + 1] <= row) ++cl;
      const uint64_t rm = l32 < len ? mask_s[cl] : 0ull;
      if (__any(rm != 0ull)) {
        if (hf == 0) W.rmask[buf][l32] = rm;
        return t;
      }
    }
    return ntile;
  };
  int cur = find(w, 0), buf = 0;
  if (cur < ntile && !(spec && cur == w)) fetch(cur, 0);
  while (cur < ntile) {
    const int pos_cur = prow;
    f32x16 sc[NQT];
#pragma unroll
    for (int nt = 0; nt < NQT; ++nt) {
      sc[nt] = mfma32x32x16(kr[0], qv[nt][0], f32x16{});
#pragma unroll
      for (int st = 1; st < 8; ++st) sc[nt] = mfma32x32x16(kr[st], qv[nt][st], sc[nt]);
    }
    // next tile: K into the (now free) registers, V into the other buffer
    const int nxt = find(cur + kDecWaves, buf ^ 1);
    if (nxt < ntile) fetch(nxt, buf ^ 1);
    const uint16_t* vl = W.v[buf];
    // row masks of the 16 rows this lane's accumulators cover: rows 8j + 4hf + i
    uint64_t rmv[16];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) rmv[4 * j + i] = W.rmask[buf][8 * j + 4 * hf + i];

#pragma unroll
    for (int nt = 0; nt < NQT; ++nt) {
      const int qi = 32 * nt + l32;
      float x[16];
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        bool keep = qi < nq && ((rmv[r] >> qi) & 1ull);
        if (CAUSAL) {
          // every lane takes part in the exchange (lane R holds row R's position)
          const int rp = __shfl(pos_cur, 8 * (r / 4) + 4 * hf + (r % 4));
          keep = keep && rp <= qlim[nt];
        }
        x[r] = keep ? sc[nt][r] : -INFINITY;
        mx = fmaxf(mx, x[r]);
      }
      mx = xor32_max(mx) * sl2;
      const float mnew = fmaxf(m[nt], mx);
      const float muse = (mnew == -INFINITY) ? 0.f : mnew;
      float ps = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        x[r] = fast_exp2(fmaf(x[r], sl2, -muse));
        ps += x[r];
      }
      ps = xor32_add(ps);
      const float alpha = fast_exp2(m[nt] - muse);
      l[nt] = l[nt] * alpha + ps;
      m[nt] = mnew;
      bf16x8 pv[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) pv[ks][e] = (__bf16)x[8 * ks + e];
      const int gl = lane & 15, gsub = (lane >> 4) & 1;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) o[nt][dt][r] *= alpha;
        const int dim = 32 * dt + 16 * gsub + 4 * (gl & 3);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const int k0 = 16 * ks + 4 * hf + (gl >> 2), k1 = k0 + 8;
          const v4i16 lo = lds_read_tr16(vl + k0 * kD + 8 * ((dim >> 3) ^ swz_key128(k0)) + (dim & 7));
          const v4i16 hi = lds_read_tr16(vl + k1 * kD + 8 * ((dim >> 3) ^ swz_key128(k1)) + (dim & 7));
          const short __attribute__((ext_vector_type(8))) ab = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          o[nt][dt] = mfma32x32x16(__builtin_bit_cast(bf16x8, ab), pv[ks], o[nt][dt]);
        }
      }
    }
    wait_lgkm0();  // done reading this buffer before it is refilled
    cur = nxt;
    buf ^= 1;
  }
  wait_vmcnt<0>();  // every copy this wave issued was consumed; make it explicit before LDS reuse

  // ---- merge the waves of this workgroup through LDS (tile buffers are free now),
  //      one query tile at a time, then write the range's partial
  //      (max, sum, unnormalised output)
  float* red_o = reinterpret_cast<float*>(&L[0]);       // [wave][query 32][kD]
  float* red_ml = reinterpret_cast<float*>(&mask_s[0]);  // [wave][query 32][2]
  static_assert(sizeof(L) >= kDecWaves * 32 * kD * sizeof(float), "LDS reuse");
  static_assert(sizeof(mask_s) >= kDecWaves * 32 * 2 * sizeof(float), "LDS reuse");
#pragma unroll
  for (int nt = 0; nt < NQT; ++nt) {
    __syncthreads();
    const int qi = 32 * nt + l32;
    if (qi < nq) {
      if (hf == 0) {
        red_ml[(w * 32 + l32) * 2] = m[nt];
        red_ml[(w * 32 + l32) * 2 + 1] = l[nt];
      }
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) red_o[(w * 32 + l32) * kD + 32 * dt + 8 * (r / 4) + 4 * hf + (r % 4)] = o[nt][dt][r];
    }
    __syncthreads();
    const int nq_t = min(32, nq - 32 * nt);
    for (int e = threadIdx.x; e < nq_t * kD; e += blockDim.x) {
      const int q = e / kD, d = e % kD;
      float M = -INFINITY;
#pragma unroll
      for (int ww = 0; ww < kDecWaves; ++ww) M = fmaxf(M, red_ml[(ww * 32 + q) * 2]);
      const float Mu = M == -INFINITY ? 0.f : M;
      float Ls = 0.f, Os = 0.f;
#pragma unroll
      for (int ww = 0; ww < kDecWaves; ++ww) {
        const float f = fast_exp2(red_ml[(ww * 32 + q) * 2] - Mu);
        Ls += red_ml[(ww * 32 + q) * 2 + 1] * f;
        Os += red_o[(ww * 32 + q) * kD + d] * f;
      }
      float* pp = part + (((int64_t)g * nsplit + split) * 64 + 32 * nt + q) * (kD + 2);
      pp[2 + d] = Os;
      if (d == 0) {
        pp[0] = M;
        pp[1] = Ls;
      }
    }
  }
}

// Fixed-order merge of the partials of every packed-row range.
__global__ __launch_bounds__(128) void k_decode_combine(GatherParams p, const float* __restrict__ part, int nslot) {
  const int grp = p.hq / p.hkv;
  const int th = blockIdx.x;  // (t, h)
  const int t = th / p.hq, h = th % p.hq;
  const int g = h / grp;
  const int qi = t * grp + (h - g * grp);
  const int d = threadIdx.x;
  float M = -INFINITY;
#pragma unroll 8
  for (int s = 0; s < nslot; ++s) M = fmaxf(M, part[(((int64_t)g * nslot + s) * 64 + qi) * (kD + 2)]);
  const float Mu = M == -INFINITY ? 0.f : M;
  float Ls = 0.f, Os = 0.f;
#pragma unroll 8
  for (int s = 0; s < nslot; ++s) {
    const float* pp = part + (((int64_t)g * nslot + s) * 64 + qi) * (kD + 2);
    const float f = fast_exp2(pp[0] - Mu);
    Ls += pp[1] * f;
    Os += pp[2 + d] * f;
  }
  const float val = Ls > 0.f ? Os / Ls : 0.f;
  const int64_t o = (int64_t)th * kD + d;
  if (p.out_bf16) reinterpret_cast<uint16_t*>(p.out)[o] = (uint16_t)f2bf(val);
  else reinterpret_cast<float*>(p.out)[o] = val;
  if (p.lse != nullptr && d == 0) p.lse[th] = Ls > 0.f ? (M + __log2f(Ls)) * kLn2 : -INFINITY;
}

// ================================================================ token gather (16 heads per KV head)
constexpr int kGatherWaves = 4;

__global__ __launch_bounds__(64 * kGatherWaves) void k_token_gather(GatherParams p) {
  __shared__ uint16_t VT[kGatherWaves][kD * kVS];
  __shared__ int32_t KEYS[kGatherWaves][kBlk];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, l16 = lane & 15, qd = lane >> 4;
  const int64_t item = (int64_t)blockIdx.x * kGatherWaves + w;  // (t, g)
  if (item >= (int64_t)p.T * p.hkv) return;
  const int t = (int)(item / p.hkv), g = (int)(item % p.hkv);
  const int64_t N = p.n_ctx;
  const uint16_t* kb = p.k + (int64_t)g * N * kD;
  const uint16_t* vb = p.v + (int64_t)g * N * kD;
  const int32_t* ids = p.tok_idx + (int64_t)t * p.n_tok;
  const int h = g * 16 + l16;
  const float sl2 = p.scale * kLog2e;
  // Q^T: lane holds head l16, dims 32qd + 8s .. +7 at step s
  bf16x8 qv[4];
  {
    const uint16_t* qr = p.q + ((int64_t)t * p.hq + h) * kD + 32 * qd;
#pragma unroll
    for (int s = 0; s < 4; ++s) qv[s] = as_bf16x8(ldg16(qr + 8 * s));
  }
  f32x4 o[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int r = 0; r < 4; ++r) o[dt][r] = 0.f;
  float m = -INFINITY, l = 0.f;
  const int ntile = (p.n_tok + kBlk - 1) / kBlk;
  const int64_t qlim = p.q_pos != nullptr ? (int64_t)p.q_pos[t] : INT64_MAX;
  // the next tile's ids are requested one tile ahead, so a tile waits for one
  // memory latency (its K and V rows) instead of two
  int id_next = ntile > 0 && lane < min(kBlk, p.n_tok) ? ids[lane] : -1;
  for (int tt = 0; tt < ntile; ++tt) {
    const int base = tt * kBlk;
    int myid = id_next;
    if (tt + 1 < ntile) {
      const int nbase = base + kBlk;
      id_next = lane < min(kBlk, p.n_tok - nbase) ? ids[nbase + lane] : -1;
    }
    if (myid >= N || myid > qlim) myid = -1;  // out-of-range and future ids are treated as padding
    KEYS[w][lane] = myid;
    wave_sync();
    // rows to load (invalid slots read row 0 of a valid key; they are masked)
    int first = KEYS[w][0] >= 0 ? KEYS[w][0] : 0;
    int rows[16];
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int id = KEYS[w][v_slot(lane, n, e)];
        rows[4 * n + e] = id >= 0 ? id : first;
      }
    VRegs VR;
    v_fetch(VR, vb, rows, lane);
    bf16x8 ka[4][4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const int id = KEYS[w][16 * mt + l16];
      const uint16_t* kr = kb + (int64_t)(id >= 0 ? id : first) * kD + 32 * qd;
#pragma unroll
      for (int s = 0; s < 4; ++s) ka[mt][s] = as_bf16x8(ldg16(kr + 8 * s));
    }
    wave_sync();
    v_store<16>(VT[w], VR, lane);
    wave_sync();
    f32x4 sc[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
      for (int r = 0; r < 4; ++r) sc[mt][r] = 0.f;
#pragma unroll
      for (int s = 0; s < 4; ++s) sc[mt] = mfma16x16x32(ka[mt][s], qv[s], sc[mt]);
    }
    // element (mt, r): head l16, key slot 16mt + 4qd + r
    float x[16];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int slot = 16 * mt + 4 * qd + r;
        x[4 * mt + r] = KEYS[w][slot] >= 0 ? sc[mt][r] * sl2 : -INFINITY;
      }
    float mx = x[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, x[r]);
    mx = xor16_max(mx);
    mx = xor32_max(mx);
    const float mnew = fmaxf(m, mx);
    const float muse = (mnew == -INFINITY) ? 0.f : mnew;
    const float alpha = fast_exp2(m - muse);
    float ps = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      x[r] = fast_exp2(x[r] - muse);
      ps += x[r];
    }
    ps = xor16_add(ps);
    ps = xor32_add(ps);
    l = l * alpha + ps;
    m = mnew;
    // P^T for k-step ks: registers of M tiles 2ks and 2ks+1
    bf16x8 pv[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      u32x4 u;
#pragma unroll
      for (int e = 0; e < 4; ++e) u[e] = pack_bf16x2(x[8 * ks + 2 * e], x[8 * ks + 2 * e + 1]);
      pv[ks] = as_bf16x8(u);
    }
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
#pragma unroll
      for (int r = 0; r < 4; ++r) o[dt][r] *= alpha;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 a = as_bf16x8(*reinterpret_cast<const u32x4*>(&VT[w][(16 * dt + l16) * kVS + 32 * ks + 8 * qd]));
        o[dt] = mfma16x16x32(a, pv[ks], o[dt]);
      }
    }
    wave_sync();
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const int64_t orow = (int64_t)t * p.hq + h;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    const int d0 = 16 * dt + 4 * qd;
    if (p.out_bf16) {
      u32x2 pk;
      pk[0] = pack_bf16x2(o[dt][0] * inv, o[dt][1] * inv);
      pk[1] = pack_bf16x2(o[dt][2] * inv, o[dt][3] * inv);
      *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(p.out) + orow * kD + d0) = pk;
    } else {
      f32x4 v4;
      for (int r = 0; r < 4; ++r) v4[r] = o[dt][r] * inv;
      *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p.out) + orow * kD + d0) = v4;
    }
  }
  if (p.lse != nullptr && qd == 0) p.lse[orow] = l > 0.f ? (m + __log2f(l)) * kLn2 : -INFINITY;
}

// ================================================================ token gather, any head grouping
// One wave per (token, query head) over its own list (tok_idx [T, hq, n_tok])
// or its token's list ([T, n_tok]), any number of query heads per KV head.
// Per 64-id tile each lane scores one listed key (its 256-byte K row against
// q from LDS, fp32), the wave takes the tile's max and sum, and the P.V
// update gives each lane 8 dimensions of every fourth key (V rows read 16
// bytes per lane, one row per 16 lanes); the four key groups are summed at the
// end in a fixed order.
constexpr int kListWaves = 4;

__global__ __launch_bounds__(64 * kListWaves) void k_token_gather_list(GatherParams p) {
  __shared__ float QS[kListWaves][kD];
  __shared__ float PS[kListWaves][kBlk];
  __shared__ int32_t IDS[kListWaves][kBlk];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t item = (int64_t)blockIdx.x * kListWaves + w;  // (t, h)
  if (item >= (int64_t)p.T * p.hq) return;  // whole waves only: no workgroup barrier below
  const int t = (int)(item / p.hq), h = (int)(item % p.hq);
  const int g = h / (p.hq / p.hkv);
  const int64_t N = p.n_ctx;
  const uint16_t* kb = p.k + (int64_t)g * N * kD;
  const uint16_t* vb = p.v + (int64_t)g * N * kD;
  const int32_t* ids = p.tok_idx + (p.tok_per_head ? item : (int64_t)t) * p.n_tok;
  const int64_t qlim = p.q_pos != nullptr ? (int64_t)p.q_pos[t] : INT64_MAX;
  const float sl2 = p.scale * kLog2e;
  {
    const uint16_t* qr = p.q + item * kD;
    QS[w][2 * lane] = bf2f(qr[2 * lane]);
    QS[w][2 * lane + 1] = bf2f(qr[2 * lane + 1]);
  }
  wave_sync();
  const int kg = lane >> 4, dc = lane & 15;
  float o[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = 0.f;
  float m = -INFINITY, l = 0.f;
  int id_next = lane < p.n_tok ? ids[lane] : -1;  // the next tile's ids, read one tile ahead
  for (int base = 0; base < p.n_tok; base += kBlk) {
    int id = id_next;
    if (base + kBlk < p.n_tok) id_next = base + kBlk + lane < p.n_tok ? ids[base + kBlk + lane] : -1;
    if (id >= N || id > qlim) id = -1;  // out-of-range and future ids are padding
    float s = -INFINITY;
    if (id >= 0) {
      const uint16_t* kr = kb + (int64_t)id * kD;
      float acc = 0.f;
#pragma unroll
      for (int c = 0; c < kD / 8; ++c) {
        const u32x4 kv = ldg16(kr + 8 * c);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc = fmaf(QS[w][8 * c + 2 * e], __uint_as_float(kv[e] << 16), acc);
          acc = fmaf(QS[w][8 * c + 2 * e + 1], __uint_as_float(kv[e] & 0xffff0000u), acc);
        }
      }
      s = acc * sl2;
    }
    float mx = s;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    const float mnew = fmaxf(m, mx);
    if (mnew == -INFINITY) continue;  // nothing admissible yet (wave-uniform)
    const float alpha = fast_exp2(m - mnew);  // m = -inf gives 0
    const float pr = id >= 0 ? fast_exp2(s - mnew) : 0.f;
    float ps = pr;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) ps += __shfl_xor(ps, off);
    l = l * alpha + ps;
    m = mnew;
    PS[w][lane] = pr;
    IDS[w][lane] = id;
    wave_sync();
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] *= alpha;
#pragma unroll 4
    for (int i = 0; i < kBlk / 4; ++i) {
      const int j = 4 * i + kg;
      const int jid = IDS[w][j];
      if (jid >= 0) {
        const float pj = PS[w][j];
        const u32x4 vv = ldg16(vb + (int64_t)jid * kD + 8 * dc);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          o[2 * e] = fmaf(pj, __uint_as_float(vv[e] << 16), o[2 * e]);
          o[2 * e + 1] = fmaf(pj, __uint_as_float(vv[e] & 0xffff0000u), o[2 * e + 1]);
        }
      }
    }
    wave_sync();  // PS / IDS are rewritten by the next tile
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    o[e] = xor16_add(o[e]);
    o[e] = xor32_add(o[e]);
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  if (kg == 0) {
    if (p.out_bf16) {
      u32x4 pk;
#pragma unroll
      for (int e = 0; e < 4; ++e) pk[e] = pack_bf16x2(o[2 * e] * inv, o[2 * e + 1] * inv);
      stg16(reinterpret_cast<uint16_t*>(p.out) + item * kD + 8 * dc, pk);
    } else {
      float* op = reinterpret_cast<float*>(p.out) + item * kD + 8 * dc;
      f32x4 a = {o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv};
      f32x4 b = {o[4] * inv, o[5] * inv, o[6] * inv, o[7] * inv};
      *reinterpret_cast<f32x4*>(op) = a;
      *reinterpret_cast<f32x4*>(op + 4) = b;
    }
  }
  if (p.lse != nullptr && lane == 0) p.lse[item] = l > 0.f ? (m + __log2f(l)) * kLn2 : -INFINITY;
}

size_t a256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace

// ---------------------------------------------------------------- launchers
size_t cluster_pack_workspace_bytes(int64_t hkv, int64_t n, int C) {
  const int64_t nseg = (n + kSeg - 1) / kSeg;
  return a256((size_t)(hkv * nseg * C) * 4);
}

hipError_t launch_cluster_pack(const int32_t* labels, int64_t hkv, int64_t n, int C, int32_t* ptr, int32_t* perm,
                               const void* k, const void* v, void* kp, void* vp, int head_dim, int elem_bytes,
                               int32_t* err, void* ws, hipStream_t stream) {
  const int nseg = (int)((n + kSeg - 1) / kSeg);
  int32_t* seg = reinterpret_cast<int32_t*>(ws);
  const dim3 grid((unsigned)(hkv * nseg));
  hipLaunchKernelGGL(k_pack_count, grid, dim3(256), (size_t)C * 4, stream, labels, n, C, nseg, seg, err);
  if (C <= kScanThreads)
    hipLaunchKernelGGL(k_pack_scan_cm, dim3((unsigned)hkv), dim3(kScanThreads), 0, stream, C, nseg, seg, ptr);
  else
    hipLaunchKernelGGL(k_pack_scan, dim3((unsigned)hkv), dim3(kScanThreads), 0, stream, C, nseg, seg, ptr);
  hipLaunchKernelGGL(k_pack_scatter, grid, dim3(256), 0, stream, labels, n, C, nseg, seg, perm);
  if (kp != nullptr) {
    const int row_bytes = head_dim * elem_bytes;
    const int64_t chunks = hkv * n * (row_bytes / 16);
    const unsigned blocks = (unsigned)std::min<int64_t>(8192, (chunks + 255) / 256);
    hipLaunchKernelGGL(k_pack_copy, dim3(blocks), dim3(256), 0, stream, (const uint8_t*)k, (uint8_t*)kp, perm, ptr, n, C,
                       row_bytes, chunks);
    hipLaunchKernelGGL(k_pack_copy, dim3(blocks), dim3(256), 0, stream, (const uint8_t*)v, (uint8_t*)vp, perm, ptr, n, C,
                       row_bytes, chunks);
  }
  return hipGetLastError();
}

size_t cluster_decode_workspace_bytes(int T, int hq, int hkv, int C, int64_t n_ctx) {
  (void)T;
  (void)hq;
  (void)C;
  return a256((size_t)hkv * decode_splits(n_ctx) * 64 * (kD + 2) * 4);
}

hipError_t launch_cluster_decode(const GatherParams& p, void* ws, hipStream_t stream) {
  const int nsplit = decode_splits(p.n_ctx);
  float* part = reinterpret_cast<float*>(ws);
  const int nq = p.T * (p.hq / p.hkv);
  const dim3 grid(p.hkv * nsplit);
  const bool causal = p.q_pos != nullptr;
  if (nq <= 32 && !causal)
    hipLaunchKernelGGL((k_decode_split<1, false>), grid, dim3(64 * kDecWaves), 0, stream, p, part, nsplit);
  else if (nq <= 32)
    hipLaunchKernelGGL((k_decode_split<1, true>), grid, dim3(64 * kDecWaves), 0, stream, p, part, nsplit);
  else if (!causal)
    hipLaunchKernelGGL((k_decode_split<2, false>), grid, dim3(64 * kDecWaves), 0, stream, p, part, nsplit);
  else
    hipLaunchKernelGGL((k_decode_split<2, true>), grid, dim3(64 * kDecWaves), 0, stream, p, part, nsplit);
  hipLaunchKernelGGL(k_decode_combine, dim3(p.T * p.hq), dim3(kD), 0, stream, p, part, nsplit);
  return hipGetLastError();
}

size_t token_gather_workspace_bytes(int T, int hq, int n_tok) {
  (void)T;
  (void)hq;
  (void)n_tok;
  return 0;
}

hipError_t launch_token_gather(const GatherParams& p, void* ws, hipStream_t stream) {
  (void)ws;
  if (p.tok_per_head || p.hq != 16 * p.hkv) {
    const int64_t items = (int64_t)p.T * p.hq;
    hipLaunchKernelGGL(k_token_gather_list, dim3((unsigned)((items + kListWaves - 1) / kListWaves)),
                       dim3(64 * kListWaves), 0, stream, p);
    return hipGetLastError();
  }
  const int64_t items = (int64_t)p.T * p.hkv;
  hipLaunchKernelGGL(k_token_gather, dim3((unsigned)((items + kGatherWaves - 1) / kGatherWaves)),
                     dim3(64 * kGatherWaves), 0, stream, p);
  return hipGetLastError();
}

}  // namespace sa
