// Cheap estimators: block mean pooling and pooled block scores, and
// query-centroid scores.
//
// "MInference 1.0" article, §方法介紹: block-sparse indices come from the
// mean-pooled Q and K; pooling commutes with the product, so the pooled score
// of a block pair is the mean of that 64x64 block of Q K^T.
// Squeezed Attention page, §技术方案: every query is compared with every
// cluster centroid, the centroids being held in on-chip shared memory.
#include "common.h"
#include "launch.h"
#include "select_util.h"

namespace sa {
namespace {

constexpr int kBlk = 64;

// ---------------------------------------------------------------- k_pool
// One workgroup per (row of heads, block): 64 rows x D read with 16-byte
// loads (HBM-streaming), fp32 partial sums per thread, a fixed-order
// reduction through LDS, then the mean.
template <typename T, int D>
__global__ __launch_bounds__(256) void k_pool(const T* __restrict__ x, int hq, HeadList hl, int64_t seq, int nb,
                                              float* __restrict__ out) {
  constexpr int E = 16 / sizeof(T);  // elements per 16-byte chunk
  constexpr int CPR = D / E;         // chunks per row
  constexpr int RPP = 256 / CPR;     // rows per pass
  __shared__ float red[RPP][D];
  const int tid = threadIdx.x;
  const int64_t r = blockIdx.x / nb;
  const int j = blockIdx.x % nb;
  const int rp = tid / CPR, c = tid % CPR;
  int sb, sh;
  listed_row(r, hq, hl, sb, sh);
  const T* base = x + (((int64_t)sb * hq + sh) * seq + (int64_t)j * kBlk) * D + c * E;
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
#pragma unroll
  for (int row = rp; row < kBlk; row += RPP) {
    const u32x4 v = ldg16(base + (int64_t)row * D);
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += bf2f((uint16_t)((v[e >> 1] >> ((e & 1) * 16)) & 0xffffu));
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] += __uint_as_float(v[e]);
    }
  }
#pragma unroll
  for (int e = 0; e < E; ++e) red[rp][c * E + e] = acc[e];
  __syncthreads();
  if (tid < D) {
    float s = 0.f;
#pragma unroll
    for (int q = 0; q < RPP; ++q) s += red[q][tid];
    out[((int64_t)r * nb + j) * D + tid] = s * (1.0f / kBlk);
  }
}

// ---------------------------------------------------------------- k_block_score
// S[b,h,i,j] = pooled_q[b,h,i] . pooled_k[b,g(h),j] * scale for j <= i.
// 64x64 output tile per workgroup, 4x4 per thread, fp32 FMAs in dimension
// order.  Tiles strictly above the diagonal only write -inf.
__global__ __launch_bounds__(256) void k_block_score(const float* __restrict__ pq, const float* __restrict__ pk,
                                                     int hq, int hkv, HeadList hl, int nb, int D, float scale,
                                                     float* __restrict__ S) {
  __shared__ float Qs[64][33];
  __shared__ float Ks[64][33];
  const int tid = threadIdx.x, tx = tid % 16, ty = tid / 16;
  const int nbt = (nb + 63) / 64;
  const int bh = blockIdx.x / (nbt * nbt);
  const int tile = blockIdx.x % (nbt * nbt);
  const int ti = tile / nbt, tj = tile % nbt;
  int b, h;
  listed_row(bh, hq, hl, b, h);
  const int g = (h * hkv) / hq;
  float* Sb = S + (int64_t)bh * nb * nb;
  if (tj > ti) {
    for (int e = tid; e < 64 * 64; e += 256) {
      const int i = ti * 64 + e / 64, j = tj * 64 + e % 64;
      if (i < nb && j < nb) Sb[(int64_t)i * nb + j] = -INFINITY;
    }
    return;
  }
  const float* Qb = pq + (int64_t)bh * nb * D;
  const float* Kb = pk + ((int64_t)b * hkv + g) * nb * D;
  float acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[a][c] = 0.f;
  for (int d0 = 0; d0 < D; d0 += 32) {
    for (int e = tid; e < 64 * 32; e += 256) {
      const int rr = e / 32, dd = e % 32;
      const int qi = ti * 64 + rr, kj = tj * 64 + rr;
      Qs[rr][dd] = qi < nb ? Qb[(int64_t)qi * D + d0 + dd] : 0.f;
      Ks[rr][dd] = kj < nb ? Kb[(int64_t)kj * D + d0 + dd] : 0.f;
    }
    __syncthreads();
#pragma unroll 8
    for (int dd = 0; dd < 32; ++dd) {
      float qv[4], kv[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) qv[a] = Qs[ty + 16 * a][dd];
#pragma unroll
      for (int c = 0; c < 4; ++c) kv[c] = Ks[tx + 16 * c][dd];
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[a][c] = fmaf(qv[a], kv[c], acc[a][c]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int i = ti * 64 + ty + 16 * a, j = tj * 64 + tx + 16 * c;
      if (i < nb && j < nb) Sb[(int64_t)i * nb + j] = (j <= i) ? acc[a][c] * scale : -INFINITY;
    }
}

// 128x128 tile of S per workgroup on the fp32 matrix cores
// (v_mfma_f32_32x32x2_f32: fp32 products, fp32 accumulation).  The pooled Q
// and K rows of the tile pass through LDS 32 dimensions at a time.  Step kk of
// the product takes dimension 2kk + hf from lane half hf, so within each group
// of 8 dimensions LDS holds the even ones, then the odd ones: one 16-byte read
// gives a lane its operands for four steps.  Row pitch 36 floats: sixteen
// consecutive rows' 16-byte reads hit distinct banks.  Wave (wi, wj) computes
// the 64x64 quarter (wi, wj) as 2x2 MFMA tiles.  Tiles above the diagonal only
// write -inf.
template <int D>
__global__ __launch_bounds__(256) void k_block_score_mfma(const float* __restrict__ pq, const float* __restrict__ pk,
                                                          int hq, int hkv, HeadList hl, int nb, float scale,
                                                          float* __restrict__ S) {
  constexpr int T = 128, DC = 32, P = DC + 4;
  __shared__ __attribute__((aligned(16))) float Qs[T * P];
  __shared__ __attribute__((aligned(16))) float Ks[T * P];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, hf = lane >> 5, l32 = lane & 31;
  const int nbt = (nb + T - 1) / T;
  const int bh = blockIdx.x / (nbt * nbt);
  const int tile = blockIdx.x % (nbt * nbt);
  const int ti = tile / nbt, tj = tile % nbt;
  int b, h;
  listed_row(bh, hq, hl, b, h);
  const int g = (h * hkv) / hq;
  float* Sb = S + (int64_t)bh * nb * nb;
  if (tj > ti) {
    if ((nb & 3) == 0 && (reinterpret_cast<uintptr_t>(S) & 15) == 0) {  // 16-byte aligned rows
      const f32x4 ninf = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
      for (int e = tid; e < T * T / 4; e += 256) {
        const int i = ti * T + e / (T / 4), j = tj * T + 4 * (e % (T / 4));
        if (i < nb && j < nb) *reinterpret_cast<f32x4*>(Sb + (int64_t)i * nb + j) = ninf;
      }
    } else {
      for (int e = tid; e < T * T; e += 256) {
        const int i = ti * T + e / T, j = tj * T + e % T;
        if (i < nb && j < nb) Sb[(int64_t)i * nb + j] = -INFINITY;
      }
    }
    return;
  }
  const float* Qb = pq + (int64_t)bh * nb * D;
  const float* Kb = pk + ((int64_t)b * hkv + g) * nb * D;
  const int wi = wv >> 1, wj = wv & 1;
  f32x16 acc[2][2] = {};
  for (int d0 = 0; d0 < D; d0 += DC) {
    for (int e = tid; e < T * (DC / 4); e += 256) {
      const int rr = e / (DC / 4), c4 = e % (DC / 4);
      const int qi = ti * T + rr, kj = tj * T + rr;
      const f32x4 z = {0.f, 0.f, 0.f, 0.f};
      const f32x4 vq = qi < nb ? *reinterpret_cast<const f32x4*>(Qb + (int64_t)qi * D + d0 + 4 * c4) : z;
      const f32x4 vk = kj < nb ? *reinterpret_cast<const f32x4*>(Kb + (int64_t)kj * D + d0 + 4 * c4) : z;
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int j = 4 * c4 + x, pos = (j & ~7) + 4 * (j & 1) + ((j & 7) >> 1);  // even dims, then odd ones
        Qs[rr * P + pos] = vq[x];
        Ks[rr * P + pos] = vk[x];
      }
    }
    __syncthreads();
#pragma unroll
    for (int k8 = 0; k8 < DC / 8; ++k8) {
      // steps 4k8 .. 4k8+3: dimensions 8k8 + 2x + hf
      f32x4 qa[2], kb[2];
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        qa[m] = *reinterpret_cast<const f32x4*>(&Qs[(64 * wi + 32 * m + l32) * P + 8 * k8 + 4 * hf]);  // A: row l32
        kb[m] = *reinterpret_cast<const f32x4*>(&Ks[(64 * wj + 32 * m + l32) * P + 8 * k8 + 4 * hf]);  // B: column l32
      }
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int n = 0; n < 2; ++n)
            acc[m][n] = __builtin_amdgcn_mfma_f32_32x32x2f32(qa[m][x], kb[n][x], acc[m][n], 0, 0, 0);
    }
    __syncthreads();
  }
  // element r of tile (m, n): row 64wi + 32m + 8(r/4) + 4hf + r%4, column 64wj + 32n + l32
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = ti * T + 64 * wi + 32 * m + 8 * (r / 4) + 4 * hf + (r % 4);
        const int j = tj * T + 64 * wj + 32 * n + l32;
        if (i < nb && j < nb) Sb[(int64_t)i * nb + j] = (j <= i) ? acc[m][n][r] * scale : -INFINITY;
      }
}

// ---------------------------------------------------------------- k_centroid_score
// One workgroup per (KV head, chunk of 8 centroids), 256 of them at the decode
// size.  The chunk's centroids and all queries of the KV head's group sit in
// LDS; each thread computes (query, centroid) dot products in fp32.
constexpr int kCentChunk = 8;

template <typename T>
__global__ __launch_bounds__(256) void k_centroid_score(const T* __restrict__ q, const float* __restrict__ cent,
                                                        int T_, int hq, int hkv, int C, int D, float scale,
                                                        float* __restrict__ out) {
  extern __shared__ float sm[];
  const int grp = hq / hkv;
  const int nq = T_ * grp;
  const int nchunk = (C + kCentChunk - 1) / kCentChunk;
  const int g = blockIdx.x / nchunk, c0 = (blockIdx.x % nchunk) * kCentChunk;
  float* Cs = sm;                         // [kCentChunk][D+1]
  float* Qs = sm + kCentChunk * (D + 1);  // [nq][D+1]
  for (int e = threadIdx.x; e < kCentChunk * D; e += blockDim.x) {
    const int c = e / D, d = e % D;
    Cs[c * (D + 1) + d] = (c0 + c < C) ? cent[((int64_t)g * C + c0 + c) * D + d] : 0.f;
  }
  for (int e = threadIdx.x; e < nq * D; e += blockDim.x) {
    const int qi = e / D, d = e % D;
    const int t = qi / grp, h = g * grp + qi % grp;
    const T* qp = q + ((int64_t)t * hq + h) * D + d;
    float v;
    if constexpr (sizeof(T) == 2) v = bf2f(*reinterpret_cast<const uint16_t*>(qp));
    else v = *reinterpret_cast<const float*>(qp);
    Qs[qi * (D + 1) + d] = v;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < nq * kCentChunk; e += blockDim.x) {
    const int qi = e / kCentChunk, c = e % kCentChunk;
    if (c0 + c >= C) continue;
    const float* qr = Qs + qi * (D + 1);
    const float* cr = Cs + c * (D + 1);
    float acc = 0.f;
    if (D == 128) {
#pragma unroll
      for (int d = 0; d < 128; ++d) acc = fmaf(qr[d], cr[d], acc);
    } else {
#pragma unroll 8
      for (int d = 0; d < D; ++d) acc = fmaf(qr[d], cr[d], acc);
    }
    const int t = qi / grp, h = g * grp + qi % grp;
    out[((int64_t)t * hq + h) * C + c0 + c] = acc * scale;
  }
}

// ---------------------------------------------------------------- k_centroid_topk
// Centroid scores and the per-row top-k in one pass, for decode: a workgroup
// covers nrow query heads of one token that share a KV head (one head per
// workgroup at launch, which spreads the centroid rows' loads over four times
// as many CUs as one workgroup per KV head).  Thread c owns centroids c, c+256,
// ...: it reads each centroid row (its loads issued together) and computes its
// score for every row (dimension order, fp32, as k_centroid_score), keeping
// order-preserving keys in LDS.  Per row, an
// MSB-first radix select (8-bit digits, LDS histograms, 32 threads per row for
// the digit) finds the k-th key T; candidates above T and the lowest-index
// keys equal to T are written in cluster order.
constexpr int kCtThreads = 256;
constexpr int kCtMaxRows = 8;
constexpr int kCtMaxC = 1024;

// MASS: one row per workgroup; instead of the fixed top-k, the adaptive
// budget of sa_select_mass (mass_select_lds) on the row's keys, with k as the
// upper clamp.
template <typename T, bool MASS>
__global__ __launch_bounds__(kCtThreads) void k_centroid_topk(const T* __restrict__ q, const float* __restrict__ cent,
                                                              int hq, int hkv, int C, int D, float scale, int k,
                                                              int kmax, int nsub, float mass, int k_min,
                                                              int32_t* __restrict__ idx, int32_t* __restrict__ cnt,
                                                              int32_t* err) {
  __shared__ float qs[kCtMaxRows][128];
  __shared__ uint32_t keys[kCtMaxRows][kCtMaxC];
  __shared__ uint32_t hist[kCtMaxRows][256];
  __shared__ uint32_t s_digit[kCtMaxRows][2];
  __shared__ int32_t s_need[kCtMaxRows];
  __shared__ uint32_t s_wave[kCtThreads / 64][kCtMaxRows][2];
  __shared__ uint32_t s_nan;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  // workgroup (t, s, g): token t, KV head g (innermost, so one KV head's
  // centroid rows stay in one XCD's L2), rows s*nrow .. of the g's query heads
  const int grp = hq / hkv, nrow = grp / nsub;
  const int g = blockIdx.x % hkv, ts = blockIdx.x / hkv;
  const int t = ts / nsub, h0 = g * grp + (ts % nsub) * nrow;
  const int kr = min(k, C);
  if (tid == 0) s_nan = 0u;
  for (int e = tid; e < nrow * D; e += kCtThreads) {
    const int hh = e / D, d = e % D;
    const T* qp = q + ((int64_t)t * hq + h0 + hh) * D + d;
    if constexpr (sizeof(T) == 2) qs[hh][d] = bf2f(*reinterpret_cast<const uint16_t*>(qp));
    else qs[hh][d] = *reinterpret_cast<const float*>(qp);
  }
  if (tid < nrow) s_need[tid] = kr;
  __syncthreads();
  // ---- scores -> keys
  bool nan_seen = false;
  for (int c = tid; c < C; c += kCtThreads) {
    const float* cr = cent + ((int64_t)g * C + c) * D;
    float acc[kCtMaxRows];
#pragma unroll
    for (int hh = 0; hh < kCtMaxRows; ++hh) acc[hh] = 0.f;
    auto fma4 = [&](int d0, const f32x4& m4) {
#pragma unroll
      for (int hh = 0; hh < kCtMaxRows; ++hh)
        if (hh < nrow) {
          acc[hh] = fmaf(qs[hh][d0], m4[0], acc[hh]);
          acc[hh] = fmaf(qs[hh][d0 + 1], m4[1], acc[hh]);
          acc[hh] = fmaf(qs[hh][d0 + 2], m4[2], acc[hh]);
          acc[hh] = fmaf(qs[hh][d0 + 3], m4[3], acc[hh]);
        }
    };
    // the row's loads are issued before its products (16 in flight), so one
    // memory latency covers a 64-dimension half instead of one per 4 dimensions
    int d0 = 0;
    for (; d0 + 64 <= D; d0 += 64) {
      f32x4 m4[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) m4[u] = *reinterpret_cast<const f32x4*>(cr + d0 + 4 * u);
#pragma unroll
      for (int u = 0; u < 16; ++u) fma4(d0 + 4 * u, m4[u]);
    }
    for (; d0 < D; d0 += 4) fma4(d0, *reinterpret_cast<const f32x4*>(cr + d0));
#pragma unroll
    for (int hh = 0; hh < kCtMaxRows; ++hh)
      if (hh < nrow) {
        const float sc = acc[hh] * scale;
        nan_seen |= is_nan(sc);
        keys[hh][c] = order_key(sc);
      }
  }
  if (nan_seen) atomicOr(&s_nan, 1u);
  if constexpr (MASS) {
    // one row: (key << 32 | ~index) pairs, padded to a power of two, then the adaptive budget
    __shared__ uint64_t kv[kCtMaxC];
    __shared__ uint32_t bm[kCtMaxC / 32];
    __shared__ uint64_t wtmp[kCtThreads / 64];
    __shared__ uint32_t utmp[kCtThreads / 64];
    __syncthreads();
    int P = 64;
    while (P < C) P <<= 1;
    for (int c = tid; c < P; c += kCtThreads)
      kv[c] = c < C ? (((uint64_t)keys[0][c] << 32) | (uint64_t)(~(uint32_t)c)) : 0ull;
    __syncthreads();
    const int64_t row = (int64_t)t * hq + h0;
    mass_select_lds<kCtThreads>(kv, bm, wtmp, utmp, C, P, mass, k_min, k, idx + row * kmax, kmax, cnt + row);
    if (tid == 0 && s_nan && err != nullptr) atomicOr(reinterpret_cast<unsigned int*>(err), 1u);
    return;
  }
  // ---- radix select: T[hh] = the kr-th largest key of row hh
  uint32_t Tk[kCtMaxRows];
#pragma unroll
  for (int hh = 0; hh < kCtMaxRows; ++hh) Tk[hh] = 0u;
  constexpr int TPR = kCtThreads / kCtMaxRows;  // 32 threads per row in the digit search
#pragma unroll 1
  for (int shift = 24; shift >= 0; shift -= 8) {
    const uint32_t hmask = shift == 24 ? 0u : ~((1u << (shift + 8)) - 1u);
    for (int e = tid; e < kCtMaxRows * 256; e += kCtThreads) (&hist[0][0])[e] = 0u;
    __syncthreads();
    for (int c = tid; c < C; c += kCtThreads)
#pragma unroll
      for (int hh = 0; hh < kCtMaxRows; ++hh)
        if (hh < nrow) {
          const uint32_t key = keys[hh][c];
          if ((key & hmask) == (Tk[hh] & hmask)) atomicAdd(&hist[hh][(key >> shift) & 255u], 1u);
        }
    __syncthreads();
    {
      const int row = tid / TPR, seg = tid % TPR;
      if (row < nrow) {
        const int rneed = s_need[row];
        uint32_t loc = 0u;
#pragma unroll
        for (int x = 0; x < 8; ++x) loc += hist[row][8 * seg + x];
        uint32_t incl = loc;
#pragma unroll
        for (int off = 1; off < TPR; off <<= 1) {
          const uint32_t o = __shfl_down(incl, off, TPR);
          if (seg + off < TPR) incl += o;
        }
        const uint32_t above = incl - loc;
        if (rneed == 0) {
          if (seg == TPR - 1) {
            s_digit[row][0] = 255u;
            s_digit[row][1] = 0u;
          }
        } else if (above < (uint32_t)rneed && (uint32_t)rneed <= incl) {
          uint32_t acc = above;
          for (int dg = 8 * seg + 7; dg >= 8 * seg; --dg) {
            const uint32_t hc = hist[row][dg];
            if (acc + hc >= (uint32_t)rneed) {
              s_digit[row][0] = (uint32_t)dg;
              s_digit[row][1] = acc;
              break;
            }
            acc += hc;
          }
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int hh = 0; hh < kCtMaxRows; ++hh)
      if (hh < nrow) Tk[hh] |= s_digit[hh][0] << shift;
    if (tid < nrow) s_need[tid] -= (int)s_digit[tid][1];  // read again after two more barriers
  }
  __syncthreads();
  // ---- emission in cluster order: chunks of 256 candidates, ballots per wave
  const uint64_t lt = (1ull << lane) - 1ull;
  int base_f[kCtMaxRows], base_t[kCtMaxRows];
#pragma unroll
  for (int hh = 0; hh < kCtMaxRows; ++hh) base_f[hh] = base_t[hh] = 0;
  for (int c0 = 0; c0 < C; c0 += kCtThreads) {
    const int c = c0 + tid;
    uint64_t mf[kCtMaxRows], mt[kCtMaxRows];
#pragma unroll
    for (int hh = 0; hh < kCtMaxRows; ++hh) {
      const uint32_t key = (c < C && hh < nrow) ? keys[hh][c] : 0u;
      const bool live = c < C && hh < nrow;
      mf[hh] = __ballot(live && key > Tk[hh]);
      mt[hh] = __ballot(live && key == Tk[hh]);
      if (lane == 0) {
        s_wave[wv][hh][0] = (uint32_t)__popcll(mf[hh]);
        s_wave[wv][hh][1] = (uint32_t)__popcll(mt[hh]);
      }
    }
    __syncthreads();
#pragma unroll
    for (int hh = 0; hh < kCtMaxRows; ++hh) {
      if (hh >= nrow) continue;
      int wf = 0, wt = 0, af = 0, at = 0;
      for (int x = 0; x < kCtThreads / 64; ++x) {
        const int f = (int)s_wave[x][hh][0], e = (int)s_wave[x][hh][1];
        if (x < wv) {
          wf += f;
          wt += e;
        }
        af += f;
        at += e;
      }
      const int need = s_need[hh];
      const int fb = base_f[hh] + wf + (int)__popcll(mf[hh] & lt);
      const int tb = base_t[hh] + wt + (int)__popcll(mt[hh] & lt);
      int32_t* out = idx + ((int64_t)t * hq + h0 + hh) * kmax;
      if ((mf[hh] >> lane) & 1ull) out[fb + min(tb, need)] = c;
      else if (((mt[hh] >> lane) & 1ull) && tb < need) out[fb + tb] = c;
      base_f[hh] += af;
      base_t[hh] += at;
    }
    __syncthreads();
  }
  for (int e = tid; e < nrow * kmax; e += kCtThreads) {
    const int hh = e / kmax, pos = e % kmax;
    const int64_t row = (int64_t)t * hq + h0 + hh;
    if (pos >= kr) idx[row * kmax + pos] = -1;
    if (pos == 0) cnt[row] = kr;
  }
  if (tid == 0 && s_nan && err != nullptr) atomicOr(reinterpret_cast<unsigned int*>(err), 1u);
}

}  // namespace

hipError_t launch_centroid_topk(const void* q, bool q_bf16, const float* cent, int T, int hq, int hkv, int C,
                                int head_dim, float scale, int k, int kmax, float mass, int k_min, int32_t* idx,
                                int32_t* cnt, int32_t* err, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  // one query head per workgroup: four times the workgroups of one per KV head,
  // so the centroid rows' loads spread over more CUs
  const int nsub = hq / hkv;
  const dim3 grid((unsigned)(T * hkv * nsub));
#define SA_CT_LAUNCH(TQ, M)                                                                                 \
  hipLaunchKernelGGL((k_centroid_topk<TQ, M>), grid, dim3(kCtThreads), 0, stream, (const TQ*)q, cent, hq, hkv, C, \
                     head_dim, scale, k, kmax, nsub, mass, k_min, idx, cnt, err)
  if (q_bf16) {
    if (mass > 0.f) SA_CT_LAUNCH(uint16_t, true);
    else SA_CT_LAUNCH(uint16_t, false);
  } else {
    if (mass > 0.f) SA_CT_LAUNCH(float, true);
    else SA_CT_LAUNCH(float, false);
  }
#undef SA_CT_LAUNCH
  return hipGetLastError();
}

hipError_t launch_pool(const void* x, int64_t batch, int hq, const HeadList& hl, int64_t seq, int head_dim,
                       bool bf16, int block, float* out, hipStream_t stream) {
  if (block != kBlk) return hipErrorInvalidValue;
  const int nb = (int)(seq / kBlk);
  const int64_t nblk = batch * (hl.n > 0 ? hl.n : hq) * nb;
  if (nblk == 0) return hipSuccess;
  const dim3 grid((unsigned)nblk);
  if (bf16 && head_dim == 128)
    hipLaunchKernelGGL((k_pool<uint16_t, 128>), grid, dim3(256), 0, stream, (const uint16_t*)x, hq, hl, seq, nb, out);
  else if (bf16 && head_dim == 64)
    hipLaunchKernelGGL((k_pool<uint16_t, 64>), grid, dim3(256), 0, stream, (const uint16_t*)x, hq, hl, seq, nb, out);
  else if (!bf16 && head_dim == 128)
    hipLaunchKernelGGL((k_pool<float, 128>), grid, dim3(256), 0, stream, (const float*)x, hq, hl, seq, nb, out);
  else if (!bf16 && head_dim == 64)
    hipLaunchKernelGGL((k_pool<float, 64>), grid, dim3(256), 0, stream, (const float*)x, hq, hl, seq, nb, out);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_block_score(const float* pq, const float* pk, int batch, int hq, int hkv, const HeadList& hl,
                              int nb, int head_dim, float scale, float* scores, hipStream_t stream) {
  const int64_t rows = (int64_t)batch * (hl.n > 0 ? hl.n : hq);
  if (head_dim == 128 || head_dim == 64) {
    const int nbt2 = (nb + 127) / 128;
    const int64_t n2 = rows * nbt2 * nbt2;
    if (n2 == 0) return hipSuccess;
    if (head_dim == 128)
      hipLaunchKernelGGL((k_block_score_mfma<128>), dim3((unsigned)n2), dim3(256), 0, stream, pq, pk, hq, hkv, hl,
                         nb, scale, scores);
    else
      hipLaunchKernelGGL((k_block_score_mfma<64>), dim3((unsigned)n2), dim3(256), 0, stream, pq, pk, hq, hkv, hl,
                         nb, scale, scores);
    return hipGetLastError();
  }
  const int nbt = (nb + 63) / 64;
  const int64_t n = rows * nbt * nbt;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_block_score, dim3((unsigned)n), dim3(256), 0, stream, pq, pk, hq, hkv, hl, nb, head_dim,
                     scale, scores);
  return hipGetLastError();
}

hipError_t launch_centroid_score(const void* q, bool q_bf16, const float* cent, int T, int hq, int hkv,
                                 int C, int head_dim, float scale, float* out, hipStream_t stream) {
  const int grp = hq / hkv;
  const size_t lds = (size_t)(kCentChunk + T * grp) * (head_dim + 1) * sizeof(float);
  if (lds > 160 * 1024) return hipErrorInvalidValue;
  const int nchunk = (C + kCentChunk - 1) / kCentChunk;
  const dim3 grid(hkv * nchunk);
  if (q_bf16)
    hipLaunchKernelGGL((k_centroid_score<uint16_t>), grid, dim3(256), lds, stream, (const uint16_t*)q, cent, T,
                       hq, hkv, C, head_dim, scale, out);
  else
    hipLaunchKernelGGL((k_centroid_score<float>), grid, dim3(256), lds, stream, (const float*)q, cent, T, hq,
                       hkv, C, head_dim, scale, out);
  return hipGetLastError();
}

}  // namespace sa
