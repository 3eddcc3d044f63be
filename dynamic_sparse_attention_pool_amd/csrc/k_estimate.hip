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

// ---------------------------------------------------------------- k_block_score_direct
// S[b,h,i,j] = pooled_q[b,h,i] . pooled_k[b,g(h),j] * scale for j <= i.
// One wave per 64x64 tile of S at or below the diagonal (four waves per
// workgroup, tiles enumerated row by row over the lower triangle), operands
// straight from memory: the contraction over d is split between the two lane
// halves (half hf takes dimensions hf*D/2 .. +D/2-1, step kk its kk-th), so a
// lane reads 16 consecutive floats of its row per 16 steps with four 16-byte
// loads; the next 16 steps' operands are in flight while the current ones run
// on v_mfma_f32_32x32x2_f32 (fp32 products and accumulation) over four
// independent accumulators.  Entries above the diagonal are not written.
template <int D>
__global__ __launch_bounds__(256) void k_block_score_direct(const float* __restrict__ pq, const float* __restrict__ pk,
                                                            int hq, int hkv, HeadList hl, int64_t rows, int nb,
                                                            float scale, float* __restrict__ S,
                                                            int32_t* __restrict__ err) {
  constexpr int HALF = D / 2, NCH = HALF / 16;
  const int lane = threadIdx.x & 63, hf = lane >> 5, l32 = lane & 31;
  const int nbt = (nb + 63) / 64;
  const int64_t per_head = (int64_t)nbt * (nbt + 1) / 2;
  const int64_t wid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wid >= rows * per_head) return;  // whole waves only; no workgroup barrier below
  const int64_t bh = wid / per_head;
  const int t = (int)(wid % per_head);
  int ti = (int)((sqrtf(8.f * (float)t + 1.f) - 1.f) * 0.5f);
  while ((int64_t)(ti + 1) * (ti + 2) / 2 <= t) ++ti;
  while ((int64_t)ti * (ti + 1) / 2 > t) --ti;
  const int tj = t - ti * (ti + 1) / 2;
  int b, h;
  listed_row(bh, hq, hl, b, h);
  const int g = (h * hkv) / hq;
  const float* Qb = pq + bh * (int64_t)nb * D;
  const float* Kb = pk + ((int64_t)b * hkv + g) * (int64_t)nb * D;
  const float* qr[2];
  const float* kr[2];
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    qr[m] = Qb + (int64_t)min(64 * ti + 32 * m + l32, nb - 1) * D + HALF * hf;
    kr[m] = Kb + (int64_t)min(64 * tj + 32 * m + l32, nb - 1) * D + HALF * hf;
  }
  f32x4 A[2][2][4], B[2][2][4];
  auto load = [&](int c, int buf) {
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        A[buf][m][v] = *reinterpret_cast<const f32x4*>(qr[m] + 16 * c + 4 * v);
        B[buf][m][v] = *reinterpret_cast<const f32x4*>(kr[m] + 16 * c + 4 * v);
      }
  };
  f32x16 acc[2][2] = {};
  load(0, 0);
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    if (c + 1 < NCH) load(c + 1, (c + 1) & 1);
#pragma unroll
    for (int u = 0; u < 16; ++u)
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int n = 0; n < 2; ++n)
          acc[m][n] = __builtin_amdgcn_mfma_f32_32x32x2f32(A[c & 1][m][u / 4][u % 4], B[c & 1][n][u / 4][u % 4],
                                                          acc[m][n], 0, 0, 0);
  }
  // element r of tile (m, n): row 64ti + 32m + 8(r/4) + 4hf + r%4, column 64tj + 32n + l32
  float* Sb = S + bh * (int64_t)nb * nb;
  bool bad = false;
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = 64 * ti + 32 * m + 8 * (r / 4) + 4 * hf + (r % 4);
        const int j = 64 * tj + 32 * n + l32;
        if (i < nb && j <= i) {
          const float v = acc[m][n][r] * scale;
          Sb[(int64_t)i * nb + j] = v;
          bad |= nonfinite(v);
        }
      }
  flag_nonfinite(err, bad);
}

// ---------------------------------------------------------------- k_centroid_score
// One workgroup per (KV head, chunk of 8 centroids), 256 of them at the decode
// size.  The chunk's centroids and all queries of the KV head's group sit in
// LDS; each thread computes (query, centroid) dot products in fp32.
constexpr int kCentChunk = 8;

template <typename T>
__global__ __launch_bounds__(256) void k_centroid_score(const T* __restrict__ q, const float* __restrict__ cent,
                                                        int T_, int hq, int hkv, int C, int D, float scale,
                                                        float* __restrict__ out, int32_t* __restrict__ err) {
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
    const float v = acc * scale;
    out[((int64_t)t * hq + h) * C + c0 + c] = v;
    flag_nonfinite(err, nonfinite(v));
  }
}

// ---------------------------------------------------------------- k_centroid_topk
// Centroid scores and the adaptive budget in one pass, for decode: one
// workgroup per (token, query head).  Thread c owns centroids c, c+256, ...: it
// reads each centroid row (its loads issued together) and computes the row's
// score (dimension order, fp32, as k_centroid_score), keeping order-preserving
// keys in LDS; the adaptive budget of sa_select_mass (mass_select_lds) then
// runs on those keys, with k as the upper clamp.  The fixed budget takes
// k_centroid_topk_wave.
constexpr int kCtThreads = 256;
constexpr int kCtMaxC = 1024;

template <typename T>
__global__ __launch_bounds__(kCtThreads) void k_centroid_topk(const T* __restrict__ q, const float* __restrict__ cent,
                                                              int hq, int hkv, int C, int D, float scale, int k,
                                                              int kmax, float mass, int k_min,
                                                              int32_t* __restrict__ idx, int32_t* __restrict__ cnt,
                                                              int32_t* err) {
  __shared__ float qs[128];
  __shared__ uint32_t keys[kCtMaxC];
  __shared__ uint64_t kv[kCtMaxC];
  __shared__ uint32_t bm[kCtMaxC / 32];
  __shared__ uint64_t wtmp[kCtThreads / 64];
  __shared__ uint32_t utmp[kCtThreads / 64];
  __shared__ uint32_t s_nan;
  const int tid = threadIdx.x;
  // workgroup (t, h): KV head innermost, so one KV head's centroid rows stay
  // in one XCD's L2
  const int grp = hq / hkv;
  const int g = blockIdx.x % hkv, ts = blockIdx.x / hkv;
  const int t = ts / grp, h = g * grp + ts % grp;
  const int64_t row = (int64_t)t * hq + h;
  if (tid == 0) s_nan = 0u;
  for (int d = tid; d < D; d += kCtThreads) {
    const T* qp = q + row * D + d;
    if constexpr (sizeof(T) == 2) qs[d] = bf2f(*reinterpret_cast<const uint16_t*>(qp));
    else qs[d] = *reinterpret_cast<const float*>(qp);
  }
  __syncthreads();
  // ---- scores -> keys
  bool nan_seen = false;
  for (int c = tid; c < C; c += kCtThreads) {
    const float* cr = cent + ((int64_t)g * C + c) * D;
    float acc = 0.f;
    auto fma4 = [&](int d0, const f32x4& m4) {
      acc = fmaf(qs[d0], m4[0], acc);
      acc = fmaf(qs[d0 + 1], m4[1], acc);
      acc = fmaf(qs[d0 + 2], m4[2], acc);
      acc = fmaf(qs[d0 + 3], m4[3], acc);
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
    const float sc = acc * scale;
    nan_seen |= is_nan(sc);
    keys[c] = order_key(sc);
  }
  if (nan_seen) atomicOr(&s_nan, 1u);
  __syncthreads();
  // (key << 32 | ~index) pairs, padded to a power of two, then the adaptive budget
  int P = 64;
  while (P < C) P <<= 1;
  for (int c = tid; c < P; c += kCtThreads) kv[c] = c < C ? (((uint64_t)keys[c] << 32) | (uint64_t)(~(uint32_t)c)) : 0ull;
  __syncthreads();
  mass_select_lds<kCtThreads>(kv, bm, wtmp, utmp, C, P, mass, k_min, k, idx + row * kmax, kmax, cnt + row);
  if (tid == 0 && s_nan && err != nullptr) atomicOr(reinterpret_cast<unsigned int*>(err), 1u);
}

}  // namespace

// Centroid scores and the fixed top-k of one (token, query head) row per wave,
// with no workgroup barrier.  Lane l owns centroids l, l+64, ... (NPL of them):
// it reads their rows (a quarter row per centroid at a time, all loads of a
// quarter in flight together) and computes each score exactly as
// k_centroid_score does (fp32 FMAs in dimension order, then the scale), so
// the selection is bit-identical to sa_estimate(CENTROID) + sa_select_topk.
// The k-th largest order-preserving key T comes from a 32-step bitwise search
// (a candidate bit stays when at least k keys reach the prefix), and the
// emission walks the centroids in index order, 64 per ballot: keys above T,
// then keys equal to T while the k budget lasts (lower index first).
namespace {
// Top-k of one row whose scores a wave holds, NPL per lane (lane l has
// candidates l, l+64, ...): the k-th largest order-preserving key T by a
// 32-step bitwise search (a candidate bit stays when at least k keys reach the
// prefix), then emission in candidate order, 64 per ballot: keys above T and
// keys equal to T while the budget lasts (lower index first).  NaN scores set
// bit 0 of err.
template <int NPL>
__device__ __forceinline__ void wave_topk_emit(const float* acc, int C, float scale, int k, int kmax, int32_t* out,
                                               int32_t* cnt_out, int32_t* err, int lane) {
  uint32_t key[NPL];
  bool nan_seen = false;
#pragma unroll
  for (int j = 0; j < NPL; ++j) {
    const bool live = 64 * j + lane < C;
    const float sc = acc[j] * scale;
    nan_seen |= live && is_nan(sc);
    key[j] = live ? order_key(sc) : 0u;  // every real key is above 0 (NaN aside)
  }
  if (nan_seen && err != nullptr) atomicOr(reinterpret_cast<unsigned int*>(err), 1u);
  const int kr = min(k, C);
  uint32_t Tk = 0u;
  if (kr > 0) {
#pragma unroll 1
    for (int b = 31; b >= 0; --b) {
      const uint32_t cand = Tk | (1u << b);
      int n = 0;
#pragma unroll
      for (int j = 0; j < NPL; ++j) n += __popcll(__ballot(key[j] >= cand));
      if (n >= kr) Tk = cand;
    }
  }
  int nabove = 0;
#pragma unroll
  for (int j = 0; j < NPL; ++j) nabove += __popcll(__ballot(kr > 0 && key[j] > Tk));
  const int need = kr - nabove;
  const uint64_t lt = (1ull << lane) - 1ull;
  int base_sel = 0, base_tie = 0;
#pragma unroll
  for (int j = 0; j < NPL; ++j) {
    const bool live = kr > 0 && 64 * j + lane < C;
    const uint64_t mt = __ballot(live && key[j] == Tk);
    const int tie_rank = base_tie + (int)__popcll(mt & lt);
    const bool sel = live && (key[j] > Tk || (((mt >> lane) & 1ull) && tie_rank < need));
    const uint64_t ms = __ballot(sel);
    if (sel) out[base_sel + (int)__popcll(ms & lt)] = 64 * j + lane;
    base_sel += (int)__popcll(ms);
    base_tie += (int)__popcll(mt);
  }
  for (int e = base_sel + lane; e < kmax; e += 64) out[e] = -1;
  if (lane == 0) *cnt_out = base_sel;
}

template <typename T, int NPL>
__global__ __launch_bounds__(64) void k_centroid_topk_wave(const T* __restrict__ q, const float* __restrict__ cent,
                                                           int hq, int hkv, int C, int D, float scale, int k, int kmax,
                                                           int32_t* __restrict__ idx, int32_t* __restrict__ cnt,
                                                           int32_t* err) {
  __shared__ float qs[128];
  const int lane = threadIdx.x;
  // block -> (KV head innermost, so each XCD reads one KV head's centroid table)
  const int grp = hq / hkv;
  const int g = blockIdx.x % hkv, rest = blockIdx.x / hkv;
  const int t = rest / grp, h = g * grp + rest % grp;
  const int64_t row = (int64_t)t * hq + h;
  const float* cbase = cent + (int64_t)g * C * D;
  constexpr int U = NPL <= 4 ? 8 : NPL <= 8 ? 4 : 2;  // 16-byte loads per centroid per chunk: 32 in flight
  f32x4 mA[NPL][U], mB[NPL][U];
  auto load_chunk = [&](int d0, f32x4 (&dst)[NPL][U]) {
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      const int c = min(64 * j + lane, C - 1);
#pragma unroll
      for (int u = 0; u < U; ++u)
        dst[j][u] = d0 + 4 * u < D ? *reinterpret_cast<const f32x4*>(cbase + (int64_t)c * D + d0 + 4 * u) : f32x4{};
    }
  };
  float acc[NPL];
#pragma unroll
  for (int j = 0; j < NPL; ++j) acc[j] = 0.f;
  auto fma_chunk = [&](int d0, const f32x4 (&m)[NPL][U]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (d0 + 4 * u >= D) break;
#pragma unroll
      for (int j = 0; j < NPL; ++j) {
        acc[j] = fmaf(qs[d0 + 4 * u], m[j][u][0], acc[j]);
        acc[j] = fmaf(qs[d0 + 4 * u + 1], m[j][u][1], acc[j]);
        acc[j] = fmaf(qs[d0 + 4 * u + 2], m[j][u][2], acc[j]);
        acc[j] = fmaf(qs[d0 + 4 * u + 3], m[j][u][3], acc[j]);
      }
    }
  };
  // the first chunk's centroid loads go out before the query's, so the two
  // memory latencies overlap; afterwards the next chunk is in flight while
  // the current one is multiplied (dimension order is kept)
  constexpr int CH = 4 * U;  // dimensions per chunk
  load_chunk(0, mA);
  for (int d = lane; d < D; d += 64) {
    const T* qp = q + row * D + d;
    if constexpr (sizeof(T) == 2) qs[d] = bf2f(*reinterpret_cast<const uint16_t*>(qp));
    else qs[d] = *reinterpret_cast<const float*>(qp);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  for (int d0 = 0; d0 < D; d0 += 2 * CH) {
    if (d0 + CH < D) load_chunk(d0 + CH, mB);
    fma_chunk(d0, mA);
    if (d0 + CH >= D) break;
    if (d0 + 2 * CH < D) load_chunk(d0 + 2 * CH, mA);
    fma_chunk(d0 + CH, mB);
  }
  wave_topk_emit<NPL>(acc, C, scale, k, kmax, idx + row * kmax, cnt + row, err, lane);
}

}  // namespace

hipError_t launch_centroid_topk(const void* q, bool q_bf16, const float* cent, int T, int hq, int hkv, int C,
                                int head_dim, float scale, int k, int kmax, float mass, int k_min, int32_t* idx,
                                int32_t* cnt, int32_t* err, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  if (!(mass > 0.f)) {
    // fixed budget: one wave per (token, query head)
    const dim3 gw((unsigned)(T * hq));
#define SA_CTW_LAUNCH(TQ, NPL)                                                                                        \
  hipLaunchKernelGGL((k_centroid_topk_wave<TQ, NPL>), gw, dim3(64), 0, stream, (const TQ*)q, cent, hq, hkv, C, head_dim, \
                     scale, k, kmax, idx, cnt, err)
    if (q_bf16) {
      if (C <= 256) SA_CTW_LAUNCH(uint16_t, 4);
      else if (C <= 512) SA_CTW_LAUNCH(uint16_t, 8);
      else SA_CTW_LAUNCH(uint16_t, 16);
    } else {
      if (C <= 256) SA_CTW_LAUNCH(float, 4);
      else if (C <= 512) SA_CTW_LAUNCH(float, 8);
      else SA_CTW_LAUNCH(float, 16);
    }
#undef SA_CTW_LAUNCH
    return hipGetLastError();
  }
  // adaptive budget: one workgroup per (token, query head)
  const dim3 grid((unsigned)(T * hq));
  if (q_bf16)
    hipLaunchKernelGGL((k_centroid_topk<uint16_t>), grid, dim3(kCtThreads), 0, stream, (const uint16_t*)q, cent, hq, hkv,
                       C, head_dim, scale, k, kmax, mass, k_min, idx, cnt, err);
  else
    hipLaunchKernelGGL((k_centroid_topk<float>), grid, dim3(kCtThreads), 0, stream, (const float*)q, cent, hq, hkv, C,
                       head_dim, scale, k, kmax, mass, k_min, idx, cnt, err);
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
                              int nb, int head_dim, float scale, float* scores, int32_t* err, hipStream_t stream) {
  const int64_t rows = (int64_t)batch * (hl.n > 0 ? hl.n : hq);
  if (head_dim == 128 || head_dim == 64) {
    const int64_t nbt = (nb + 63) / 64;
    const int64_t waves = rows * (nbt * (nbt + 1) / 2);  // 64x64 tiles at or below the diagonal
    if (waves == 0) return hipSuccess;
    const dim3 grid((unsigned)((waves + 3) / 4));
    if (head_dim == 128)
      hipLaunchKernelGGL((k_block_score_direct<128>), grid, dim3(256), 0, stream, pq, pk, hq, hkv, hl, rows, nb, scale,
                         scores, err);
    else
      hipLaunchKernelGGL((k_block_score_direct<64>), grid, dim3(256), 0, stream, pq, pk, hq, hkv, hl, rows, nb, scale,
                         scores, err);
    return hipGetLastError();
  }
  return hipErrorInvalidValue;
}

hipError_t launch_centroid_score(const void* q, bool q_bf16, const float* cent, int T, int hq, int hkv,
                                 int C, int head_dim, float scale, float* out, int32_t* err, hipStream_t stream) {
  const int grp = hq / hkv;
  const size_t lds = (size_t)(kCentChunk + T * grp) * (head_dim + 1) * sizeof(float);
  if (lds > 160 * 1024) return hipErrorInvalidValue;
  const int nchunk = (C + kCentChunk - 1) / kCentChunk;
  const dim3 grid(hkv * nchunk);
  if (q_bf16)
    hipLaunchKernelGGL((k_centroid_score<uint16_t>), grid, dim3(256), lds, stream, (const uint16_t*)q, cent, T,
                       hq, hkv, C, head_dim, scale, out, err);
  else
    hipLaunchKernelGGL((k_centroid_score<float>), grid, dim3(256), lds, stream, (const float*)q, cent, T, hq,
                       hkv, C, head_dim, scale, out, err);
  return hipGetLastError();
}

}  // namespace sa
