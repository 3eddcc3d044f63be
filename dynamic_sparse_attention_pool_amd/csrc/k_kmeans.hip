// Offline clustering of the fixed context's keys: Lloyd iterations per KV head.
//
// Squeezed Attention page, §技术方案, offline stage: the context's keys are
// clustered, every cluster gets a centroid and every key an index to its
// cluster.  One iteration = assignment (nearest centroid by squared distance,
// ties to the lower cluster index) + update (each centroid becomes the mean of
// its keys; an empty cluster keeps its centroid).
//
// Assignment of fp32 keys: one thread per key with the key row in registers;
// centroids pass through LDS 32 at a time together with their squared norms,
// and the thread keeps the smallest |mu|^2 - 2 x.mu (the |x|^2 term is the same
// for every centroid of a key).  Dot products run in dimension order in fp32.
// Assignment of bf16 keys on the matrix cores: every centroid is split into
// three bf16 parts (hi = bf16(mu), lo = bf16(mu - hi), lo2 = bf16(mu - hi -
// lo); their sum is mu to about 2^-24 relative), so x.mu = x.hi + x.lo + x.lo2
// with exact bf16 products accumulated in fp32 by v_mfma_f32_32x32x16_bf16.
// Update: the cluster-major order of the labels (the stable counting sort of
// the cluster pack) gives each cluster's keys in token order; one workgroup
// per (KV head, cluster) sums them in that order, one thread per dimension,
// so the centroids are deterministic without atomics.
#include <algorithm>

#include "common.h"
#include "launch.h"

namespace sa {
namespace {

constexpr int kKmKeys = 256;   // keys (threads) per assignment workgroup
size_t km_a256(size_t x) { return (x + 255) & ~size_t(255); }
constexpr int kKmChunk = 32;   // centroids staged per pass

template <typename T, int D>
__device__ __forceinline__ void load_row(const T* src, float* x) {
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int c = 0; c < D / 8; ++c) {
      const u32x4 v = ldg16(src + 8 * c);
#pragma unroll
      for (int e = 0; e < 8; ++e) x[8 * c + e] = bf2f((uint16_t)((v[e >> 1] >> ((e & 1) * 16)) & 0xffffu));
    }
  } else {
#pragma unroll
    for (int c = 0; c < D / 4; ++c) {
      const u32x4 v = ldg16(src + 4 * c);
#pragma unroll
      for (int e = 0; e < 4; ++e) x[4 * c + e] = __uint_as_float(v[e]);
    }
  }
}

template <typename T, int D>
__global__ __launch_bounds__(kKmKeys) void k_km_assign(const T* __restrict__ keys, const float* __restrict__ cent,
                                                       int64_t n, int C, int32_t* __restrict__ labels) {
  __shared__ __attribute__((aligned(16))) float mu[kKmChunk][D];
  __shared__ float nrm[kKmChunk];
  const int tid = threadIdx.x;
  const int64_t nblk = (n + kKmKeys - 1) / kKmKeys;
  const int g = (int)(blockIdx.x / nblk);
  const int64_t t = (blockIdx.x % nblk) * kKmKeys + tid;
  const bool live = t < n;
  float x[D];
  if (live) {
    load_row<T, D>(keys + ((int64_t)g * n + t) * D, x);
  } else {
#pragma unroll
    for (int d = 0; d < D; ++d) x[d] = 0.f;
  }
  const float* cg = cent + (int64_t)g * C * D;
  float best = INFINITY;
  int arg = 0;
  for (int c0 = 0; c0 < C; c0 += kKmChunk) {
    const int nc = min(kKmChunk, C - c0);
    __syncthreads();
    for (int e = tid; e < nc * (D / 4); e += kKmKeys) {
      const int c = e / (D / 4), q = e % (D / 4);
      *reinterpret_cast<f32x4*>(&mu[c][4 * q]) = *reinterpret_cast<const f32x4*>(cg + (int64_t)(c0 + c) * D + 4 * q);
    }
    __syncthreads();
    if (tid < nc) {
      float s = 0.f;
      for (int d = 0; d < D; ++d) s = fmaf(mu[tid][d], mu[tid][d], s);
      nrm[tid] = s;
    }
    __syncthreads();
    for (int c = 0; c < nc; ++c) {
      float dot = 0.f;
#pragma unroll
      for (int q = 0; q < D / 4; ++q) {
        const f32x4 m4 = *reinterpret_cast<const f32x4*>(&mu[c][4 * q]);
        dot = fmaf(x[4 * q], m4[0], dot);
        dot = fmaf(x[4 * q + 1], m4[1], dot);
        dot = fmaf(x[4 * q + 2], m4[2], dot);
        dot = fmaf(x[4 * q + 3], m4[3], dot);
      }
      const float dist = fmaf(-2.f, dot, nrm[c]);
      if (dist < best) {  // strict: the lower index keeps a tie
        best = dist;
        arg = c0 + c;
      }
    }
  }
  if (live) labels[(int64_t)g * n + t] = arg;
}

// Centroid split for the matrix-core assignment: parts [g][c][3][D] bf16 and
// the squared norm (fp32, dimension order) of every centroid.
template <int D>
__global__ __launch_bounds__(D) void k_km_split(const float* __restrict__ cent, int C, uint16_t* __restrict__ parts,
                                               float* __restrict__ nrm) {
  __shared__ float sq[D];
  const int gc = blockIdx.x, d = threadIdx.x;
  const float m = cent[(int64_t)gc * D + d];
  const uint32_t hi = f2bf(m);
  const float r1 = m - bf2f((uint16_t)hi);
  const uint32_t lo = f2bf(r1);
  const uint32_t lo2 = f2bf(r1 - bf2f((uint16_t)lo));
  uint16_t* pr = parts + (int64_t)gc * 3 * D;
  pr[d] = (uint16_t)hi;
  pr[D + d] = (uint16_t)lo;
  pr[2 * D + d] = (uint16_t)lo2;
  sq[d] = m;
  __syncthreads();
  if (d == 0) {
    float s = 0.f;
    for (int e = 0; e < D; ++e) s = fmaf(sq[e], sq[e], s);
    nrm[gc] = s;
  }
}

// C x key tiles of |mu|^2 - 2 (mu . x): wave = 64 keys (two operand tiles held
// in registers), workgroup = 4 waves.  For each tile of 32 centroids the three
// parts' rows (A operand, read from the L2-resident split table) multiply the
// keys (B operand); lane (l32, hf) then holds key 32kt + l32 and the 16
// centroids 32ct + 8(r/4) + 4hf + r%4, ascending in r, so a strict compare in
// that order keeps the lowest index among equal distances; the two lane halves
// are merged by one exchange with the same rule.
constexpr int kKmWaves = 4;
constexpr int kKmKeysPerWave = 64;

template <int D>
__global__ __launch_bounds__(64 * kKmWaves) void k_km_assign_mfma(const uint16_t* __restrict__ keys,
                                                                 const uint16_t* __restrict__ parts,
                                                                 const float* __restrict__ nrm, int64_t n, int C,
                                                                 int32_t* __restrict__ labels) {
  constexpr int NS = D / 16;
  constexpr int RS = 3 * D + 8;            // LDS row of one centroid's three parts, padded by 16 bytes
  constexpr int CPR = 3 * D / 8;           // 16-byte chunks per centroid row
  constexpr int CPT = 32 * CPR;            // per tile of 32 centroids
  constexpr int NT = 64 * kKmWaves;
  constexpr int PER = (CPT + NT - 1) / NT;
  __shared__ __attribute__((aligned(16))) uint16_t cs[2][32 * RS];
  __shared__ float cn[2][32];
  const int tid = threadIdx.x;
  const int lane = tid & 63, hf = lane >> 5, l32 = lane & 31, wv = tid >> 6;
  constexpr int kPerWg = kKmWaves * kKmKeysPerWave;
  const int64_t nblk = (n + kPerWg - 1) / kPerWg;
  const int g = (int)(blockIdx.x / nblk);
  const int64_t k0 = (blockIdx.x % nblk) * kPerWg + (int64_t)wv * kKmKeysPerWave;
  const uint16_t* kg = keys + (int64_t)g * n * D;
  bf16x8 xb[2][NS];
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    const int64_t row = std::min(k0 + 32 * kt + l32, n - 1);
#pragma unroll
    for (int s4 = 0; s4 < NS; ++s4) xb[kt][s4] = as_bf16x8(ldg16(kg + row * D + 16 * s4 + 8 * hf));
  }
  const uint16_t* pg = parts + (int64_t)g * C * 3 * D;
  const float* ng = nrm + (int64_t)g * C;
  // one tile of 32 centroids (three bf16 parts each, and the squared norms)
  // goes global -> registers -> LDS, shared by the workgroup's four waves
  u32x4 rg[PER];
  float rn = 0.f;
  auto fetch = [&](int ct) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int q = tid + u * NT;
      if (q < CPT) {
        const int crow = std::min(32 * ct + q / CPR, C - 1);
        rg[u] = ldg16(pg + (int64_t)crow * 3 * D + 8 * (q % CPR));
      }
    }
    if (tid < 32) rn = ng[std::min(32 * ct + tid, C - 1)];
  };
  auto put = [&](int buf) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int q = tid + u * NT;
      if (q < CPT) *reinterpret_cast<u32x4*>(&cs[buf][(q / CPR) * RS + 8 * (q % CPR)]) = rg[u];
    }
    if (tid < 32) cn[buf][tid] = rn;
  };
  float best[2] = {INFINITY, INFINITY};
  int arg[2] = {0, 0};
  const int nct = (C + 31) / 32;
  fetch(0);
  put(0);
  __syncthreads();
  for (int ct = 0; ct < nct; ++ct) {
    const int buf = ct & 1;
    const bool nx = ct + 1 < nct;
    if (nx) fetch(ct + 1);  // in flight during this tile's products
    const uint16_t* cr = &cs[buf][l32 * RS + 8 * hf];
    f32x16 acc[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int part = 0; part < 3; ++part) {
      bf16x8 a[NS];
#pragma unroll
      for (int s4 = 0; s4 < NS; ++s4) a[s4] = as_bf16x8(*reinterpret_cast<const u32x4*>(cr + part * D + 16 * s4));
#pragma unroll
      for (int s4 = 0; s4 < NS; ++s4)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) acc[kt] = mfma32x32x16(a[s4], xb[kt][s4], acc[kt]);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int cl = 8 * (r / 4) + 4 * hf + (r % 4);
      const int c = 32 * ct + cl;
      const float nr = cn[buf][cl];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const float dist = fmaf(-2.f, acc[kt][r], nr);
        if (c < C && dist < best[kt]) {
          best[kt] = dist;
          arg[kt] = c;
        }
      }
    }
    if (nx) put(buf ^ 1);
    __syncthreads();  // the next tile is in LDS; this one is no longer read
  }
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    const float ob = __shfl_xor(best[kt], 32);
    const int oa = __shfl_xor(arg[kt], 32);
    if (ob < best[kt] || (ob == best[kt] && oa < arg[kt])) arg[kt] = oa;
    const int64_t key = k0 + 32 * kt + l32;
    if (hf == 0 && key < n) labels[(int64_t)g * n + key] = arg[kt];
  }
}

// One workgroup per (KV head, cluster), one thread per dimension.  The
// cluster's row ids are staged in LDS (2048 at a time), then each thread sums
// its dimension over the rows in token order with 32 rows' loads in flight, so
// the largest cluster costs one memory latency per 32 rows.
constexpr int kKmStage = 2048;
constexpr int kKmInFlight = 32;

template <typename T, int D>
__global__ __launch_bounds__(D) __attribute__((amdgpu_waves_per_eu(1, 4))) void k_km_update(const T* __restrict__ keys, const int32_t* __restrict__ ptr,
                                                 const int32_t* __restrict__ perm, int64_t n, int C,
                                                 float* __restrict__ cent) {
  __shared__ int32_t rs[kKmStage];
  const int g = blockIdx.x / C, c = blockIdx.x % C, d = threadIdx.x;
  const int32_t b = ptr[(int64_t)g * (C + 1) + c], e = ptr[(int64_t)g * (C + 1) + c + 1];
  if (e <= b) return;  // empty cluster: the centroid stays (the whole workgroup leaves)
  const T* kg = keys + (int64_t)g * n * D + d;
  const int32_t* pg = perm + (int64_t)g * n;
  auto val = [&](int32_t row) -> float {
    if constexpr (sizeof(T) == 2) return bf2f(kg[(int64_t)row * D]);
    else return kg[(int64_t)row * D];
  };
  float s = 0.f;
  for (int32_t cb = b; cb < e; cb += kKmStage) {
    const int nn = min(kKmStage, e - cb);
    __syncthreads();  // the previous chunk's ids are consumed
    for (int i = d; i < nn; i += D) rs[i] = pg[cb + i];
    __syncthreads();
    int r = 0;
    for (; r + kKmInFlight <= nn; r += kKmInFlight) {
      float v[kKmInFlight];
#pragma unroll
      for (int x = 0; x < kKmInFlight; ++x) v[x] = val(rs[r + x]);
#pragma unroll
      for (int x = 0; x < kKmInFlight; ++x) s += v[x];
    }
    for (; r < nn; ++r) s += val(rs[r]);
  }
  cent[((int64_t)g * C + c) * D + d] = s / (float)(e - b);
}

}  // namespace

// pack workspace, then (bf16 keys) the centroid parts and squared norms
size_t kmeans_workspace_bytes(int64_t hkv, int64_t n, int C, int head_dim) {
  return km_a256(cluster_pack_workspace_bytes(hkv, n, C)) + km_a256((size_t)(hkv * C) * 3 * head_dim * 2) +
         km_a256((size_t)(hkv * C) * 4);
}

hipError_t launch_kmeans(const void* keys, bool bf16, int64_t hkv, int64_t n, int head_dim, int C, int iters,
                         float* cent, int32_t* labels, int32_t* ptr, int32_t* perm, void* ws, hipStream_t stream) {
  if (hkv == 0 || n == 0) return hipSuccess;
  const dim3 ga((unsigned)(hkv * ((n + kKmKeys - 1) / kKmKeys)));
  const dim3 gm((unsigned)(hkv * ((n + kKmWaves * kKmKeysPerWave - 1) / (kKmWaves * kKmKeysPerWave))));
  const dim3 gu((unsigned)(hkv * C));
  char* wsb = static_cast<char*>(ws);
  void* pack_ws = wsb;
  uint16_t* parts = reinterpret_cast<uint16_t*>(wsb + km_a256(cluster_pack_workspace_bytes(hkv, n, C)));
  float* nrm = reinterpret_cast<float*>(reinterpret_cast<char*>(parts) + km_a256((size_t)(hkv * C) * 3 * head_dim * 2));
  for (int it = 0; it < iters; ++it) {
#define SA_KM_ASSIGN_F32(D_) \
  hipLaunchKernelGGL((k_km_assign<float, D_>), ga, dim3(kKmKeys), 0, stream, (const float*)keys, cent, n, C, labels);
#define SA_KM_ASSIGN_BF16(D_)                                                                                     \
  hipLaunchKernelGGL((k_km_split<D_>), dim3((unsigned)(hkv * C)), dim3(D_), 0, stream, cent, C, parts, nrm);     \
  hipLaunchKernelGGL((k_km_assign_mfma<D_>), gm, dim3(64 * kKmWaves), 0, stream, (const uint16_t*)keys, parts, nrm, \
                     n, C, labels);
#define SA_KM_STEP(T_, D_, ASSIGN)                                                                                \
  ASSIGN                                                                                                          \
  {                                                                                                               \
    const hipError_t e = launch_cluster_pack(labels, hkv, n, C, ptr, perm, nullptr, nullptr, nullptr, nullptr,   \
                                             head_dim, 0, nullptr, pack_ws, stream);                              \
    if (e != hipSuccess) return e;                                                                                \
  }                                                                                                               \
  hipLaunchKernelGGL((k_km_update<T_, D_>), gu, dim3(D_), 0, stream, (const T_*)keys, ptr, perm, n, C, cent);
    if (bf16 && head_dim == 128) {
      SA_KM_STEP(uint16_t, 128, SA_KM_ASSIGN_BF16(128))
    } else if (bf16 && head_dim == 64) {
      SA_KM_STEP(uint16_t, 64, SA_KM_ASSIGN_BF16(64))
    } else if (!bf16 && head_dim == 128) {
      SA_KM_STEP(float, 128, SA_KM_ASSIGN_F32(128))
    } else if (!bf16 && head_dim == 64) {
      SA_KM_STEP(float, 64, SA_KM_ASSIGN_F32(64))
    } else {
      return hipErrorInvalidValue;
    }
#undef SA_KM_STEP
#undef SA_KM_ASSIGN_F32
#undef SA_KM_ASSIGN_BF16
  }
  return hipGetLastError();
}

}  // namespace sa
