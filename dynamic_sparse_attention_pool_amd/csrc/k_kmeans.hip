// Offline clustering of the fixed context's keys: Lloyd iterations per KV head.
//
// Squeezed Attention page, §技术方案, offline stage: the context's keys are
// clustered, every cluster gets a centroid and every key an index to its
// cluster.  One iteration = assignment (nearest centroid by squared distance,
// ties to the lower cluster index) + update (each centroid becomes the mean of
// its keys; an empty cluster keeps its centroid).
//
// Assignment: one thread per key with the key row in registers; centroids pass
// through LDS 32 at a time together with their squared norms, and the thread
// keeps the smallest |mu|^2 - 2 x.mu (the |x|^2 term is the same for every
// centroid of a key).  Dot products run in dimension order in fp32.
// Update: the cluster-major order of the labels (the stable counting sort of
// the cluster pack) gives each cluster's keys in token order; one workgroup
// per (KV head, cluster) sums them in that order, one thread per dimension,
// so the centroids are deterministic without atomics.
#include "common.h"
#include "launch.h"

namespace sa {
namespace {

constexpr int kKmKeys = 256;   // keys (threads) per assignment workgroup
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

// One workgroup per (KV head, cluster), one thread per dimension.
template <typename T, int D>
__global__ __launch_bounds__(D) void k_km_update(const T* __restrict__ keys, const int32_t* __restrict__ ptr,
                                                 const int32_t* __restrict__ perm, int64_t n, int C,
                                                 float* __restrict__ cent) {
  const int g = blockIdx.x / C, c = blockIdx.x % C, d = threadIdx.x;
  const int32_t b = ptr[(int64_t)g * (C + 1) + c], e = ptr[(int64_t)g * (C + 1) + c + 1];
  if (e <= b) return;  // empty cluster: the centroid stays
  const T* kg = keys + (int64_t)g * n * D;
  const int32_t* pg = perm + (int64_t)g * n;
  auto val = [&](int64_t row) -> float {
    if constexpr (sizeof(T) == 2) return bf2f(kg[row * D + d]);
    else return kg[row * D + d];
  };
  // 8 rows' loads in flight at a time; the sum still runs in token order
  float s = 0.f;
  int32_t r = b;
  for (; r + 8 <= e; r += 8) {
    int64_t rows[8];
#pragma unroll
    for (int x = 0; x < 8; ++x) rows[x] = pg[r + x];
    float v[8];
#pragma unroll
    for (int x = 0; x < 8; ++x) v[x] = val(rows[x]);
#pragma unroll
    for (int x = 0; x < 8; ++x) s += v[x];
  }
  for (; r < e; ++r) s += val(pg[r]);
  cent[((int64_t)g * C + c) * D + d] = s / (float)(e - b);
}

}  // namespace

size_t kmeans_workspace_bytes(int64_t hkv, int64_t n, int C) {
  return cluster_pack_workspace_bytes(hkv, n, C);
}

hipError_t launch_kmeans(const void* keys, bool bf16, int64_t hkv, int64_t n, int head_dim, int C, int iters,
                         float* cent, int32_t* labels, int32_t* ptr, int32_t* perm, void* ws, hipStream_t stream) {
  if (hkv == 0 || n == 0) return hipSuccess;
  const dim3 ga((unsigned)(hkv * ((n + kKmKeys - 1) / kKmKeys)));
  const dim3 gu((unsigned)(hkv * C));
  for (int it = 0; it < iters; ++it) {
#define SA_KM_STEP(T_, D_)                                                                                        \
  hipLaunchKernelGGL((k_km_assign<T_, D_>), ga, dim3(kKmKeys), 0, stream, (const T_*)keys, cent, n, C, labels); \
  {                                                                                                               \
    const hipError_t e = launch_cluster_pack(labels, hkv, n, C, ptr, perm, nullptr, nullptr, nullptr, nullptr,   \
                                             head_dim, 0, nullptr, ws, stream);                                   \
    if (e != hipSuccess) return e;                                                                                \
  }                                                                                                               \
  hipLaunchKernelGGL((k_km_update<T_, D_>), gu, dim3(D_), 0, stream, (const T_*)keys, ptr, perm, n, C, cent);
    if (bf16 && head_dim == 128) {
      SA_KM_STEP(uint16_t, 128)
    } else if (bf16 && head_dim == 64) {
      SA_KM_STEP(uint16_t, 64)
    } else if (!bf16 && head_dim == 128) {
      SA_KM_STEP(float, 128)
    } else if (!bf16 && head_dim == 64) {
      SA_KM_STEP(float, 64)
    } else {
      return hipErrorInvalidValue;
    }
#undef SA_KM_STEP
  }
  return hipGetLastError();
}

}  // namespace sa
