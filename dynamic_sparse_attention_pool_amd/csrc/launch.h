// Internal interface between the C-ABI layer (sa_api.cpp) and the kernels.
// Every launcher enqueues on `stream` and returns hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sa {

// Query heads covered by one launch.  n == 0: every head, in order.  n > 0:
// the launch covers (b, h[j]) for j < n; q, k, v, out and lse keep their full
// [B, Hq, ...] layout, while per-row scores and tables of the launch are
// indexed compactly by b*n + j.  Passed by value in the kernel arguments.
constexpr int kMaxListedHeads = 256;
struct HeadList {
  int32_t n;
  int16_t h[kMaxListedHeads];
};

// Compact row bh -> (batch, query head).
__host__ __device__ inline void listed_row(int64_t bh, int hq, const HeadList& hl, int& b, int& h) {
  if (hl.n > 0) {
    b = (int)(bh / hl.n);
    h = hl.h[bh % hl.n];
  } else {
    b = (int)(bh / hq);
    h = (int)(bh % hq);
  }
}

// ---------------------------------------------------------------- forward
struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* lse;
  const int32_t* block_idx;
  const int32_t* block_cnt;
  const int32_t* iv;
  const int32_t* iv_cnt;
  const int32_t* col;
  const int32_t* col_cnt;
  int64_t seq;
  int32_t batch, heads_q, heads_kv, nqb;
  int32_t kmax, max_iv, max_col;
  float scale;
  int32_t order;  // workgroup order of the bf16 kernel, chosen by launch_fwd
  int32_t ashape, n_sink, n_local;  // block lists generated: blocks 0..n_sink-1 and the n_local up to the diagonal
  HeadList hl;
};
hipError_t launch_fwd(const FwdParams& p, int head_dim, int mode, bool in_bf16, bool out_bf16,
                      hipStream_t stream);

// ---------------------------------------------------------------- estimate
// rows of x: batch*hq rows of seq tokens; with a head list, the listed rows only
// (out compact).
hipError_t launch_pool(const void* x, int64_t batch, int hq, const HeadList& hl, int64_t seq, int head_dim,
                       bool bf16, int block, float* out, hipStream_t stream);
// Estimators: err (optional device int32) gets bit 0 when a score they write
// (outside the masked entries) is NaN or infinite.
hipError_t launch_block_score(const float* pq, const float* pk, int batch, int hq, int hkv, const HeadList& hl,
                              int nb, int head_dim, float scale, float* scores, int32_t* err, hipStream_t stream);
hipError_t launch_centroid_score(const void* q, bool q_bf16, const float* cent, int T, int hq, int hkv,
                                 int C, int head_dim, float scale, float* out, int32_t* err, hipStream_t stream);
// centroid scores and a per-row top-k in one pass (query heads per KV head <= 8,
// clusters <= 1024, head_dim <= 128)
hipError_t launch_centroid_topk(const void* q, bool q_bf16, const float* cent, int T, int hq, int hkv, int C,
                                int head_dim, float scale, int k, int kmax, float mass, int k_min, int32_t* idx,
                                int32_t* cnt, int32_t* err, hipStream_t stream);
hipError_t launch_indexer(const uint16_t* q, const uint16_t* k, const float* w, int T, int hi, int64_t nk,
                          int64_t pos0, float* out, int32_t* err, hipStream_t stream);
// Candidate slots of chunk c (keys c*chunk ..) of an indexer row with n causal
// keys when `expect` kept keys are expected over the row: twice the chunk's
// share plus 64, rounded up to a multiple of 64, at most the chunk's keys.
// Every chunk of a row but the last is full, so chunk c's run starts at
// c * idx_slots(n, 0, ...).  32-bit arithmetic: n < 2^31, chunk <= 8192 and
// expect <= 4096 keep 2 * expect * len + n below 2^32.
__host__ __device__ inline int64_t idx_slots(int64_t n, int64_t c, int64_t chunk, int64_t expect) {
  const uint32_t nn = (uint32_t)n;
  const uint32_t len = (uint32_t)(n - c * chunk < chunk ? n - c * chunk : chunk);
  const uint32_t share = (2u * (uint32_t)expect * len + nn - 1u) / nn;
  const uint32_t s = (share + 63u) / 64u * 64u + 64u;
  return s < len ? s : len;
}
size_t indexer_topk_workspace_bytes(int T, int64_t nk, int64_t pos0, int k);
hipError_t launch_indexer_topk(const uint16_t* q, const uint16_t* k, const float* w, int T, int hi, int64_t nk,
                               int64_t pos0, int kk, int kmax, int32_t* idx, int32_t* cnt, int32_t* err, void* ws,
                               hipStream_t stream);
size_t vs_workspace_bytes(int64_t rows, int64_t seq);
hipError_t launch_vs_estimate(const uint16_t* q, const uint16_t* k, int batch, int hq, int hkv,
                              const HeadList& hl, int64_t seq, int head_dim, int last_q, float scale, float* a_v,
                              float* a_s, int32_t* err, void* ws, hipStream_t stream);

// pooled block scores and per-row top-k in one pass (at most 2048 blocks per row)
constexpr int kBlockTopkMaxBlocks = 2048;
struct BlockTopkParams {
  const float* pq;  // pooled queries, rows compact as in the head list
  const float* pk;  // pooled keys [B*Hkv, nb, d]
  int32_t* idx;
  int32_t* cnt;
  int32_t* err;
  int32_t batch, hq, hkv, nb, kmax;
  int32_t n_sink, n_local, k, rnum, rden;
  float scale;
  HeadList hl;
};
hipError_t launch_block_topk(const BlockTopkParams& p, int head_dim, hipStream_t stream);

// ---------------------------------------------------------------- select
struct SelectParams {
  const float* scores;
  int64_t rows, ncand, ld, period, offset;
  int32_t causal, n_sink, n_local, k, rnum, rden, kmax;
  int32_t* idx;
  int32_t* cnt;
  int32_t* err;
};
hipError_t launch_select(const SelectParams& p, hipStream_t stream);

constexpr int kMassMax = 4096;  // candidates per row of the adaptive selection
struct MassParams {
  const float* scores;
  int64_t rows, ncand, ld;
  float mass;
  int32_t k_min, k_max, kmax;
  int32_t* idx;
  int32_t* cnt;
  int32_t* err;
};
hipError_t launch_select_mass(const MassParams& p, hipStream_t stream);

struct VsBuildParams {
  int64_t rows, seq;
  int32_t bs, n_vert, n_slash;
  const int32_t* vert;
  const int32_t* vert_cnt;
  const int32_t* slash;
  const int32_t* slash_cnt;
  int32_t* iv;
  int32_t* iv_cnt;
  int32_t* col;
  int32_t* col_cnt;
};
hipError_t launch_vs_build(const VsBuildParams& p, hipStream_t stream);

// ---------------------------------------------------------------- decode / gather
struct GatherParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* cluster_ptr;
  const int32_t* sel;
  const int32_t* tok_idx;
  const int32_t* q_pos;  // optional [T]: query t sees context positions <= q_pos[t]
  const int32_t* perm;   // cluster mode with q_pos: context position of each packed row [hkv, n_ctx]
  void* out;
  float* lse;
  int64_t n_ctx;
  int32_t T, hq, hkv, C, n_sel, n_tok;
  int32_t tok_per_head;  // token mode: lists [T, hq, n_tok] instead of [T, n_tok]
  float scale;
  bool out_bf16;
};
size_t cluster_decode_workspace_bytes(int T, int hq, int hkv, int C, int64_t n_ctx);
hipError_t launch_cluster_decode(const GatherParams& p, void* ws, hipStream_t stream);
size_t token_gather_workspace_bytes(int T, int hq, int n_tok);
hipError_t launch_token_gather(const GatherParams& p, void* ws, hipStream_t stream);

size_t cluster_pack_workspace_bytes(int64_t hkv, int64_t n, int C);
hipError_t launch_cluster_pack(const int32_t* labels, int64_t hkv, int64_t n, int C, int32_t* ptr,
                               int32_t* perm, const void* k, const void* v, void* kp, void* vp,
                               int head_dim, int elem_bytes, int32_t* err, void* ws, hipStream_t stream);

// ---------------------------------------------------------------- offline k-means
size_t kmeans_workspace_bytes(int64_t hkv, int64_t n, int C, int head_dim);
hipError_t launch_kmeans(const void* keys, bool bf16, int64_t hkv, int64_t n, int head_dim, int C, int iters,
                         float* cent, int32_t* labels, int32_t* ptr, int32_t* perm, void* ws, hipStream_t stream);

}  // namespace sa
