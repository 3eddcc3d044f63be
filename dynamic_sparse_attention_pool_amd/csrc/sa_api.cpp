// C-ABI layer of libsa: argument validation, workspace sizing and dispatch.
// Every check runs on the host before any launch; see include/sa.h for the
// contract of each entry point.
#include "sa.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "launch.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return SA_OK;
}

int launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(SA_ERR_LAUNCH, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
  return ok();
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Also clears any error an earlier, unrelated runtime call left behind, so that
// the launchers' hipGetLastError() reports only this call's launches.
hipStream_t as_stream(void* s) {
  (void)hipGetLastError();
  return reinterpret_cast<hipStream_t>(s);
}

constexpr int kBlock = 64;

// Host head list -> launch-argument form; rejects duplicates and heads outside
// [0, hq).  A NULL list means every head.
int make_head_list(const int32_t* list, int32_t n, int64_t hq, const char* who, sa::HeadList& hl) {
  hl.n = 0;
  if (!list) return ok();
  if (n <= 0 || n > sa::kMaxListedHeads || n > hq)
    return fail(SA_ERR_VALUE, "%s: n_heads_list must lie in [1, min(heads_q, %d)]", who, sa::kMaxListedHeads);
  bool seen[sa::kMaxListedHeads] = {};
  for (int j = 0; j < n; ++j) {
    const int32_t h = list[j];
    if (h < 0 || h >= hq || h >= sa::kMaxListedHeads) return fail(SA_ERR_VALUE, "%s: head_list[%d] = %d is not a query head", who, j, h);
    if (seen[h]) return fail(SA_ERR_VALUE, "%s: head %d listed twice", who, h);
    seen[h] = true;
    hl.h[j] = (int16_t)h;
  }
  hl.n = n;
  return ok();
}

// ---------------------------------------------------------------- estimate
int check_estimate(const sa_estimate_args* a, size_t* ws) {
  if (!a) return fail(SA_ERR_NULL, "sa_estimate: args is NULL");
  *ws = 0;
  if (!a->q || !a->k || !a->scores) return fail(SA_ERR_NULL, "sa_estimate: q, k and scores are required");
  if (a->heads_q <= 0 || a->heads_kv <= 0 || a->seq_q <= 0 || a->seq_k <= 0 || a->head_dim <= 0)
    return fail(SA_ERR_SHAPE, "sa_estimate: sizes must be positive");
  if (!aligned16(a->q) || !aligned16(a->k)) return fail(SA_ERR_ALIGN, "sa_estimate: q and k must be 16-byte aligned");
  switch (a->kind) {
    case SA_EST_BLOCK_MEANPOOL: {
      if (a->dtype != SA_F32 && a->dtype != SA_BF16) return fail(SA_ERR_DTYPE, "sa_estimate(BLOCK): dtype must be F32 or BF16");
      if (a->block_size != kBlock) return fail(SA_ERR_UNSUPPORTED, "sa_estimate(BLOCK): block_size must be 64");
      if (a->head_dim != 64 && a->head_dim != 128) return fail(SA_ERR_UNSUPPORTED, "sa_estimate(BLOCK): head_dim must be 64 or 128");
      if (a->batch <= 0) return fail(SA_ERR_SHAPE, "sa_estimate(BLOCK): batch must be positive");
      if (a->heads_q % a->heads_kv) return fail(SA_ERR_SHAPE, "sa_estimate(BLOCK): heads_q must be a multiple of heads_kv");
      if (a->seq_q != a->seq_k) return fail(SA_ERR_SHAPE, "sa_estimate(BLOCK): seq_q must equal seq_k (prefill)");
      if (a->seq_q % kBlock) return fail(SA_ERR_SHAPE, "sa_estimate(BLOCK): seq must be a multiple of 64");
      if (!(a->scale > 0.f)) return fail(SA_ERR_VALUE, "sa_estimate: scale must be > 0");
      sa::HeadList hl;
      if (const int rc = make_head_list(a->head_list, a->n_heads_list, a->heads_q, "sa_estimate(BLOCK)", hl)) return rc;
      const int64_t nb = a->seq_q / kBlock;
      const int64_t nh = hl.n > 0 ? hl.n : a->heads_q;
      if (!a->pooled_q) *ws += align256((size_t)(a->batch * nh * nb * a->head_dim) * 4);
      if (!a->pooled_k) *ws += align256((size_t)(a->batch * a->heads_kv * nb * a->head_dim) * 4);
      return ok();
    }
    case SA_EST_VSLASH: {
      if (a->dtype != SA_BF16) return fail(SA_ERR_DTYPE, "sa_estimate(VSLASH): dtype must be BF16");
      if (a->head_dim != 128 && a->head_dim != 64) return fail(SA_ERR_UNSUPPORTED, "sa_estimate(VSLASH): head_dim must be 64 or 128");
      if (a->last_q != 64) return fail(SA_ERR_UNSUPPORTED, "sa_estimate(VSLASH): last_q must be 64");
      if (a->batch <= 0) return fail(SA_ERR_SHAPE, "sa_estimate(VSLASH): batch must be positive");
      if (a->heads_q % a->heads_kv) return fail(SA_ERR_SHAPE, "sa_estimate(VSLASH): heads_q must be a multiple of heads_kv");
      if (a->seq_q != a->seq_k || a->seq_q % kBlock) return fail(SA_ERR_SHAPE, "sa_estimate(VSLASH): seq_q == seq_k, a multiple of 64");
      if (!a->scores2) return fail(SA_ERR_NULL, "sa_estimate(VSLASH): scores2 (slash scores) is required");
      if (!(a->scale > 0.f)) return fail(SA_ERR_VALUE, "sa_estimate: scale must be > 0");
      sa::HeadList hl;
      if (const int rc = make_head_list(a->head_list, a->n_heads_list, a->heads_q, "sa_estimate(VSLASH)", hl)) return rc;
      *ws = sa::vs_workspace_bytes(a->batch * (hl.n > 0 ? hl.n : a->heads_q), a->seq_q);
      return ok();
    }
    case SA_EST_CENTROID: {
      if (a->head_list) return fail(SA_ERR_UNSUPPORTED, "sa_estimate(CENTROID): no head list");
      if (a->dtype != SA_F32 && a->dtype != SA_BF16) return fail(SA_ERR_DTYPE, "sa_estimate(CENTROID): dtype must be F32 or BF16");
      if (!a->centroids) return fail(SA_ERR_NULL, "sa_estimate(CENTROID): centroids required");
      if (a->n_centroids <= 0) return fail(SA_ERR_SHAPE, "sa_estimate(CENTROID): n_centroids must be positive");
      if (a->heads_q % a->heads_kv) return fail(SA_ERR_SHAPE, "sa_estimate(CENTROID): heads_q must be a multiple of heads_kv");
      const int64_t nq = a->seq_q * (a->heads_q / a->heads_kv);
      if ((32 + nq) * (a->head_dim + 1) * 4 > 160 * 1024)
        return fail(SA_ERR_UNSUPPORTED, "sa_estimate(CENTROID): queries per KV head x head_dim too large for LDS");
      if (!(a->scale > 0.f)) return fail(SA_ERR_VALUE, "sa_estimate: scale must be > 0");
      return ok();
    }
    case SA_EST_INDEXER: {
      if (a->head_list) return fail(SA_ERR_UNSUPPORTED, "sa_estimate(INDEXER): no head list");
      if (a->dtype != SA_BF16) return fail(SA_ERR_DTYPE, "sa_estimate(INDEXER): dtype must be BF16");
      if (!a->weights) return fail(SA_ERR_NULL, "sa_estimate(INDEXER): weights required");
      if (a->head_dim != 64) return fail(SA_ERR_UNSUPPORTED, "sa_estimate(INDEXER): head_dim must be 64");
      if (a->heads_q % 8 || a->heads_q > 64)
        return fail(SA_ERR_UNSUPPORTED, "sa_estimate(INDEXER): indexer heads must be a multiple of 8, at most 64");
      if (a->heads_kv != 1) return fail(SA_ERR_SHAPE, "sa_estimate(INDEXER): one indexer key head");
      if (a->q_pos0 < 0) return fail(SA_ERR_VALUE, "sa_estimate(INDEXER): q_pos0 must be >= 0");
      if (a->seq_k > ((int64_t)1 << 31) - 64) return fail(SA_ERR_SHAPE, "sa_estimate(INDEXER): seq_k too large");
      if (a->seq_k % 4) return fail(SA_ERR_SHAPE, "sa_estimate(INDEXER): seq_k must be a multiple of 4");
      if (!aligned16(a->scores)) return fail(SA_ERR_ALIGN, "sa_estimate(INDEXER): scores must be 16-byte aligned");
      return ok();
    }
    default:
      return fail(SA_ERR_VALUE, "sa_estimate: unknown kind %d", a->kind);
  }
}

// ---------------------------------------------------------------- select
int64_t select_max_count(const sa_select_args* a) {
  auto count = [&](int64_t n) {
    const int64_t pb = n < a->n_sink ? n : a->n_sink;
    const int64_t pe = (n - a->n_local) > pb ? (n - a->n_local) : pb;
    const int64_t npool = pe - pb;
    int64_t k = a->ratio_den > 0 ? ((int64_t)a->ratio_num * n + a->ratio_den - 1) / a->ratio_den : a->k;
    if (k > npool) k = npool;
    if (k < 0) k = 0;
    return n - npool + k;
  };
  if (!a->causal) return count(a->ncand);
  int64_t best = 0;
  const int64_t periods = a->rows < a->causal_period ? a->rows : a->causal_period;
  for (int64_t m = 0; m < periods; ++m) {
    int64_t n = m + a->causal_offset + 1;
    if (n > a->ncand) n = a->ncand;
    const int64_t c = count(n);
    if (c > best) best = c;
  }
  return best;
}

int check_select(const sa_select_args* a) {
  if (!a) return fail(SA_ERR_NULL, "sa_select_topk: args is NULL");
  if (a->rows != 0 && (!a->scores || !a->idx || !a->cnt))
    return fail(SA_ERR_NULL, "sa_select_topk: scores, idx and cnt are required");
  if (a->rows < 0 || a->ncand <= 0 || a->ld < a->ncand) return fail(SA_ERR_SHAPE, "sa_select_topk: need ncand > 0 and ld >= ncand");
  if (a->ncand > (int64_t)1 << 24) return fail(SA_ERR_SHAPE, "sa_select_topk: ncand above 2^24");
  if (a->rows > 0x7fffffff) return fail(SA_ERR_SHAPE, "sa_select_topk: too many rows");
  if (a->n_sink < 0 || a->n_local < 0) return fail(SA_ERR_VALUE, "sa_select_topk: n_sink and n_local must be >= 0");
  if (a->ratio_den < 0 || a->ratio_num < 0 || (a->ratio_den == 0 && a->k < 0))
    return fail(SA_ERR_VALUE, "sa_select_topk: budget must be k >= 0 or ratio_num/ratio_den with both >= 0");
  if (a->causal && (a->causal_period <= 0 || a->causal_offset < 0))
    return fail(SA_ERR_VALUE, "sa_select_topk: causal needs causal_period > 0 and causal_offset >= 0");
  if (a->kmax <= 0) return fail(SA_ERR_SHAPE, "sa_select_topk: kmax must be positive");
  const int64_t need = select_max_count(a);
  if (need > a->kmax) return fail(SA_ERR_SHAPE, "sa_select_topk: kmax %d is below the largest possible count %lld", a->kmax, (long long)need);
  return ok();
}

}  // namespace

extern "C" {

const char* sa_last_error(void) { return g_err.c_str(); }

int sa_version(void) { return SA_ABI_VERSION; }

size_t sa_args_size(int which) {
  switch (which) {
    case 0: return sizeof(sa_estimate_args);
    case 1: return sizeof(sa_select_args);
    case 2: return sizeof(sa_vs_build_args);
    case 3: return sizeof(sa_fwd_args);
    case 4: return sizeof(sa_gather_args);
    case 5: return sizeof(sa_cluster_pack_args);
    case 6: return sizeof(sa_select_mass_args);
    case 7: return sizeof(sa_kmeans_args);
    case 8: return sizeof(sa_estimate_topk_args);
    case 9: return sizeof(sa_indexer_topk_args);
    default: return 0;
  }
}

// ---------------------------------------------------------------- estimate
int sa_estimate_workspace_bytes(const sa_estimate_args* a, size_t* bytes) {
  if (!bytes) return fail(SA_ERR_NULL, "sa_estimate_workspace_bytes: bytes is NULL");
  size_t ws = 0;
  const int rc = check_estimate(a, &ws);
  if (rc) return rc;
  *bytes = ws;
  return ok();
}

int sa_estimate(const sa_estimate_args* a, void* workspace, size_t workspace_bytes, void* stream) {
  size_t ws = 0;
  int rc = check_estimate(a, &ws);
  if (rc) return rc;
  if (ws > 0 && (!workspace || workspace_bytes < ws))
    return fail(SA_ERR_WORKSPACE, "sa_estimate: workspace of %zu bytes required", ws);
  if (workspace && !aligned16(workspace)) return fail(SA_ERR_ALIGN, "sa_estimate: workspace must be 16-byte aligned");
  const hipStream_t st = as_stream(stream);
  switch (a->kind) {
    case SA_EST_BLOCK_MEANPOOL: {
      sa::HeadList hl, all;
      all.n = 0;
      make_head_list(a->head_list, a->n_heads_list, a->heads_q, "sa_estimate(BLOCK)", hl);  // checked above
      const int64_t nb = a->seq_q / kBlock;
      const int64_t nh = hl.n > 0 ? hl.n : a->heads_q;
      char* w = static_cast<char*>(workspace);
      float* pq = a->pooled_q;
      float* pk = a->pooled_k;
      if (!pq) {
        pq = reinterpret_cast<float*>(w);
        w += align256((size_t)(a->batch * nh * nb * a->head_dim) * 4);
      }
      if (!pk) pk = reinterpret_cast<float*>(w);
      const bool bf = a->dtype == SA_BF16;
      hipError_t e = sa::launch_pool(a->q, a->batch, (int)a->heads_q, hl, a->seq_q, (int)a->head_dim, bf, kBlock, pq, st);
      if (e == hipSuccess)
        e = sa::launch_pool(a->k, a->batch, (int)a->heads_kv, all, a->seq_k, (int)a->head_dim, bf, kBlock, pk, st);
      if (e == hipSuccess)
        e = sa::launch_block_score(pq, pk, (int)a->batch, (int)a->heads_q, (int)a->heads_kv, hl, (int)nb,
                                   (int)a->head_dim, a->scale, a->scores, a->err_flag, st);
      return launched(e, "sa_estimate(BLOCK)");
    }
    case SA_EST_VSLASH: {
      sa::HeadList hl;
      make_head_list(a->head_list, a->n_heads_list, a->heads_q, "sa_estimate(VSLASH)", hl);  // checked above
      return launched(sa::launch_vs_estimate((const uint16_t*)a->q, (const uint16_t*)a->k, (int)a->batch, (int)a->heads_q,
                                             (int)a->heads_kv, hl, a->seq_q, (int)a->head_dim, a->last_q, a->scale,
                                             a->scores, a->scores2, a->err_flag, workspace, st),
                      "sa_estimate(VSLASH)");
    }
    case SA_EST_CENTROID:
      return launched(sa::launch_centroid_score(a->q, a->dtype == SA_BF16, a->centroids, (int)a->seq_q, (int)a->heads_q,
                                                (int)a->heads_kv, (int)a->n_centroids, (int)a->head_dim, a->scale, a->scores,
                                                a->err_flag, st),
                      "sa_estimate(CENTROID)");
    case SA_EST_INDEXER:
      return launched(sa::launch_indexer((const uint16_t*)a->q, (const uint16_t*)a->k, a->weights, (int)a->seq_q,
                                         (int)a->heads_q, a->seq_k, a->q_pos0, a->scores, a->err_flag, st),
                      "sa_estimate(INDEXER)");
  }
  return fail(SA_ERR_VALUE, "sa_estimate: unknown kind");
}

// ---------------------------------------------------------------- select
int sa_select_topk_workspace_bytes(const sa_select_args* a, size_t* bytes) {
  if (!bytes) return fail(SA_ERR_NULL, "sa_select_topk_workspace_bytes: bytes is NULL");
  const int rc = check_select(a);
  if (rc) return rc;
  *bytes = 0;
  return ok();
}

int sa_select_topk(const sa_select_args* a, void* workspace, size_t workspace_bytes, void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  const int rc = check_select(a);
  if (rc) return rc;
  sa::SelectParams p;
  p.scores = a->scores;
  p.rows = a->rows;
  p.ncand = a->ncand;
  p.ld = a->ld;
  p.period = a->causal ? a->causal_period : 1;
  p.offset = a->causal_offset;
  p.causal = a->causal;
  p.n_sink = a->n_sink;
  p.n_local = a->n_local;
  p.k = a->k;
  p.rnum = a->ratio_num;
  p.rden = a->ratio_den;
  p.kmax = a->kmax;
  p.idx = a->idx;
  p.cnt = a->cnt;
  p.err = a->err_flag;
  return launched(sa::launch_select(p, as_stream(stream)), "sa_select_topk");
}

int sa_select_mass(const sa_select_mass_args* a, void* stream) {
  if (!a) return fail(SA_ERR_NULL, "sa_select_mass: args is NULL");
  if (a->rows != 0 && (!a->scores || !a->idx || !a->cnt))
    return fail(SA_ERR_NULL, "sa_select_mass: scores, idx and cnt are required");
  if (a->rows < 0 || a->rows > 0x7fffffff || a->ncand <= 0 || a->ld < a->ncand)
    return fail(SA_ERR_SHAPE, "sa_select_mass: need rows >= 0, ncand > 0 and ld >= ncand");
  if (a->ncand > sa::kMassMax) return fail(SA_ERR_SHAPE, "sa_select_mass: ncand above %d", sa::kMassMax);
  if (!(a->mass > 0.f && a->mass <= 1.f)) return fail(SA_ERR_VALUE, "sa_select_mass: mass must lie in (0, 1]");
  if (a->k_min < 0 || a->k_max < a->k_min) return fail(SA_ERR_VALUE, "sa_select_mass: need 0 <= k_min <= k_max");
  const int64_t need = a->k_max < a->ncand ? a->k_max : a->ncand;
  if (a->kmax <= 0 || a->kmax < need)
    return fail(SA_ERR_SHAPE, "sa_select_mass: kmax %d is below min(k_max, ncand) = %lld", a->kmax, (long long)need);
  sa::MassParams p;
  p.scores = a->scores;
  p.rows = a->rows;
  p.ncand = a->ncand;
  p.ld = a->ld;
  p.mass = a->mass;
  p.k_min = a->k_min;
  p.k_max = a->k_max;
  p.kmax = a->kmax;
  p.idx = a->idx;
  p.cnt = a->cnt;
  p.err = a->err_flag;
  return launched(sa::launch_select_mass(p, as_stream(stream)), "sa_select_mass");
}

// ---------------------------------------------------------------- fused block estimate + top-k
static int check_centroid_topk(const sa_estimate_topk_args* a) {
  if (!a->q || !a->k_ptr || !a->idx || !a->cnt) return fail(SA_ERR_NULL, "sa_estimate_topk(CENTROID): q, centroids, idx and cnt are required");
  if (!aligned16(a->q) || !aligned16(a->k_ptr)) return fail(SA_ERR_ALIGN, "sa_estimate_topk(CENTROID): q and centroids must be 16-byte aligned");
  if (a->dtype != SA_F32 && a->dtype != SA_BF16) return fail(SA_ERR_DTYPE, "sa_estimate_topk(CENTROID): dtype must be F32 or BF16");
  if (a->head_list || a->n_sink || a->n_local || a->ratio_den)
    return fail(SA_ERR_UNSUPPORTED, "sa_estimate_topk(CENTROID): fixed k only (no head list, forced members or ratio)");
  if (a->seq < 0 || a->heads_q <= 0 || a->heads_kv <= 0 || a->head_dim <= 0) return fail(SA_ERR_SHAPE, "sa_estimate_topk(CENTROID): sizes must be positive");
  if (a->heads_q % a->heads_kv || a->heads_q / a->heads_kv > 8)
    return fail(SA_ERR_UNSUPPORTED, "sa_estimate_topk(CENTROID): heads_q must be 1..8 times heads_kv");
  if (a->head_dim > 128 || a->head_dim % 4) return fail(SA_ERR_UNSUPPORTED, "sa_estimate_topk(CENTROID): head_dim must be a multiple of 4, at most 128");
  if (a->n_centroids < 1 || a->n_centroids > 1024) return fail(SA_ERR_SHAPE, "sa_estimate_topk(CENTROID): n_centroids must lie in [1, 1024]");
  if (a->seq * a->heads_q > 0x7fffffff) return fail(SA_ERR_SHAPE, "sa_estimate_topk(CENTROID): too many query rows");
  if (!(a->scale > 0.f)) return fail(SA_ERR_VALUE, "sa_estimate_topk(CENTROID): scale must be > 0");
  if (a->k < 0) return fail(SA_ERR_VALUE, "sa_estimate_topk(CENTROID): k must be >= 0");
  if (a->mass != 0.f) {
    if (!(a->mass > 0.f && a->mass <= 1.f)) return fail(SA_ERR_VALUE, "sa_estimate_topk(CENTROID): mass must lie in (0, 1]");
    if (a->k_min < 0 || a->k_min > a->k) return fail(SA_ERR_VALUE, "sa_estimate_topk(CENTROID): need 0 <= k_min <= k");
  }
  const int32_t need = a->k < a->n_centroids ? a->k : a->n_centroids;
  if (a->kmax <= 0 || a->kmax < need) return fail(SA_ERR_SHAPE, "sa_estimate_topk(CENTROID): kmax %d is below min(k, C) = %d", a->kmax, need);
  return ok();
}

static int check_estimate_topk(const sa_estimate_topk_args* a, size_t* ws, sa::HeadList& hl) {
  if (!a) return fail(SA_ERR_NULL, "sa_estimate_topk: args is NULL");
  *ws = 0;
  hl.n = 0;
  if (a->kind == SA_EST_CENTROID) return check_centroid_topk(a);
  if (a->kind != SA_EST_BLOCK_MEANPOOL) return fail(SA_ERR_UNSUPPORTED, "sa_estimate_topk: only BLOCK_MEANPOOL and CENTROID");
  if (!a->q || !a->k_ptr || !a->idx || !a->cnt) return fail(SA_ERR_NULL, "sa_estimate_topk: q, k, idx and cnt are required");
  if (!aligned16(a->q) || !aligned16(a->k_ptr)) return fail(SA_ERR_ALIGN, "sa_estimate_topk: q and k must be 16-byte aligned");
  if ((a->pooled_q && !aligned16(a->pooled_q)) || (a->pooled_k && !aligned16(a->pooled_k)))
    return fail(SA_ERR_ALIGN, "sa_estimate_topk: pooled buffers must be 16-byte aligned");
  if (a->dtype != SA_F32 && a->dtype != SA_BF16) return fail(SA_ERR_DTYPE, "sa_estimate_topk: dtype must be F32 or BF16");
  if (a->block_size != kBlock) return fail(SA_ERR_UNSUPPORTED, "sa_estimate_topk: block_size must be 64");
  if (a->head_dim != 64 && a->head_dim != 128) return fail(SA_ERR_UNSUPPORTED, "sa_estimate_topk: head_dim must be 64 or 128");
  if (a->batch <= 0 || a->heads_q <= 0 || a->heads_kv <= 0 || a->seq <= 0) return fail(SA_ERR_SHAPE, "sa_estimate_topk: sizes must be positive");
  if (a->heads_q % a->heads_kv) return fail(SA_ERR_SHAPE, "sa_estimate_topk: heads_q must be a multiple of heads_kv");
  if (a->seq % kBlock) return fail(SA_ERR_SHAPE, "sa_estimate_topk: seq must be a multiple of 64");
  const int64_t nb = a->seq / kBlock;
  if (nb > sa::kBlockTopkMaxBlocks) return fail(SA_ERR_UNSUPPORTED, "sa_estimate_topk: at most %d blocks per row", sa::kBlockTopkMaxBlocks);
  if (!(a->scale > 0.f)) return fail(SA_ERR_VALUE, "sa_estimate_topk: scale must be > 0");
  if (a->n_sink < 0 || a->n_local < 0) return fail(SA_ERR_VALUE, "sa_estimate_topk: n_sink and n_local must be >= 0");
  if (a->ratio_den < 0 || a->ratio_num < 0 || (a->ratio_den == 0 && a->k < 0))
    return fail(SA_ERR_VALUE, "sa_estimate_topk: budget must be k >= 0 or ratio_num/ratio_den with both >= 0");
  if (const int rc = make_head_list(a->head_list, a->n_heads_list, a->heads_q, "sa_estimate_topk", hl)) return rc;
  // the largest count of any row
  int64_t need = 0;
  for (int64_t i = 0; i < nb; ++i) {
    const int64_t n = i + 1;
    const int64_t pb = n < a->n_sink ? n : a->n_sink;
    const int64_t pe = (n - a->n_local) > pb ? (n - a->n_local) : pb;
    int64_t kk = a->ratio_den > 0 ? ((int64_t)a->ratio_num * n + a->ratio_den - 1) / a->ratio_den : a->k;
    if (kk > pe - pb) kk = pe - pb;
    if (kk < 0) kk = 0;
    const int64_t c = n - (pe - pb) + kk;
    if (c > need) need = c;
  }
  if (a->kmax <= 0 || a->kmax < need)
    return fail(SA_ERR_SHAPE, "sa_estimate_topk: kmax %d is below the largest possible count %lld", a->kmax, (long long)need);
  const int64_t nh = hl.n > 0 ? hl.n : a->heads_q;
  if (!a->pooled_q) *ws += align256((size_t)(a->batch * nh * nb * a->head_dim) * 4);
  if (!a->pooled_k) *ws += align256((size_t)(a->batch * a->heads_kv * nb * a->head_dim) * 4);
  return ok();
}

int sa_estimate_topk_workspace_bytes(const sa_estimate_topk_args* a, size_t* bytes) {
  if (!bytes) return fail(SA_ERR_NULL, "sa_estimate_topk_workspace_bytes: bytes is NULL");
  size_t ws = 0;
  sa::HeadList hl;
  const int rc = check_estimate_topk(a, &ws, hl);
  if (rc) return rc;
  *bytes = ws;
  return ok();
}

int sa_estimate_topk(const sa_estimate_topk_args* a, void* workspace, size_t workspace_bytes, void* stream) {
  size_t ws = 0;
  sa::HeadList hl, all;
  all.n = 0;
  const int rc = check_estimate_topk(a, &ws, hl);
  if (rc) return rc;
  if (ws > 0 && (!workspace || workspace_bytes < ws))
    return fail(SA_ERR_WORKSPACE, "sa_estimate_topk: workspace of %zu bytes required", ws);
  if (workspace && !aligned16(workspace)) return fail(SA_ERR_ALIGN, "sa_estimate_topk: workspace must be 16-byte aligned");
  const hipStream_t st = as_stream(stream);
  if (a->kind == SA_EST_CENTROID)
    return launched(sa::launch_centroid_topk(a->q, a->dtype == SA_BF16, static_cast<const float*>(a->k_ptr), (int)a->seq,
                                             (int)a->heads_q, (int)a->heads_kv, a->n_centroids, (int)a->head_dim,
                                             a->scale, a->k, a->kmax, a->mass, a->k_min, a->idx, a->cnt, a->err_flag,
                                             st),
                    "sa_estimate_topk(CENTROID)");
  const int64_t nb = a->seq / kBlock;
  const int64_t nh = hl.n > 0 ? hl.n : a->heads_q;
  char* w = static_cast<char*>(workspace);
  float* pq = a->pooled_q;
  float* pk = a->pooled_k;
  if (!pq) {
    pq = reinterpret_cast<float*>(w);
    w += align256((size_t)(a->batch * nh * nb * a->head_dim) * 4);
  }
  if (!pk) pk = reinterpret_cast<float*>(w);
  const bool bf = a->dtype == SA_BF16;
  hipError_t e = sa::launch_pool(a->q, a->batch, (int)a->heads_q, hl, a->seq, (int)a->head_dim, bf, kBlock, pq, st);
  if (e == hipSuccess)
    e = sa::launch_pool(a->k_ptr, a->batch, (int)a->heads_kv, all, a->seq, (int)a->head_dim, bf, kBlock, pk, st);
  if (e == hipSuccess) {
    sa::BlockTopkParams p;
    p.pq = pq;
    p.pk = pk;
    p.idx = a->idx;
    p.cnt = a->cnt;
    p.err = a->err_flag;
    p.batch = (int32_t)a->batch;
    p.hq = (int32_t)a->heads_q;
    p.hkv = (int32_t)a->heads_kv;
    p.nb = (int32_t)nb;
    p.kmax = a->kmax;
    p.n_sink = a->n_sink;
    p.n_local = a->n_local;
    p.k = a->k;
    p.rnum = a->ratio_num;
    p.rden = a->ratio_den;
    p.scale = a->scale;
    p.hl = hl;
    e = sa::launch_block_topk(p, (int)a->head_dim, st);
  }
  return launched(e, "sa_estimate_topk");
}

// ---------------------------------------------------------------- vertical-slash tables
int sa_vs_build(const sa_vs_build_args* a, void* stream) {
  if (!a) return fail(SA_ERR_NULL, "sa_vs_build: args is NULL");
  if (!a->vert || !a->vert_cnt || !a->slash || !a->slash_cnt || !a->iv || !a->iv_cnt || !a->col || !a->col_cnt)
    return fail(SA_ERR_NULL, "sa_vs_build: all table pointers are required");
  if (a->block_size != kBlock) return fail(SA_ERR_UNSUPPORTED, "sa_vs_build: block_size must be 64");
  if (a->rows < 0 || a->seq <= 0 || a->seq % kBlock || a->n_vert <= 0 || a->n_slash <= 0)
    return fail(SA_ERR_SHAPE, "sa_vs_build: need seq a positive multiple of 64 and positive capacities");
  if (a->seq > 0x7fffffff - 64) return fail(SA_ERR_SHAPE, "sa_vs_build: seq too large");
  sa::VsBuildParams p;
  p.rows = a->rows;
  p.seq = a->seq;
  p.bs = a->block_size;
  p.n_vert = a->n_vert;
  p.n_slash = a->n_slash;
  p.vert = a->vert;
  p.vert_cnt = a->vert_cnt;
  p.slash = a->slash;
  p.slash_cnt = a->slash_cnt;
  p.iv = a->iv;
  p.iv_cnt = a->iv_cnt;
  p.col = a->col;
  p.col_cnt = a->col_cnt;
  return launched(sa::launch_vs_build(p, as_stream(stream)), "sa_vs_build");
}

// ---------------------------------------------------------------- forward
static int check_fwd(const sa_fwd_args* a) {
  if (!a) return fail(SA_ERR_NULL, "sa_block_sparse_fwd: args is NULL");
  if (!a->q || !a->k || !a->v || !a->out) return fail(SA_ERR_NULL, "sa_block_sparse_fwd: q, k, v and out are required");
  if (!aligned16(a->q) || !aligned16(a->k) || !aligned16(a->v) || !aligned16(a->out))
    return fail(SA_ERR_ALIGN, "sa_block_sparse_fwd: q, k, v and out must be 16-byte aligned");
  if (a->dtype != SA_F32 && a->dtype != SA_BF16) return fail(SA_ERR_DTYPE, "sa_block_sparse_fwd: dtype must be F32 or BF16");
  if (a->out_dtype != SA_F32 && a->out_dtype != SA_BF16) return fail(SA_ERR_DTYPE, "sa_block_sparse_fwd: out_dtype must be F32 or BF16");
  if (a->dtype == SA_F32 && a->out_dtype != SA_F32) return fail(SA_ERR_DTYPE, "sa_block_sparse_fwd: F32 inputs need F32 output");
  if (a->block_size != kBlock) return fail(SA_ERR_UNSUPPORTED, "sa_block_sparse_fwd: block_size must be 64");
  if (a->head_dim != 64 && a->head_dim != 128) return fail(SA_ERR_UNSUPPORTED, "sa_block_sparse_fwd: head_dim must be 64 or 128");
  if (a->batch <= 0 || a->heads_q <= 0 || a->heads_kv <= 0 || a->seq <= 0) return fail(SA_ERR_SHAPE, "sa_block_sparse_fwd: sizes must be positive");
  if (a->heads_q % a->heads_kv) return fail(SA_ERR_SHAPE, "sa_block_sparse_fwd: heads_q must be a multiple of heads_kv");
  if (a->seq % kBlock) return fail(SA_ERR_SHAPE, "sa_block_sparse_fwd: seq must be a multiple of 64");
  if (a->seq > 0x7fffffff - 64) return fail(SA_ERR_SHAPE, "sa_block_sparse_fwd: seq too large");
  if (a->batch * a->heads_q * (a->seq / kBlock) > 0x7fffffff) return fail(SA_ERR_SHAPE, "sa_block_sparse_fwd: too many query blocks");
  if (!(a->scale > 0.f)) return fail(SA_ERR_VALUE, "sa_block_sparse_fwd: scale must be > 0");
  if (a->mode == SA_FWD_BLOCK) {
    if (!a->block_idx || !a->block_cnt) return fail(SA_ERR_NULL, "sa_block_sparse_fwd(BLOCK): block_idx and block_cnt required");
    if (a->kmax <= 0) return fail(SA_ERR_SHAPE, "sa_block_sparse_fwd(BLOCK): kmax must be positive");
    if (a->dtype == SA_BF16 && a->kmax > 2048)
      return fail(SA_ERR_UNSUPPORTED, "sa_block_sparse_fwd(BLOCK): bf16 path stages at most 2048 blocks per row (kmax)");
  } else if (a->mode == SA_FWD_VSLASH) {
    if (!a->iv || !a->iv_cnt || !a->col || !a->col_cnt) return fail(SA_ERR_NULL, "sa_block_sparse_fwd(VSLASH): tables required");
    if (a->max_iv <= 0 || a->max_col <= 0) return fail(SA_ERR_SHAPE, "sa_block_sparse_fwd(VSLASH): capacities must be positive");
    if (a->dtype == SA_BF16 && (a->max_iv > 64 || a->max_col > 1920))
      return fail(SA_ERR_UNSUPPORTED, "sa_block_sparse_fwd(VSLASH): bf16 path stages at most 64 intervals and 1920 columns per row");
  } else if (a->mode == SA_FWD_ASHAPE) {
    if (a->n_sink < 0 || a->n_local < 0) return fail(SA_ERR_VALUE, "sa_block_sparse_fwd(ASHAPE): n_sink and n_local must be >= 0");
    if ((int64_t)a->n_sink + a->n_local > 2048)
      return fail(SA_ERR_UNSUPPORTED, "sa_block_sparse_fwd(ASHAPE): n_sink + n_local above 2048 blocks");
  } else {
    return fail(SA_ERR_VALUE, "sa_block_sparse_fwd: unknown mode %d", a->mode);
  }
  sa::HeadList hl;
  return make_head_list(a->head_list, a->n_heads_list, a->heads_q, "sa_block_sparse_fwd", hl);
}

int sa_block_sparse_fwd_workspace_bytes(const sa_fwd_args* a, size_t* bytes) {
  if (!bytes) return fail(SA_ERR_NULL, "sa_block_sparse_fwd_workspace_bytes: bytes is NULL");
  const int rc = check_fwd(a);
  if (rc) return rc;
  *bytes = 0;
  return ok();
}

int sa_block_sparse_fwd(const sa_fwd_args* a, void* workspace, size_t workspace_bytes, void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  const int rc = check_fwd(a);
  if (rc) return rc;
  sa::FwdParams p;
  p.q = a->q;
  p.k = a->k;
  p.v = a->v;
  p.out = a->out;
  p.lse = a->lse;
  p.block_idx = a->block_idx;
  p.block_cnt = a->block_cnt;
  p.iv = a->iv;
  p.iv_cnt = a->iv_cnt;
  p.col = a->col;
  p.col_cnt = a->col_cnt;
  p.seq = a->seq;
  p.batch = (int32_t)a->batch;
  p.heads_q = (int32_t)a->heads_q;
  p.heads_kv = (int32_t)a->heads_kv;
  p.nqb = (int32_t)(a->seq / kBlock);
  p.kmax = a->kmax;
  p.max_iv = a->max_iv;
  p.max_col = a->max_col;
  p.scale = a->scale;
  p.order = 0;
  p.ashape = a->mode == SA_FWD_ASHAPE;
  p.n_sink = a->n_sink;
  p.n_local = a->n_local;
  make_head_list(a->head_list, a->n_heads_list, a->heads_q, "sa_block_sparse_fwd", p.hl);  // checked above
  // the A-shape lists are generated by the block-mode kernels
  const int kmode = a->mode == SA_FWD_VSLASH ? 1 : 0;
  return launched(sa::launch_fwd(p, (int)a->head_dim, kmode, a->dtype == SA_BF16, a->out_dtype == SA_BF16,
                                 as_stream(stream)),
                  "sa_block_sparse_fwd");
}

// ---------------------------------------------------------------- offline k-means
static int check_kmeans(const sa_kmeans_args* a, size_t* ws) {
  if (!a) return fail(SA_ERR_NULL, "sa_kmeans: args is NULL");
  *ws = 0;
  if (!a->k || !a->centroids || !a->labels) return fail(SA_ERR_NULL, "sa_kmeans: k, centroids and labels are required");
  if ((a->cluster_ptr == nullptr) != (a->perm == nullptr))
    return fail(SA_ERR_NULL, "sa_kmeans: give both cluster_ptr and perm, or neither");
  if (!aligned16(a->k) || !aligned16(a->centroids)) return fail(SA_ERR_ALIGN, "sa_kmeans: k and centroids must be 16-byte aligned");
  if (a->dtype != SA_F32 && a->dtype != SA_BF16) return fail(SA_ERR_DTYPE, "sa_kmeans: dtype must be F32 or BF16");
  if (a->head_dim != 64 && a->head_dim != 128) return fail(SA_ERR_UNSUPPORTED, "sa_kmeans: head_dim must be 64 or 128");
  if (a->heads_kv <= 0 || a->n_ctx <= 0) return fail(SA_ERR_SHAPE, "sa_kmeans: sizes must be positive");
  if (a->n_ctx > 0x7fffffff || a->heads_kv * a->n_ctx > 0x7fffffff) return fail(SA_ERR_SHAPE, "sa_kmeans: too many keys");
  if (a->n_clusters < 1 || a->n_clusters > 4096) return fail(SA_ERR_SHAPE, "sa_kmeans: n_clusters must lie in [1, 4096]");
  if (a->heads_kv * a->n_clusters > 0x7fffffff) return fail(SA_ERR_SHAPE, "sa_kmeans: too many clusters");
  if (a->iters < 1) return fail(SA_ERR_VALUE, "sa_kmeans: iters must be >= 1");
  *ws = sa::kmeans_workspace_bytes(a->heads_kv, a->n_ctx, a->n_clusters, (int)a->head_dim);
  if (!a->cluster_ptr)
    *ws += align256((size_t)(a->heads_kv * (a->n_clusters + 1)) * 4) + align256((size_t)(a->heads_kv * a->n_ctx) * 4);
  return ok();
}

int sa_kmeans_workspace_bytes(const sa_kmeans_args* a, size_t* bytes) {
  if (!bytes) return fail(SA_ERR_NULL, "sa_kmeans_workspace_bytes: bytes is NULL");
  size_t ws = 0;
  const int rc = check_kmeans(a, &ws);
  if (rc) return rc;
  *bytes = ws;
  return ok();
}

int sa_kmeans(const sa_kmeans_args* a, void* workspace, size_t workspace_bytes, void* stream) {
  size_t ws = 0;
  const int rc = check_kmeans(a, &ws);
  if (rc) return rc;
  if (!workspace || workspace_bytes < ws) return fail(SA_ERR_WORKSPACE, "sa_kmeans: workspace of %zu bytes required", ws);
  if (!aligned16(workspace)) return fail(SA_ERR_ALIGN, "sa_kmeans: workspace must be 16-byte aligned");
  char* w = static_cast<char*>(workspace);
  void* pack_ws = w;
  w += align256(sa::kmeans_workspace_bytes(a->heads_kv, a->n_ctx, a->n_clusters, (int)a->head_dim));
  int32_t* ptr = a->cluster_ptr;
  int32_t* perm = a->perm;
  if (!ptr) {
    ptr = reinterpret_cast<int32_t*>(w);
    w += align256((size_t)(a->heads_kv * (a->n_clusters + 1)) * 4);
    perm = reinterpret_cast<int32_t*>(w);
  }
  return launched(sa::launch_kmeans(a->k, a->dtype == SA_BF16, a->heads_kv, a->n_ctx, (int)a->head_dim, a->n_clusters,
                                    a->iters, a->centroids, a->labels, ptr, perm, pack_ws, as_stream(stream)),
                  "sa_kmeans");
}

// ---------------------------------------------------------------- gather / decode
static int check_gather(const sa_gather_args* a, size_t* ws) {
  if (!a) return fail(SA_ERR_NULL, "sa_gather_decode: args is NULL");
  *ws = 0;
  if (!a->q || !a->k || !a->v || !a->out) return fail(SA_ERR_NULL, "sa_gather_decode: q, k, v and out are required");
  if (!aligned16(a->q) || !aligned16(a->k) || !aligned16(a->v) || !aligned16(a->out))
    return fail(SA_ERR_ALIGN, "sa_gather_decode: q, k, v and out must be 16-byte aligned");
  if (a->dtype != SA_BF16) return fail(SA_ERR_DTYPE, "sa_gather_decode: dtype must be BF16");
  if (a->out_dtype != SA_F32 && a->out_dtype != SA_BF16) return fail(SA_ERR_DTYPE, "sa_gather_decode: out_dtype must be F32 or BF16");
  if (a->head_dim != 128) return fail(SA_ERR_UNSUPPORTED, "sa_gather_decode: head_dim must be 128");
  if (a->n_q <= 0 || a->heads_q <= 0 || a->heads_kv <= 0 || a->n_ctx <= 0) return fail(SA_ERR_SHAPE, "sa_gather_decode: sizes must be positive");
  if (a->heads_q % a->heads_kv) return fail(SA_ERR_SHAPE, "sa_gather_decode: heads_q must be a multiple of heads_kv");
  if (a->n_ctx > 0x7fffffff) return fail(SA_ERR_SHAPE, "sa_gather_decode: n_ctx too large");
  if (!(a->scale > 0.f)) return fail(SA_ERR_VALUE, "sa_gather_decode: scale must be > 0");
  if (a->mode == SA_GATHER_CLUSTER) {
    if (!a->cluster_ptr || !a->sel) return fail(SA_ERR_NULL, "sa_gather_decode(CLUSTER): cluster_ptr and sel required");
    if (a->n_clusters <= 0 || a->n_sel <= 0) return fail(SA_ERR_SHAPE, "sa_gather_decode(CLUSTER): n_clusters and n_sel must be positive");
    if (a->n_q * (a->heads_q / a->heads_kv) > 64)
      return fail(SA_ERR_UNSUPPORTED, "sa_gather_decode(CLUSTER): at most 64 queries per KV head");
    if (a->n_clusters > 1024) return fail(SA_ERR_UNSUPPORTED, "sa_gather_decode(CLUSTER): at most 1024 clusters");
    if (a->q_pos && !a->perm) return fail(SA_ERR_NULL, "sa_gather_decode(CLUSTER): q_pos needs perm");
    *ws = sa::cluster_decode_workspace_bytes((int)a->n_q, (int)a->heads_q, (int)a->heads_kv, a->n_clusters, a->n_ctx);
  } else if (a->mode == SA_GATHER_TOKEN) {
    if (!a->tok_idx) return fail(SA_ERR_NULL, "sa_gather_decode(TOKEN): tok_idx required");
    if (a->n_tok <= 0) return fail(SA_ERR_SHAPE, "sa_gather_decode(TOKEN): n_tok must be positive");
    if (a->tok_per_head != 0 && a->tok_per_head != 1) return fail(SA_ERR_VALUE, "sa_gather_decode(TOKEN): tok_per_head must be 0 or 1");
    *ws = sa::token_gather_workspace_bytes((int)a->n_q, (int)a->heads_q, a->n_tok);
  } else {
    return fail(SA_ERR_VALUE, "sa_gather_decode: unknown mode %d", a->mode);
  }
  return ok();
}

int sa_gather_decode_workspace_bytes(const sa_gather_args* a, size_t* bytes) {
  if (!bytes) return fail(SA_ERR_NULL, "sa_gather_decode_workspace_bytes: bytes is NULL");
  size_t ws = 0;
  const int rc = check_gather(a, &ws);
  if (rc) return rc;
  *bytes = ws;
  return ok();
}

static sa::GatherParams gather_params(const sa_gather_args* a) {
  sa::GatherParams p;
  p.q = (const uint16_t*)a->q;
  p.k = (const uint16_t*)a->k;
  p.v = (const uint16_t*)a->v;
  p.cluster_ptr = a->cluster_ptr;
  p.sel = a->sel;
  p.tok_idx = a->tok_idx;
  p.q_pos = a->q_pos;
  p.perm = a->perm;
  p.tok_per_head = a->mode == SA_GATHER_TOKEN ? a->tok_per_head : 0;
  p.out = a->out;
  p.lse = a->lse;
  p.n_ctx = a->n_ctx;
  p.T = (int32_t)a->n_q;
  p.hq = (int32_t)a->heads_q;
  p.hkv = (int32_t)a->heads_kv;
  p.C = a->n_clusters;
  p.n_sel = a->n_sel;
  p.n_tok = a->n_tok;
  p.scale = a->scale;
  p.out_bf16 = a->out_dtype == SA_BF16;
  return p;
}

static int launch_gather(const sa_gather_args* a, void* workspace, void* stream) {
  const sa::GatherParams p = gather_params(a);
  if (a->mode == SA_GATHER_CLUSTER)
    return launched(sa::launch_cluster_decode(p, workspace, as_stream(stream)), "sa_gather_decode(CLUSTER)");
  return launched(sa::launch_token_gather(p, workspace, as_stream(stream)), "sa_gather_decode(TOKEN)");
}

int sa_gather_decode(const sa_gather_args* a, void* workspace, size_t workspace_bytes, void* stream) {
  size_t ws = 0;
  const int rc = check_gather(a, &ws);
  if (rc) return rc;
  if (ws > 0 && (!workspace || workspace_bytes < ws))
    return fail(SA_ERR_WORKSPACE, "sa_gather_decode: workspace of %zu bytes required", ws);
  if (workspace && !aligned16(workspace)) return fail(SA_ERR_ALIGN, "sa_gather_decode: workspace must be 16-byte aligned");
  return launch_gather(a, workspace, stream);
}

}  // extern "C"

// ---------------------------------------------------------------- allocation-free decode
// Scratch of sa_gather_decode_static: a file-scope device array, one copy per
// GPU for the life of the process.  On the host the name only identifies the
// symbol; its device address comes from hipGetSymbolAddress, taken once per
// device with that device current and kept here.
namespace {
static __device__ __align__(256) unsigned char scratch[SA_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int static_scratch(void** out) {
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SA_ERR_LAUNCH, "sa_gather_decode_static: hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(SA_ERR_UNSUPPORTED, "sa_gather_decode_static: device %d", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    const hipError_t r = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (r != hipSuccess || ptr == nullptr)
      return fail(SA_ERR_LAUNCH, "sa_gather_decode_static: hipGetSymbolAddress: %s", hipGetErrorString(r));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return SA_OK;
}
}  // namespace

extern "C" {

int sa_gather_decode_static(const sa_gather_args* a, void* stream) {
  size_t ws = 0;
  const int rc = check_gather(a, &ws);
  if (rc) return rc;
  if (ws > SA_STATIC_SCRATCH_BYTES)
    return fail(SA_ERR_UNSUPPORTED, "sa_gather_decode_static: this call needs %zu bytes of scratch; the static buffer holds %zu",
                ws, (size_t)SA_STATIC_SCRATCH_BYTES);
  void* ptr = nullptr;
  if (ws > 0) {
    const int r = static_scratch(&ptr);
    if (r) return r;
  }
  (void)as_stream(stream);  // clears an unrelated earlier runtime error, as every entry point does
  return launch_gather(a, ptr, stream);
}

// ---------------------------------------------------------------- cluster pack
static int check_pack(const sa_cluster_pack_args* a, size_t* ws) {
  if (!a) return fail(SA_ERR_NULL, "sa_cluster_pack: args is NULL");
  *ws = 0;
  if (!a->labels || !a->cluster_ptr || !a->perm) return fail(SA_ERR_NULL, "sa_cluster_pack: labels, cluster_ptr and perm required");
  if (a->heads_kv <= 0 || a->n_ctx <= 0 || a->n_clusters <= 0) return fail(SA_ERR_SHAPE, "sa_cluster_pack: sizes must be positive");
  if (a->n_ctx > 0x7fffffff) return fail(SA_ERR_SHAPE, "sa_cluster_pack: n_ctx too large");
  const bool copy = a->k || a->v || a->k_packed || a->v_packed;
  if (copy) {
    if (!a->k || !a->v || !a->k_packed || !a->v_packed) return fail(SA_ERR_NULL, "sa_cluster_pack: k, v, k_packed and v_packed go together");
    if (a->dtype != SA_F32 && a->dtype != SA_BF16) return fail(SA_ERR_DTYPE, "sa_cluster_pack: dtype must be F32 or BF16");
    const int eb = a->dtype == SA_F32 ? 4 : 2;
    if (a->head_dim <= 0 || (a->head_dim * eb) % 16) return fail(SA_ERR_SHAPE, "sa_cluster_pack: rows must be a multiple of 16 bytes");
    if (!aligned16(a->k) || !aligned16(a->v) || !aligned16(a->k_packed) || !aligned16(a->v_packed))
      return fail(SA_ERR_ALIGN, "sa_cluster_pack: k/v buffers must be 16-byte aligned");
  }
  if (a->n_clusters > 16384) return fail(SA_ERR_UNSUPPORTED, "sa_cluster_pack: at most 16384 clusters");
  *ws = sa::cluster_pack_workspace_bytes(a->heads_kv, a->n_ctx, a->n_clusters);
  return ok();
}

int sa_cluster_pack_workspace_bytes(const sa_cluster_pack_args* a, size_t* bytes) {
  if (!bytes) return fail(SA_ERR_NULL, "sa_cluster_pack_workspace_bytes: bytes is NULL");
  size_t ws = 0;
  const int rc = check_pack(a, &ws);
  if (rc) return rc;
  *bytes = ws;
  return ok();
}

int sa_cluster_pack(const sa_cluster_pack_args* a, void* workspace, size_t workspace_bytes, void* stream) {
  size_t ws = 0;
  const int rc = check_pack(a, &ws);
  if (rc) return rc;
  if (ws > 0 && (!workspace || workspace_bytes < ws))
    return fail(SA_ERR_WORKSPACE, "sa_cluster_pack: workspace of %zu bytes required", ws);
  const int eb = a->dtype == SA_F32 ? 4 : 2;
  return launched(sa::launch_cluster_pack(a->labels, a->heads_kv, a->n_ctx, a->n_clusters, a->cluster_ptr, a->perm, a->k,
                                          a->v, a->k_packed, a->v_packed, (int)a->head_dim, eb, a->err_flag, workspace,
                                          as_stream(stream)),
                  "sa_cluster_pack");
}

// ---------------------------------------------------------------- indexer top-k
static int check_indexer_topk(const sa_indexer_topk_args* a) {
  if (!a) return fail(SA_ERR_NULL, "sa_indexer_topk: args is NULL");
  if (a->seq_q < 0 || a->seq_k <= 0) return fail(SA_ERR_SHAPE, "sa_indexer_topk: seq_q must be >= 0 and seq_k > 0");
  if (a->seq_q == 0) return ok();
  if (!a->q || !a->k_ptr || !a->weights || !a->idx || !a->cnt)
    return fail(SA_ERR_NULL, "sa_indexer_topk: q, k, weights, idx and cnt are required");
  if (!aligned16(a->q) || !aligned16(a->k_ptr)) return fail(SA_ERR_ALIGN, "sa_indexer_topk: q and k must be 16-byte aligned");
  if (a->heads != 32 && a->heads != 64) return fail(SA_ERR_UNSUPPORTED, "sa_indexer_topk: heads must be 32 or 64");
  if (a->head_dim != 64) return fail(SA_ERR_UNSUPPORTED, "sa_indexer_topk: head_dim must be 64");
  if (a->q_pos0 < 0) return fail(SA_ERR_VALUE, "sa_indexer_topk: q_pos0 must be >= 0");
  if (a->seq_q > 0x7fffffff) return fail(SA_ERR_SHAPE, "sa_indexer_topk: seq_q too large");
  if (a->seq_k > ((int64_t)1 << 31) - 64) return fail(SA_ERR_SHAPE, "sa_indexer_topk: seq_k too large");
  if (a->k < 1 || a->k > 2048) return fail(SA_ERR_VALUE, "sa_indexer_topk: k must lie in [1, 2048]");
  const int64_t nmax = a->seq_k < a->q_pos0 + a->seq_q ? a->seq_k : a->q_pos0 + a->seq_q;
  const int64_t need = a->k < nmax ? a->k : nmax;
  if (a->kmax < need) return fail(SA_ERR_SHAPE, "sa_indexer_topk: kmax %d is below min(k, longest row) = %lld", a->kmax, (long long)need);
  return ok();
}

int sa_indexer_topk_workspace_bytes(const sa_indexer_topk_args* a, size_t* bytes) {
  if (!bytes) return fail(SA_ERR_NULL, "sa_indexer_topk_workspace_bytes: bytes is NULL");
  const int rc = check_indexer_topk(a);
  if (rc) return rc;
  *bytes = a->seq_q == 0 ? 0 : sa::indexer_topk_workspace_bytes((int)a->seq_q, a->seq_k, a->q_pos0, a->k);
  return ok();
}

int sa_indexer_topk(const sa_indexer_topk_args* a, void* workspace, size_t workspace_bytes, void* stream) {
  const int rc = check_indexer_topk(a);
  if (rc) return rc;
  if (a->seq_q == 0) return ok();
  const size_t ws = sa::indexer_topk_workspace_bytes((int)a->seq_q, a->seq_k, a->q_pos0, a->k);
  if (!workspace || workspace_bytes < ws) return fail(SA_ERR_WORKSPACE, "sa_indexer_topk: workspace of %zu bytes required", ws);
  if (!aligned16(workspace)) return fail(SA_ERR_ALIGN, "sa_indexer_topk: workspace must be 16-byte aligned");
  return launched(sa::launch_indexer_topk(static_cast<const uint16_t*>(a->q), static_cast<const uint16_t*>(a->k_ptr),
                                          a->weights, (int)a->seq_q, a->heads, a->seq_k, a->q_pos0, a->k, a->kmax,
                                          a->idx, a->cnt, a->err_flag, workspace, as_stream(stream)),
                  "sa_indexer_topk");
}

}  // extern "C"
