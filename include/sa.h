/*
 * sa.h — C ABI of libsa: dynamic sparse attention on AMD Instinct MI355X (gfx950).
 *
 * The method (sources cited per entry point):
 *   a cheap estimator scores key blocks, key clusters or key tokens; a per-row
 *   top-k keeps a subset; exact softmax attention runs over the kept keys only.
 *
 * Conventions shared by every entry point
 *   - Plain C.  Every tensor pointer is a DEVICE pointer owned by the caller.
 *     The library never allocates or frees device memory: scratch space comes
 *     from a caller-provided workspace whose size the matching
 *     *_workspace_bytes() call returns (0 is a valid answer).
 *   - Tensors are dense, row-major, in the documented shape order; the last
 *     dimension is contiguous.  q, k, v, out pointers must be 16-byte aligned.
 *     There is no strided-tensor descriptor: every kernel copies whole rows at
 *     the dense pitch, so a strided view must be made contiguous by the
 *     caller (the binding rejects non-contiguous tensors).
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the
 *     default stream).  No call synchronises the host.
 *   - The return value is an sa_status.  Argument errors are detected on the
 *     host before any launch and leave all outputs untouched; the message is
 *     kept per thread and returned by sa_last_error().  SA_ERR_LAUNCH reports a
 *     HIP launch failure.
 *   - Outputs are bitwise deterministic run to run (no floating-point atomics).
 *   - Element types: SA_F32 (float), SA_BF16 (bfloat16 bit patterns, uint16),
 *     SA_I32 (int32).  Scores, pooled vectors and lse are always float.
 *   - Grouped-query heads: query head h reads KV head floor(h*Hkv/Hq);
 *     Hq must be a multiple of Hkv.
 */
#ifndef SA_H_
#define SA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SA_ABI_VERSION 9

typedef enum sa_status {
  SA_OK = 0,
  SA_ERR_NULL = 1,        /* a required pointer is NULL */
  SA_ERR_SHAPE = 2,       /* a size is out of range or inconsistent */
  SA_ERR_DTYPE = 3,       /* unsupported element type */
  SA_ERR_ALIGN = 4,       /* pointer not 16-byte aligned */
  SA_ERR_WORKSPACE = 5,   /* workspace missing or smaller than required */
  SA_ERR_UNSUPPORTED = 6, /* a valid request the library does not implement */
  SA_ERR_LAUNCH = 7,      /* HIP reported an error at launch */
  SA_ERR_VALUE = 8        /* a parameter value is invalid (e.g. scale, k) */
} sa_status;

typedef enum sa_dtype { SA_F32 = 0, SA_BF16 = 1, SA_I32 = 2 } sa_dtype;

/* ======================================================================
 * sa_estimate — cheap scores that rank keys, blocks or clusters.
 *
 * kind = SA_EST_BLOCK_MEANPOOL
 *   "MInference 1.0" article, §方法介紹: block-sparse indices are estimated
 *   from mean-pooled Q and K (mean pooling commutes with the product).
 *   q [B,Hq,N,d], k [B,Hkv,N,d] (F32 or BF16), N a multiple of block_size.
 *   scores [B,Hq,nb,nb] float, nb = N/block_size:
 *     scores[b,h,i,j] = mean(q rows of block i) . mean(k rows of block j) * scale
 *     for j <= i.  Entries with j > i are not written (sa_select_topk with
 *     causal = 1 never reads them), which halves the bytes this call stores.
 *   pooled_q [B,Hq,nb,d] / pooled_k [B,Hkv,nb,d]: optional float outputs of the
 *   block means; when NULL the means live in the workspace.
 *
 * kind = SA_EST_VSLASH
 *   "MInference 1.0" article, §方法介紹: vertical and slash indices are
 *   estimated from the attention of the last queries to all keys.
 *   q [B,Hq,N,d], k [B,Hkv,N,d] (BF16).  The last `last_q` query rows, at
 *   positions N-last_q .. N-1, attend keys causally: A = softmax(q k^T scale).
 *   scores  [B,Hq,N] float: vertical score  a_v[c] = sum_r A[r,c]
 *   scores2 [B,Hq,N] float: slash score     a_s[o] = sum_r A[r, pos_r - o]
 *   Requires a workspace.
 *
 * kind = SA_EST_CENTROID
 *   Squeezed Attention page, §技术方案: each query is compared with every
 *   cluster centroid; §核心贡献/§技术方案 keep centroids in on-chip memory.
 *   q [T,Hq,d] (BF16 or F32), centroids [Hkv,C,d] float.
 *   scores [T,Hq,C] float = q[t,h] . centroids[g(h),c] * scale.
 *
 * kind = SA_EST_INDEXER
 *   IndexCache article, §长文本的算力困境: a light indexer scores every key
 *   token for every query.  Score of the synthetic workload:
 *     I[t,s] = sum_h weights[h] * max(0, q[t,h,:] . k[s,:])   for s <= q_pos0 + t
 *   q [T,Hi,di] (BF16; heads_q = Hi, head_dim = di, seq_q = T),
 *   k [Nk,di] (BF16; seq_k = Nk, heads_kv = 1), weights [Hi] float.
 *   scores [T,Nk] float, -INFINITY where s > q_pos0 + t.  No scale.
 *   di must be 64; Hi a multiple of 8, at most 64.
 *
 * Head list (BLOCK_MEANPOOL and VSLASH; "MInference 1.0" article, §方法介紹:
 * each head runs the estimate of its own pattern): head_list, when not NULL,
 * is a HOST array of n_heads_list distinct query-head indices in [0, Hq)
 * (at most 256; copied into the launch, so it may be freed on return).  Only
 * those heads are estimated, and every per-head output is compact: scores
 * [B,n,nb,nb] (BLOCK) or [B,n,N] (VSLASH), pooled_q [B,n,nb,d], with row
 * b*n + j for listed head j.  q, k and pooled_k keep their full layouts.
 * ====================================================================== */
enum { SA_EST_BLOCK_MEANPOOL = 0, SA_EST_VSLASH = 1, SA_EST_CENTROID = 2, SA_EST_INDEXER = 3 };

typedef struct sa_estimate_args {
  int32_t kind;
  int32_t dtype;          /* element type of q and k */
  int64_t batch;          /* B (BLOCK, VSLASH); ignored otherwise */
  int64_t heads_q;        /* Hq, or Hi for INDEXER */
  int64_t heads_kv;       /* Hkv; 1 for INDEXER */
  int64_t seq_q;          /* N (BLOCK, VSLASH) or T (CENTROID, INDEXER) */
  int64_t seq_k;          /* N, Nctx or Nk */
  int64_t head_dim;       /* d (64 or 128), di for INDEXER */
  int64_t n_centroids;    /* C (CENTROID) */
  int64_t q_pos0;         /* INDEXER: absolute position of query 0 */
  int32_t block_size;     /* BLOCK: 64 */
  int32_t last_q;         /* VSLASH: 64 */
  float scale;            /* BLOCK, VSLASH, CENTROID: > 0 */
  int32_t reserved0;
  const void* q;
  const void* k;
  const float* centroids; /* CENTROID */
  const float* weights;   /* INDEXER */
  float* scores;
  float* scores2;         /* VSLASH slash scores */
  float* pooled_q;        /* BLOCK, optional */
  float* pooled_k;        /* BLOCK, optional */
  const int32_t* head_list; /* BLOCK, VSLASH: optional host array */
  int32_t n_heads_list;
  int32_t reserved1;
  int32_t* err_flag;      /* optional device int32: bit 0 (value 1) is set when a
                             score written (masked entries aside) is NaN or
                             infinite, and for INDEXER also when an element of
                             q, k or weights is (its ReLU can hide a NaN
                             product); never cleared by the library */
} sa_estimate_args;

int sa_estimate_workspace_bytes(const sa_estimate_args* args, size_t* bytes);
int sa_estimate(const sa_estimate_args* args, void* workspace, size_t workspace_bytes, void* stream);

/* ======================================================================
 * sa_select_topk — per-row top-k with forced members.
 *
 * The top subset by score is kept ("MInference 1.0" article, §方法介紹;
 * Squeezed Attention page, §技术方案 "select the top-K clusters"; IndexCache
 * article, §长文本的算力困境).  Local and global members are always attended
 * ("稀疏注意力机制解析" explainer, §1.2), which gives the forced sets.
 *
 * scores: [rows, ld] float (the whole rows*ld buffer must be allocated), row r
 *   uses scores[r*ld + 0 .. n_r-1]; rows longer than 4096 candidates may also
 *   read, and ignore, up to 3 further entries of the same row.
 * Candidates of row r: 0 .. n_r-1 with
 *     n_r = causal ? min(ncand, (r % causal_period) + causal_offset + 1) : ncand
 * Forced (always kept, not counted in k): 0 .. min(n_sink,n_r)-1 and
 *     max(0, n_r-n_local) .. n_r-1.
 * Budget: k_r = (ratio_den > 0 ? ceil(ratio_num*n_r/ratio_den) : k), capped at
 *     the number of non-forced candidates.
 * Order: higher score first; equal scores -> lower index first; -0 == +0.
 * Output: idx [rows, kmax] int32 — the kept indices of row r ascending, padded
 *     with -1; cnt [rows] int32 — the number kept.  The host checks that the
 *     largest possible count fits kmax (SA_ERR_SHAPE otherwise).
 * err_flag: optional device int32; set to 1 when a candidate score is NaN
 *     (that row's output is then unspecified).  Never cleared by the library.
 * rows = 0 launches nothing (scores, idx and cnt may then be NULL).
 * Rows with up to 4096 candidates are ranked in LDS; rows with up to 131072
 * are read once (sampled bracket, LDS bitmaps); longer rows (up to 2^24) are
 * read twice, or more when the sample does not bracket the k-th score.
 * ====================================================================== */
typedef struct sa_select_args {
  const float* scores;
  int64_t rows;
  int64_t ncand;
  int64_t ld;
  int64_t causal_period;
  int64_t causal_offset;
  int32_t causal;
  int32_t n_sink;
  int32_t n_local;
  int32_t k;
  int32_t ratio_num;
  int32_t ratio_den;
  int32_t kmax;
  int32_t reserved0;
  int32_t* idx;
  int32_t* cnt;
  int32_t* err_flag;
} sa_select_args;

int sa_select_topk_workspace_bytes(const sa_select_args* args, size_t* bytes);
int sa_select_topk(const sa_select_args* args, void* workspace, size_t workspace_bytes, void* stream);

/* ======================================================================
 * sa_select_mass — adaptive budget: the fewest best-scored candidates that
 * hold a given share of the row's softmax weight.
 *
 * Squeezed Attention page, §技术方案 (key technical points): the number of
 * clusters kept adapts to the distribution of the query's centroid
 * similarities.  The page gives no rule; the one taken here treats a row's
 * scores as logits.  Candidate j weighs w_j = exp(s_j - m), m the row maximum
 * (an entry equal to m weighs exactly 1, so +inf entries share all the weight
 * and an all -inf row weighs uniformly).  Ranked in sa_select_topk's order
 * (higher score first, lower index on ties), the row keeps the shortest
 * prefix whose weight reaches mass * sum(w); that count is then clamped to
 * [k_min, k_max] and to ncand.  Weights are fp32 exponentials rounded to
 * multiples of 2^-40 and summed exactly as integers (the count does not depend
 * on the summation order); mass * sum is compared in double.
 *
 * scores: [rows, ld] float, row r uses scores[r*ld + 0 .. ncand-1];
 *   1 <= ncand <= 4096 (cluster tables), ld >= ncand.
 * mass in (0, 1]; 0 <= k_min <= k_max.
 * Output: idx [rows, kmax] int32 ascending, padded with -1 (kmax must be at
 *   least min(k_max, ncand), SA_ERR_SHAPE otherwise); cnt [rows] int32.
 * err_flag: optional device int32 set to 1 when a score is NaN (that row's
 *   output is then unspecified).  No workspace.  rows = 0 launches nothing
 *   (scores, idx and cnt may then be NULL).
 * ====================================================================== */
typedef struct sa_select_mass_args {
  const float* scores;
  int64_t rows;
  int64_t ncand;
  int64_t ld;
  float mass;
  int32_t k_min;
  int32_t k_max;
  int32_t kmax;
  int32_t* idx;
  int32_t* cnt;
  int32_t* err_flag;
} sa_select_mass_args;

int sa_select_mass(const sa_select_mass_args* args, void* stream);

/* ======================================================================
 * sa_estimate_topk — block estimate and selection in one call, without the
 * score matrix.
 *
 * "MInference 1.0" article, §方法介紹 (block indices from mean-pooled Q and K)
 * with the selection of sa_select_topk: the rule of sa_estimate(BLOCK_MEANPOOL)
 * followed by sa_select_topk on its score rows with causal = 1 and
 * causal_period = nb (row i of a head has the candidate blocks 0..i), with the
 * same n_sink / n_local / k or ratio budget, order and output format.  The
 * scores are never written to memory: a workgroup scores 16 consecutive rows,
 * keeps them in registers and selects from them.  Its pooled dot products are
 * summed in another order than sa_estimate's, so the two results are bit for
 * bit equal when every product and partial sum is exact in fp32 (e.g.
 * integer-valued inputs with scale 1); otherwise a row whose cut falls
 * between scores within fp32 rounding of each other may keep a different,
 * equally valid set.
 *
 * kind = SA_EST_BLOCK_MEANPOOL: q [B,Hq,N,d], k [B,Hkv,N,d] (F32 or BF16,
 * d = 64 or 128), N a multiple of 64 with N/64 <= 2048.
 * idx [B,n,nb,kmax] int32, cnt [B,n,nb] int32 (n = Hq, or n_heads_list with a
 * host head list as in sa_estimate); kmax must hold the largest count.
 * pooled_q / pooled_k: optional outputs as in sa_estimate.  Requires a
 * workspace unless both pooled buffers are given.
 *
 * kind = SA_EST_CENTROID (Squeezed Attention page, §技术方案: query-centroid
 * similarity, then the top-K clusters): equals sa_estimate(CENTROID) followed
 * by sa_select_topk with k and no forced members, bit for bit (the scores use
 * the same arithmetic).  q [T,Hq,d] (F32 or BF16; seq = T), k_ptr = the
 * centroid table [Hkv,C,d] float, n_centroids = C <= 1024, d <= 128, at most 8
 * query heads per KV head.  idx [T,Hq,kmax], cnt [T,Hq]; kmax >= min(k, C).
 * With mass > 0 (the adaptive budget, Squeezed Attention page, §技术方案),
 * the selection is sa_select_mass's instead, with k_max = k and k_min, bit for
 * bit: 0 < mass <= 1, 0 <= k_min <= k.
 * No workspace; head lists, ratios and forced members are not supported.
 *
 * err_flag: as in sa_select_topk.
 * ====================================================================== */
typedef struct sa_estimate_topk_args {
  int32_t kind;
  int32_t dtype;
  int64_t batch;
  int64_t heads_q;
  int64_t heads_kv;
  int64_t seq;
  int64_t head_dim;
  int32_t block_size;     /* 64 */
  float scale;
  int32_t n_sink;
  int32_t n_local;
  int32_t k;
  int32_t ratio_num;
  int32_t ratio_den;
  int32_t kmax;
  const void* q;
  const void* k_ptr;
  float* pooled_q;
  float* pooled_k;
  const int32_t* head_list;
  int32_t n_heads_list;
  int32_t n_centroids;    /* CENTROID */
  int32_t* idx;
  int32_t* cnt;
  int32_t* err_flag;
  float mass;             /* CENTROID: > 0 selects the adaptive budget */
  int32_t k_min;          /* CENTROID with mass */
} sa_estimate_topk_args;

int sa_estimate_topk_workspace_bytes(const sa_estimate_topk_args* args, size_t* bytes);
int sa_estimate_topk(const sa_estimate_topk_args* args, void* workspace, size_t workspace_bytes, void* stream);

/* ======================================================================
 * sa_vs_build — vertical-slash selections -> per-query-block key tables.
 *
 * "MInference 1.0" article, §延遲和內核中的稀疏模式, Fig. 4: vertical lines
 * are computed in 1x64 pieces and slash lines in 64x64 blocks.  Reading: the
 * slash at offset o covers, for query block i, the contiguous key tile
 * [64i-o, 64i-o+64) clipped at 0 (the square tile whose diagonal is the line).
 *
 * rows = B*Hq; vert [rows, n_vert] ascending column indices with vert_cnt
 * [rows]; slash [rows, n_slash] ascending offsets with slash_cnt [rows]
 * (the outputs of sa_select_topk).  For every row and query block i < N/64:
 *   iv  [rows, nqb, n_slash, 2]: the slash tiles united into disjoint
 *       intervals [start, end), ascending; iv_cnt [rows, nqb].
 *   col [rows, nqb, n_vert]: kept columns c <= 64i+63 outside those intervals,
 *       ascending; col_cnt [rows, nqb].
 * Counts are clipped to [0, n_vert] and [0, n_slash]; negative offsets and
 * columns outside [0, seq) are ignored.
 * ====================================================================== */
typedef struct sa_vs_build_args {
  int64_t rows;
  int64_t seq;
  int32_t block_size;     /* 64 */
  int32_t n_vert;
  int32_t n_slash;
  int32_t reserved0;
  const int32_t* vert;
  const int32_t* vert_cnt;
  const int32_t* slash;
  const int32_t* slash_cnt;
  int32_t* iv;
  int32_t* iv_cnt;
  int32_t* col;
  int32_t* col_cnt;
} sa_vs_build_args;

int sa_vs_build(const sa_vs_build_args* args, void* stream);

/* ======================================================================
 * sa_block_sparse_fwd — exact attention over the kept key sets.
 *
 * "MInference 1.0" article, §方法介紹 (block-sparse FlashAttention over the
 * estimated block indices) and §延遲和內核中的稀疏模式, Fig. 4 (vertical-slash
 * kernel).  FlashAttention tiling with an online softmax gives the exact
 * softmax over the union of the listed keys.
 *
 * q [B,Hq,N,d], k and v [B,Hkv,N,d]; dtype SA_BF16 (d = 64 or 128, bf16
 * matrix cores, fp32 accumulation) or SA_F32 (d = 64 or 128, fp32).
 * out [B,Hq,N,d] of out_dtype (SA_F32 or SA_BF16); lse [B,Hq,N] float,
 * optional (natural log of the softmax denominator, including the scale).
 * Row r of query block i attends key c only when c <= r (token-causal).
 * mode = SA_FWD_BLOCK: block_idx [B,Hq,nqb,kmax] ascending, -1 padded, and
 *   block_cnt [B,Hq,nqb]; keys = union of blocks [64j, 64j+64).
 *   Listed blocks outside 0 <= j <= i are skipped; block_cnt is clipped to
 *   [0, kmax].  bf16 inputs: kmax <= 2048.
 * mode = SA_FWD_VSLASH: the sa_vs_build tables (iv/iv_cnt with capacity
 *   max_iv, col/col_cnt with capacity max_col); keys = intervals ∪ columns.
 *   Counts are clipped to the capacities, intervals to [0, min(N, 64i+64)),
 *   and a column outside [0, N) is ignored, so no table entry can make the
 *   kernel read outside K and V.  bf16 inputs: max_iv <= 64, max_col <= 1920.
 * mode = SA_FWD_ASHAPE ("MInference 1.0" article, §方法介紹, the A-shape
 *   pattern; "稀疏注意力机制解析" explainer, §1.2, global plus local-window
 *   attention): no tables; query block i keeps blocks 0 .. n_sink-1 and the
 *   n_local blocks i-n_local+1 .. i (clipped at 0, each block once);
 *   n_sink + n_local <= 2048.
 * Head list ("MInference 1.0" article, §方法介紹: every head runs the pattern
 * assigned to it, so one layer mixes patterns by heads): head_list, when not
 * NULL, is a HOST array of n_heads_list distinct query-head indices in
 * [0, Hq) (at most 256; copied into the launch).  Only those heads are
 * computed; out and lse keep their full layouts (other heads untouched) while
 * the tables are compact, with row b*n + j for listed head j: block_idx
 * [B,n,nqb,kmax], block_cnt [B,n,nqb], and the VS tables [B*n, nqb, ...].
 * A row with no admissible key gets out = 0 and lse = -INFINITY.
 * ====================================================================== */
enum { SA_FWD_BLOCK = 0, SA_FWD_VSLASH = 1, SA_FWD_ASHAPE = 2 };

typedef struct sa_fwd_args {
  int32_t mode;
  int32_t dtype;
  int32_t out_dtype;
  int32_t block_size;     /* 64 */
  int64_t batch;
  int64_t heads_q;
  int64_t heads_kv;
  int64_t seq;
  int64_t head_dim;
  float scale;
  int32_t kmax;
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
  int32_t max_iv;
  int32_t max_col;
  int32_t n_sink;         /* ASHAPE */
  int32_t n_local;        /* ASHAPE */
  const int32_t* head_list; /* optional host array */
  int32_t n_heads_list;
  int32_t reserved1;
} sa_fwd_args;

int sa_block_sparse_fwd_workspace_bytes(const sa_fwd_args* args, size_t* bytes);
int sa_block_sparse_fwd(const sa_fwd_args* args, void* workspace, size_t workspace_bytes, void* stream);

/* ======================================================================
 * sa_gather_decode — exact attention over gathered keys.
 *
 * mode = SA_GATHER_CLUSTER (Squeezed Attention page, §技术方案: attention
 *   only over the key/value pairs of the selected clusters).
 *   q [T,Hq,d] BF16; k, v [Hkv,Nctx,d] BF16 in cluster-major order (as
 *   written by sa_cluster_pack); cluster_ptr [Hkv,C+1] int32 (cluster c of
 *   KV head g is rows cluster_ptr[g,c] .. cluster_ptr[g,c+1]-1); sel
 *   [T,Hq,n_sel] int32 cluster ids (duplicates count once; -1 ignored).
 *   T*Hq/Hkv (queries per KV head) must be <= 64.  No causal mask.
 * mode = SA_GATHER_TOKEN (IndexCache article, §长文本的算力困境 and
 *   §"偷懒"的艺术: attention over the indexer's token subset, which shared
 *   layers reuse from the nearest full layer — the index cache is simply the
 *   caller's tok_idx buffer passed to several layers).
 *   q [T,Hq,d] BF16; k, v [Hkv,Nctx,d] BF16 in context order; tok_idx
 *   [T,n_tok] int32 shared by every head of token t (tok_per_head = 0), or
 *   [T,Hq,n_tok] with one list per (token, query head) (tok_per_head = 1);
 *   ids distinct within a list, -1 padded (ids outside [0, Nctx) are padding).
 *   Shared lists with 16 query heads per KV head run the heads together on
 *   the matrix cores; other shapes take one wave per (token, head).
 * q_pos: optional device int32 [T]: query t attends only context positions
 *   <= q_pos[t] (a causal bound).  Token mode: the position is the id.
 *   Cluster mode: the position of packed row p of KV head g is perm[g,p]
 *   (sa_cluster_pack's perm, required with q_pos).  NULL: no bound.
 * d = 128.  out [T,Hq,d] (out_dtype F32 or BF16); lse [T,Hq] optional.  A
 * query with no admissible key gets out = 0 and lse = -INFINITY.
 * Cluster mode needs a workspace; token mode none.
 * ====================================================================== */
enum { SA_GATHER_CLUSTER = 0, SA_GATHER_TOKEN = 1 };

typedef struct sa_gather_args {
  int32_t mode;
  int32_t dtype;
  int32_t out_dtype;
  int32_t n_clusters;
  int64_t n_q;            /* T */
  int64_t heads_q;
  int64_t heads_kv;
  int64_t n_ctx;
  int64_t head_dim;
  float scale;
  int32_t n_sel;
  int32_t n_tok;
  int32_t tok_per_head;   /* TOKEN: 0 = tok_idx [T,n_tok], 1 = [T,Hq,n_tok] */
  const void* q;
  const void* k;
  const void* v;
  const int32_t* cluster_ptr;
  const int32_t* sel;
  const int32_t* tok_idx;
  void* out;
  float* lse;
  const int32_t* q_pos;   /* optional [T] causal bound */
  const int32_t* perm;    /* CLUSTER with q_pos: [Hkv,Nctx] */
} sa_gather_args;

int sa_gather_decode_workspace_bytes(const sa_gather_args* args, size_t* bytes);
int sa_gather_decode(const sa_gather_args* args, void* workspace, size_t workspace_bytes, void* stream);

/* ======================================================================
 * sa_gather_decode_static — sa_gather_decode that allocates nothing and takes
 * no workspace, for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 *
 * Same arguments, results and errors as sa_gather_decode (bit-identical
 * outputs).  The scratch the cluster mode needs (the per-range partials,
 * sa_gather_decode_workspace_bytes) lives in a static device array of
 * SA_STATIC_SCRATCH_BYTES that each GPU the library runs on holds until the
 * process ends; its address is looked up once per device, on the first call
 * with that device current.  A call needing more scratch returns
 * SA_ERR_UNSUPPORTED before any launch.  Every call on a GPU shares that GPU's
 * array: calls that overlap in time on one GPU (other streams or threads)
 * race, so the caller serialises them.  Nothing in the array needs clearing
 * between calls (each range's partial is written before it is read).
 * ====================================================================== */
#define SA_STATIC_SCRATCH_BYTES (32u << 20)
int sa_gather_decode_static(const sa_gather_args* args, void* stream);

/* ======================================================================
 * sa_cluster_pack — cluster-major layout of a fixed context (offline step).
 *
 * Squeezed Attention page, §技术方案, offline stage: keys are clustered and
 * each key gets an index to its cluster.  This call turns labels into the
 * cluster-major order the decode reads: a stable counting sort per KV head.
 * labels [Hkv,Nctx] int32 in [0,C) -> cluster_ptr [Hkv,C+1] int32 and perm
 * [Hkv,Nctx] int32 (perm[g,p] = context position of packed row p; token order
 * kept inside a cluster).  When k/v and k_packed/v_packed are all non-NULL
 * the rows are also copied: k_packed[g,p] = k[g,perm[g,p]] (same for v).
 * Labels outside [0,C) give SA_ERR_VALUE through err_flag semantics: the
 * optional err_flag device int32 is set to 1 and those tokens are dropped.
 * ====================================================================== */
typedef struct sa_cluster_pack_args {
  int64_t heads_kv;
  int64_t n_ctx;
  int64_t head_dim;
  int32_t n_clusters;
  int32_t dtype;          /* of k / v when copied */
  const int32_t* labels;
  int32_t* cluster_ptr;
  int32_t* perm;
  const void* k;
  const void* v;
  void* k_packed;
  void* v_packed;
  int32_t* err_flag;
} sa_cluster_pack_args;

int sa_cluster_pack_workspace_bytes(const sa_cluster_pack_args* args, size_t* bytes);
int sa_cluster_pack(const sa_cluster_pack_args* args, void* workspace, size_t workspace_bytes, void* stream);

/* ======================================================================
 * sa_kmeans — offline clustering of a fixed context's keys.
 *
 * Squeezed Attention page, §技术方案, offline stage: the keys are clustered,
 * each cluster gets a centroid and each key an index to its cluster.  Lloyd
 * iterations per KV head, `iters` times: assign every key to the centroid at
 * the smallest squared Euclidean distance (ties -> lower cluster index), then
 * move every centroid to the mean of its keys (a cluster with no key keeps its
 * centroid).  Distances are |mu|^2 - 2 k.mu in fp32 (the |k|^2 term is common
 * to all centroids of a key); means are fp32 sums in token order, so results
 * are deterministic.
 *
 * k [Hkv,N,d] (BF16 or F32, d = 64 or 128, 16-byte aligned).
 * centroids [Hkv,C,d] float: in, the initial table; out, the table after the
 *   last update (each non-empty cluster's centroid is the mean of its keys).
 * labels [Hkv,N] int32 out: the last assignment.
 * cluster_ptr [Hkv,C+1] and perm [Hkv,N] int32: optional outputs, the
 *   cluster-major order of the final labels exactly as sa_cluster_pack writes
 *   it (both or neither; when absent they live in the workspace).
 * 1 <= C <= 4096, iters >= 1.  Requires a workspace.
 * ====================================================================== */
typedef struct sa_kmeans_args {
  int64_t heads_kv;
  int64_t n_ctx;
  int64_t head_dim;
  int32_t n_clusters;
  int32_t iters;
  int32_t dtype;
  int32_t reserved0;
  const void* k;
  float* centroids;
  int32_t* labels;
  int32_t* cluster_ptr;
  int32_t* perm;
} sa_kmeans_args;

int sa_kmeans_workspace_bytes(const sa_kmeans_args* args, size_t* bytes);
int sa_kmeans(const sa_kmeans_args* args, void* workspace, size_t workspace_bytes, void* stream);

/* ======================================================================
 * sa_indexer_topk — indexer scores and the per-query top k in one call,
 * without the score matrix.
 *
 * IndexCache article, §长文本的算力困境: the indexer scores every causal key
 * for each query and its top-k keys are kept.  The result equals
 * sa_estimate(INDEXER) followed by sa_select_topk on its rows with k, no
 * forced members, causal = 1, causal_period = T and causal_offset = q_pos0
 * (row t keeps min(k, n_t) of its n_t = min(Nk, q_pos0 + t + 1) keys, higher
 * score first, lower index on ties, ascending, padded with -1).
 *
 * q [T,Hi,64] BF16, k [Nk,64] BF16, weights [Hi] float, as in
 * sa_estimate(INDEXER); Hi must be 32 or 64.  1 <= k <= 2048,
 * kmax >= min(k, Nk); idx [T,kmax] int32, cnt [T] int32.
 *
 * Method: a row of at most 8192 keys keeps all of them.  For a longer row
 * every 16th key is scored first and the query's threshold is the 256th
 * largest of its causal sampled scores (about 4096 of its keys reach it).
 * The full pass keeps only keys at or above the threshold, in per-chunk runs
 * of the workspace, and an exact radix select over the kept keys ends the
 * row.  When fewer than k keys reach the threshold, or a run overflows
 * (neither happens for scores without structure at the sampling period: k
 * lies 8 relative spreads below the expected count, the cap 16 above), the
 * row gets cnt = -1 and idx all -1, and bit 1 (value 2) of err_flag is set:
 * the caller recomputes such rows with the two-call path.
 * err_flag bit 0 (value 1): a NaN among the scores the method ranks, or a
 * NaN or infinite element of q, k or weights (the output is then
 * unspecified; the inputs are scanned only when err_flag is given).
 * err_flag is optional and never cleared by the library.
 *
 * Workspace: sa_indexer_topk_workspace_bytes (T * Nk/16 * 4 bytes of sampled
 * scores when some row exceeds 8192 keys, plus T * (8192 + 128 * Nk/8192) * 8
 * bytes of runs).  seq_q = 0 launches nothing.
 * ====================================================================== */
typedef struct sa_indexer_topk_args {
  int64_t seq_q;          /* T */
  int64_t seq_k;          /* Nk */
  int64_t q_pos0;         /* absolute position of query 0, >= 0 */
  int32_t heads;          /* Hi: 32 or 64 */
  int32_t head_dim;       /* 64 */
  int32_t k;
  int32_t kmax;
  const void* q;
  const void* k_ptr;
  const float* weights;
  int32_t* idx;
  int32_t* cnt;
  int32_t* err_flag;
} sa_indexer_topk_args;

int sa_indexer_topk_workspace_bytes(const sa_indexer_topk_args* args, size_t* bytes);
int sa_indexer_topk(const sa_indexer_topk_args* args, void* workspace, size_t workspace_bytes, void* stream);

/* ======================================================================
 * Library information.
 * ====================================================================== */
/* Message of the last failing call on this thread ("" if none). */
const char* sa_last_error(void);
/* SA_ABI_VERSION of the built library. */
int sa_version(void);
/* sizeof of the argument structs as compiled, so bindings can check layout:
 * which = 0 estimate, 1 select, 2 vs_build, 3 fwd, 4 gather, 5 cluster_pack,
 * 6 select_mass, 7 kmeans, 8 estimate_topk, 9 indexer_topk. */
size_t sa_args_size(int which);

#ifdef __cplusplus
}
#endif

#endif /* SA_H_ */
