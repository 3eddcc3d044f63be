"""Dynamic sparse attention for AMD Instinct MI355X (gfx950).

Thin Python binding over the C ABI of libsa.so (include/sa.h).  The functions
below carry the C entry points' names; they only read shapes from torch
tensors, allocate the workspace the library asks for, and pass raw device
pointers plus torch's current HIP stream.  Every step of the computation runs
in libsa's HIP kernels; importing works without a GPU, calling needs one.
"""
from __future__ import annotations

import ctypes as C
import math

from . import _ffi as F
from ._ffi import SAError, load  # noqa: F401

__all__ = ["sa_estimate", "sa_select_topk", "sa_select_mass", "sa_vs_build", "sa_block_sparse_fwd",
           "sa_gather_decode", "sa_cluster_pack", "sa_kmeans", "sa_estimate_topk", "sa_estimate_topk_centroid", "sa_indexer_topk", "SAError", "load", "BLOCK_MEANPOOL", "VSLASH", "CENTROID", "INDEXER"]

BLOCK_MEANPOOL, VSLASH, CENTROID, INDEXER = (F.SA_EST_BLOCK_MEANPOOL, F.SA_EST_VSLASH, F.SA_EST_CENTROID,
                                             F.SA_EST_INDEXER)


def _torch():
    import torch
    return torch


def _dt(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return F.SA_F32
    if t.dtype == torch.bfloat16:
        return F.SA_BF16
    if t.dtype == torch.int32:
        return F.SA_I32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _p(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("libsa takes device tensors only")
    if not t.is_contiguous():
        raise ValueError("libsa takes contiguous tensors only")
    return t.data_ptr()


def _stream():
    return _torch().cuda.current_stream().cuda_stream


def _heads(a, heads):
    """Host head list -> (ctypes int32 array kept alive by the caller, count)."""
    if heads is None:
        return None
    arr = (C.c_int32 * len(heads))(*[int(h) for h in heads])
    a.head_list = C.cast(arr, C.c_void_p)
    a.n_heads_list = len(heads)
    return arr


def _workspace(nbytes: int, like):
    if nbytes == 0:
        return None, 0
    ws = _torch().empty(nbytes, dtype=_torch().uint8, device=like.device)
    return ws, nbytes


def sa_estimate(kind: int, q, k, scores, *, scores2=None, centroids=None, weights=None, scale=None,
                block_size: int = 64, last_q: int = 64, q_pos0: int = 0, pooled_q=None, pooled_k=None,
                heads=None):
    """Estimator scores (see sa.h).  Shapes:
    BLOCK_MEANPOOL / VSLASH: q [B,Hq,N,d], k [B,Hkv,N,d];
    CENTROID: q [T,Hq,d], centroids [Hkv,C,d]; INDEXER: q [T,Hi,di], k [Nk,di], weights [Hi].
    heads: optional sequence of query heads (BLOCK_MEANPOOL, VSLASH); outputs
    are then compact over the listed heads."""
    lib = load()
    a = F.EstimateArgs()
    a.kind = kind
    a.dtype = _dt(q)
    if kind in (BLOCK_MEANPOOL, VSLASH):
        B, Hq, N, d = q.shape
        a.batch, a.heads_q, a.heads_kv, a.seq_q, a.seq_k, a.head_dim = B, Hq, k.shape[1], N, k.shape[2], d
    elif kind == CENTROID:
        T, Hq, d = q.shape
        a.batch, a.heads_q, a.heads_kv, a.seq_q, a.seq_k, a.head_dim = 1, Hq, centroids.shape[0], T, 1, d
        a.n_centroids = centroids.shape[1]
    elif kind == INDEXER:
        T, Hi, di = q.shape
        a.batch, a.heads_q, a.heads_kv, a.seq_q, a.seq_k, a.head_dim = 1, Hi, 1, T, k.shape[0], di
        a.q_pos0 = q_pos0
    else:
        raise ValueError(kind)
    a.block_size = block_size
    a.last_q = last_q
    a.scale = (1.0 / math.sqrt(a.head_dim)) if scale is None else scale
    a.q, a.k = _p(q), _p(k)
    a.centroids, a.weights = _p(centroids), _p(weights)
    a.scores, a.scores2 = _p(scores), _p(scores2)
    a.pooled_q, a.pooled_k = _p(pooled_q), _p(pooled_k)
    keep = _heads(a, heads)  # noqa: F841  (the array must outlive the calls)
    nb = C.c_size_t(0)
    F.check(lib.sa_estimate_workspace_bytes(C.byref(a), C.byref(nb)))
    ws, n = _workspace(nb.value, q)
    F.check(lib.sa_estimate(C.byref(a), _p(ws), n, _stream()))
    return ws


def sa_select_topk(scores, idx, cnt, *, k: int = 0, ratio=None, n_sink: int = 0, n_local: int = 0,
                   causal: bool = False, causal_period: int = 1, causal_offset: int = 0, ncand=None,
                   err_flag=None):
    """Row-wise top-k over scores [R, ld] float; idx [R, kmax], cnt [R] int32."""
    lib = load()
    a = F.SelectArgs()
    R, ld = scores.shape
    a.scores, a.rows, a.ld = _p(scores), R, ld
    a.ncand = ld if ncand is None else ncand
    a.causal, a.causal_period, a.causal_offset = int(causal), causal_period, causal_offset
    a.n_sink, a.n_local = n_sink, n_local
    if ratio is not None:
        a.ratio_num, a.ratio_den = ratio
    else:
        a.k = k
    a.kmax = idx.shape[1]
    a.idx, a.cnt, a.err_flag = _p(idx), _p(cnt), _p(err_flag)
    F.check(lib.sa_select_topk(C.byref(a), None, 0, _stream()))


def sa_select_mass(scores, idx, cnt, *, mass: float, k_min: int = 0, k_max=None, ncand=None, err_flag=None):
    """Adaptive count per row: the fewest best-scored candidates holding
    ``mass`` of the row's softmax weight, clamped to [k_min, k_max].
    scores [R, ld] float; idx [R, kmax], cnt [R] int32."""
    lib = load()
    a = F.SelectMassArgs()
    R, ld = scores.shape
    a.scores, a.rows, a.ld = _p(scores), R, ld
    a.ncand = ld if ncand is None else ncand
    a.mass, a.k_min = mass, k_min
    a.k_max = idx.shape[1] if k_max is None else k_max
    a.kmax = idx.shape[1]
    a.idx, a.cnt, a.err_flag = _p(idx), _p(cnt), _p(err_flag)
    F.check(lib.sa_select_mass(C.byref(a), _stream()))


def sa_estimate_topk(q, k, idx, cnt, *, n_sink: int = 0, n_local: int = 0, k_fixed: int = 0, ratio=None,
                     scale=None, pooled_q=None, pooled_k=None, heads=None, err_flag=None, workspace=None):
    """Block-sparse estimate and per-row top-k in one call (no score matrix):
    q [B,Hq,N,d], k [B,Hkv,N,d]; idx [B,n,nb,kmax], cnt [B,n,nb] int32.
    Returns the workspace (reusable by later calls of the same shape)."""
    lib = load()
    a = F.EstimateTopkArgs()
    B, Hq, N, d = q.shape
    a.kind, a.dtype, a.block_size = F.SA_EST_BLOCK_MEANPOOL, _dt(q), 64
    a.batch, a.heads_q, a.heads_kv, a.seq, a.head_dim = B, Hq, k.shape[1], N, d
    a.scale = (1.0 / math.sqrt(d)) if scale is None else scale
    a.n_sink, a.n_local = n_sink, n_local
    if ratio is not None:
        a.ratio_num, a.ratio_den = ratio
    else:
        a.k = k_fixed
    a.kmax = idx.shape[-1]
    a.q, a.k_ptr = _p(q), _p(k)
    a.pooled_q, a.pooled_k = _p(pooled_q), _p(pooled_k)
    a.idx, a.cnt, a.err_flag = _p(idx), _p(cnt), _p(err_flag)
    keep = _heads(a, heads)  # noqa: F841
    nb = C.c_size_t(0)
    F.check(lib.sa_estimate_topk_workspace_bytes(C.byref(a), C.byref(nb)))
    if nb.value and (workspace is None or workspace.numel() < nb.value):
        workspace, _ = _workspace(nb.value, q)
    F.check(lib.sa_estimate_topk(C.byref(a), _p(workspace) if nb.value else None, nb.value, _stream()))
    return workspace


def sa_estimate_topk_centroid(q, centroids, sel, cnt, *, k: int, scale=None, err_flag=None, mass=None,
                              k_min: int = 0):
    """Centroid scores and top-k clusters in one call: q [T,Hq,d],
    centroids [Hkv,C,d] float; sel [T,Hq,kmax], cnt [T,Hq] int32.  With
    ``mass``, the adaptive budget of sa_select_mass (k_min .. k clusters)."""
    lib = load()
    a = F.EstimateTopkArgs()
    T, Hq, d = q.shape
    a.kind, a.dtype = F.SA_EST_CENTROID, _dt(q)
    a.batch, a.heads_q, a.heads_kv, a.seq, a.head_dim = 1, Hq, centroids.shape[0], T, d
    a.n_centroids = centroids.shape[1]
    a.scale = (1.0 / math.sqrt(d)) if scale is None else scale
    a.k, a.kmax = k, sel.shape[-1]
    a.q, a.k_ptr = _p(q), _p(centroids)
    a.idx, a.cnt, a.err_flag = _p(sel), _p(cnt), _p(err_flag)
    if mass is not None:
        a.mass, a.k_min = mass, k_min
    F.check(lib.sa_estimate_topk(C.byref(a), None, 0, _stream()))


def sa_indexer_topk(qi, ki, idx, cnt, *, weights, q_pos0: int, k: int, err_flag=None, workspace=None):
    """Indexer scores and each query's top-k causal keys in one call (no score
    matrix): qi [T,Hi,64], ki [Nk,64] bf16, weights [Hi] float; idx [T,kmax],
    cnt [T] int32.  Rows whose sampled threshold does not hold get cnt = -1
    (and value 2 in err_flag).  Returns the workspace."""
    lib = load()
    a = F.IndexerTopkArgs()
    T, Hi, di = qi.shape
    a.seq_q, a.seq_k, a.q_pos0 = T, ki.shape[0], q_pos0
    a.heads, a.head_dim, a.k, a.kmax = Hi, di, k, idx.shape[-1]
    a.q, a.k_ptr, a.weights = _p(qi), _p(ki), _p(weights)
    a.idx, a.cnt, a.err_flag = _p(idx), _p(cnt), _p(err_flag)
    nb = C.c_size_t(0)
    F.check(lib.sa_indexer_topk_workspace_bytes(C.byref(a), C.byref(nb)))
    if nb.value and (workspace is None or workspace.numel() < nb.value):
        workspace, _ = _workspace(nb.value, qi)
    F.check(lib.sa_indexer_topk(C.byref(a), _p(workspace) if nb.value else None, nb.value, _stream()))
    return workspace


def sa_vs_build(vert, vert_cnt, slash, slash_cnt, iv, iv_cnt, col, col_cnt, seq: int, block_size: int = 64):
    """Per-query-block interval and column tables from vertical / slash selections."""
    lib = load()
    a = F.VsBuildArgs()
    a.rows, a.seq, a.block_size = vert.shape[0], seq, block_size
    a.n_vert, a.n_slash = vert.shape[1], slash.shape[1]
    a.vert, a.vert_cnt, a.slash, a.slash_cnt = _p(vert), _p(vert_cnt), _p(slash), _p(slash_cnt)
    a.iv, a.iv_cnt, a.col, a.col_cnt = _p(iv), _p(iv_cnt), _p(col), _p(col_cnt)
    F.check(lib.sa_vs_build(C.byref(a), _stream()))


def sa_block_sparse_fwd(q, k, v, out, *, block_idx=None, block_cnt=None, iv=None, iv_cnt=None, col=None,
                        col_cnt=None, ashape=None, lse=None, scale=None, block_size: int = 64, heads=None):
    """Sparse attention forward; q [B,Hq,N,d], k/v [B,Hkv,N,d], out [B,Hq,N,d].
    Keys from block tables, vertical-slash tables, or ashape=(n_sink, n_local)
    blocks; heads: optional sequence of query heads (tables compact over them)."""
    lib = load()
    a = F.FwdArgs()
    B, Hq, N, d = q.shape
    if ashape is not None:
        a.mode = F.SA_FWD_ASHAPE
        a.n_sink, a.n_local = ashape
    else:
        a.mode = F.SA_FWD_BLOCK if block_idx is not None else F.SA_FWD_VSLASH
    a.dtype, a.out_dtype, a.block_size = _dt(q), _dt(out), block_size
    a.batch, a.heads_q, a.heads_kv, a.seq, a.head_dim = B, Hq, k.shape[1], N, d
    a.scale = (1.0 / math.sqrt(d)) if scale is None else scale
    a.q, a.k, a.v, a.out, a.lse = _p(q), _p(k), _p(v), _p(out), _p(lse)
    if a.mode == F.SA_FWD_BLOCK:
        a.block_idx, a.block_cnt, a.kmax = _p(block_idx), _p(block_cnt), block_idx.shape[-1]
    elif a.mode == F.SA_FWD_VSLASH:
        a.iv, a.iv_cnt, a.col, a.col_cnt = _p(iv), _p(iv_cnt), _p(col), _p(col_cnt)
        a.max_iv, a.max_col = iv.shape[-2], col.shape[-1]
    keep = _heads(a, heads)  # noqa: F841
    F.check(lib.sa_block_sparse_fwd(C.byref(a), None, 0, _stream()))


def sa_gather_decode(q, k, v, out, *, cluster_ptr=None, sel=None, tok_idx=None, lse=None, scale=None,
                     workspace=None):
    """Gathered attention: cluster mode (cluster_ptr + sel) or token mode (tok_idx).
    q [T,Hq,d], k/v [Hkv,Nctx,d], out [T,Hq,d]."""
    lib = load()
    a = F.GatherArgs()
    T, Hq, d = q.shape
    a.mode = F.SA_GATHER_CLUSTER if sel is not None else F.SA_GATHER_TOKEN
    a.dtype, a.out_dtype = _dt(q), _dt(out)
    a.n_q, a.heads_q, a.heads_kv, a.n_ctx, a.head_dim = T, Hq, k.shape[0], k.shape[1], d
    a.scale = (1.0 / math.sqrt(d)) if scale is None else scale
    a.q, a.k, a.v, a.out, a.lse = _p(q), _p(k), _p(v), _p(out), _p(lse)
    if sel is not None:
        a.cluster_ptr, a.sel = _p(cluster_ptr), _p(sel)
        a.n_clusters, a.n_sel = cluster_ptr.shape[1] - 1, sel.shape[-1]
    else:
        a.tok_idx, a.n_tok = _p(tok_idx), tok_idx.shape[-1]
    nb = C.c_size_t(0)
    F.check(lib.sa_gather_decode_workspace_bytes(C.byref(a), C.byref(nb)))
    if workspace is None or workspace.numel() < nb.value:
        workspace, _ = _workspace(nb.value, q)
    F.check(lib.sa_gather_decode(C.byref(a), _p(workspace), 0 if workspace is None else workspace.numel(),
                                 _stream()))
    return workspace


def sa_cluster_pack(labels, cluster_ptr, perm, n_clusters: int, *, k=None, v=None, k_packed=None,
                    v_packed=None, err_flag=None):
    """Stable cluster-major order of a fixed context; optionally copies K/V rows."""
    lib = load()
    a = F.ClusterPackArgs()
    Hkv, N = labels.shape
    a.heads_kv, a.n_ctx, a.n_clusters = Hkv, N, n_clusters
    a.labels, a.cluster_ptr, a.perm = _p(labels), _p(cluster_ptr), _p(perm)
    if k is not None:
        a.head_dim, a.dtype = k.shape[-1], _dt(k)
        a.k, a.v, a.k_packed, a.v_packed = _p(k), _p(v), _p(k_packed), _p(v_packed)
    a.err_flag = _p(err_flag)
    nb = C.c_size_t(0)
    F.check(lib.sa_cluster_pack_workspace_bytes(C.byref(a), C.byref(nb)))
    ws, n = _workspace(nb.value, labels)
    F.check(lib.sa_cluster_pack(C.byref(a), _p(ws), n, _stream()))
    return ws


def sa_kmeans(k, centroids, labels, *, iters: int, cluster_ptr=None, perm=None, workspace=None):
    """Lloyd iterations per KV head: k [Hkv,N,d], centroids [Hkv,C,d] float
    (in: initial, out: final), labels [Hkv,N] int32; optional cluster_ptr
    [Hkv,C+1] and perm [Hkv,N] of the final labels.  Returns the workspace."""
    lib = load()
    a = F.KmeansArgs()
    Hkv, N, d = k.shape
    a.heads_kv, a.n_ctx, a.head_dim, a.n_clusters, a.iters, a.dtype = Hkv, N, d, centroids.shape[1], iters, _dt(k)
    a.k, a.centroids, a.labels = _p(k), _p(centroids), _p(labels)
    a.cluster_ptr, a.perm = _p(cluster_ptr), _p(perm)
    nb = C.c_size_t(0)
    F.check(lib.sa_kmeans_workspace_bytes(C.byref(a), C.byref(nb)))
    if workspace is None or workspace.numel() < nb.value:
        workspace, _ = _workspace(nb.value, k)
    F.check(lib.sa_kmeans(C.byref(a), _p(workspace), nb.value, _stream()))
    return workspace
