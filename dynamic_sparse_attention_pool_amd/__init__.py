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
           "sa_gather_decode", "sa_gather_decode_static", "sa_cluster_pack", "sa_kmeans", "sa_estimate_topk", "sa_estimate_topk_centroid", "sa_indexer_topk", "SAError", "load", "BLOCK_MEANPOOL", "VSLASH", "CENTROID", "INDEXER"]

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


def _need(t, name, like=None, *, dtypes=None, shape=None, ndim=None, optional=False):
    """Check one tensor argument before any launch: present (unless
    optional), on the device of ``like``, of one of ``dtypes`` (names:
    "f32", "bf16", "i32"), of ``ndim`` dimensions and of ``shape`` (None
    entries are free).  Raises ValueError naming the argument."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    torch = _torch()
    if like is not None and t.device != like.device:
        raise ValueError(f"{name} is on {t.device}, expected {like.device}")
    if dtypes is not None:
        names = {torch.float32: "f32", torch.bfloat16: "bf16", torch.int32: "i32"}
        if names.get(t.dtype) not in dtypes:
            raise ValueError(f"{name} has dtype {t.dtype}, expected one of {sorted(dtypes)}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} has {t.dim()} dimensions, expected {ndim}")
    if shape is not None:
        if t.dim() != len(shape) or any(w is not None and int(g) != int(w) for g, w in zip(t.shape, shape)):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


FP = ("f32", "bf16")


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


def _ws(lib_bytes_fn, a, like, workspace):
    """Workspace for a call: the caller's when it is large enough, else a new
    torch buffer.  Returns (tensor or None, size passed to the library)."""
    nb = C.c_size_t(0)
    F.check(lib_bytes_fn(C.byref(a), C.byref(nb)))
    need = nb.value
    if need == 0:
        return workspace, 0
    if workspace is not None:
        _need(workspace, "workspace", like)
        if workspace.numel() * workspace.element_size() >= need:
            return workspace, workspace.numel() * workspace.element_size()
    ws, n = _workspace(need, like)
    return ws, n


def sa_estimate(kind: int, q, k, scores, *, scores2=None, centroids=None, weights=None, scale=None,
                block_size: int = 64, last_q: int = 64, q_pos0: int = 0, pooled_q=None, pooled_k=None,
                heads=None, err_flag=None, workspace=None):
    """Estimator scores (see sa.h).  Shapes:
    BLOCK_MEANPOOL / VSLASH: q [B,Hq,N,d], k [B,Hkv,N,d];
    CENTROID: q [T,Hq,d], centroids [Hkv,C,d]; INDEXER: q [T,Hi,di], k [Nk,di], weights [Hi].
    heads: optional sequence of query heads (BLOCK_MEANPOOL, VSLASH); outputs
    are then compact over the listed heads.  err_flag: optional int32 device
    flag (bit 0: a non-finite score).  workspace: a buffer from an earlier
    call, reused when large enough.  Returns the workspace used."""
    lib = load()
    a = F.EstimateArgs()
    a.kind = kind
    _need(q, "q", dtypes=FP)
    a.dtype = _dt(q)
    qt = ("bf16",) if a.dtype == F.SA_BF16 else ("f32",)
    nh = None
    if kind in (BLOCK_MEANPOOL, VSLASH):
        _need(q, "q", ndim=4)
        B, Hq, N, d = q.shape
        _need(k, "k", q, dtypes=qt, ndim=4, shape=(B, None, N, d))
        nh = Hq if heads is None else len(heads)
        a.batch, a.heads_q, a.heads_kv, a.seq_q, a.seq_k, a.head_dim = B, Hq, k.shape[1], N, k.shape[2], d
        if kind == BLOCK_MEANPOOL:
            nb = N // block_size
            _need(scores, "scores", q, dtypes=("f32",), shape=(B, nh, nb, nb))
            _need(pooled_q, "pooled_q", q, dtypes=("f32",), shape=(B, nh, nb, d), optional=True)
            _need(pooled_k, "pooled_k", q, dtypes=("f32",), shape=(B, k.shape[1], nb, d), optional=True)
        else:
            _need(scores, "scores", q, dtypes=("f32",), shape=(B, nh, N))
            _need(scores2, "scores2", q, dtypes=("f32",), shape=(B, nh, N))
    elif kind == CENTROID:
        _need(q, "q", ndim=3)
        T, Hq, d = q.shape
        _need(centroids, "centroids", q, dtypes=("f32",), ndim=3)
        _need(centroids, "centroids", shape=(None, None, d))
        _need(scores, "scores", q, dtypes=("f32",), shape=(T, Hq, centroids.shape[1]))
        a.batch, a.heads_q, a.heads_kv, a.seq_q, a.seq_k, a.head_dim = 1, Hq, centroids.shape[0], T, 1, d
        a.n_centroids = centroids.shape[1]
    elif kind == INDEXER:
        _need(q, "q", ndim=3)
        T, Hi, di = q.shape
        _need(k, "k", q, dtypes=qt, ndim=2)
        _need(k, "k", shape=(None, di))
        _need(weights, "weights", q, dtypes=("f32",), shape=(Hi,))
        _need(scores, "scores", q, dtypes=("f32",), shape=(T, k.shape[0]))
        a.batch, a.heads_q, a.heads_kv, a.seq_q, a.seq_k, a.head_dim = 1, Hi, 1, T, k.shape[0], di
        a.q_pos0 = q_pos0
    else:
        raise ValueError(kind)
    _need(err_flag, "err_flag", q, dtypes=("i32",), optional=True)
    a.block_size = block_size
    a.last_q = last_q
    a.scale = (1.0 / math.sqrt(a.head_dim)) if scale is None else scale
    a.q, a.k = _p(q), _p(k)
    a.centroids, a.weights = _p(centroids), _p(weights)
    a.scores, a.scores2 = _p(scores), _p(scores2)
    a.pooled_q, a.pooled_k = _p(pooled_q), _p(pooled_k)
    a.err_flag = _p(err_flag)
    keep = _heads(a, heads)  # noqa: F841  (the array must outlive the calls)
    ws, n = _ws(lib.sa_estimate_workspace_bytes, a, q, workspace)
    F.check(lib.sa_estimate(C.byref(a), _p(ws) if n else None, n, _stream()))
    return ws


def _select_outputs(scores, idx, cnt, err_flag):
    _need(scores, "scores", dtypes=("f32",), ndim=2)
    R = scores.shape[0]
    _need(idx, "idx", scores, dtypes=("i32",), ndim=2)
    _need(idx, "idx", shape=(R, None))
    _need(cnt, "cnt", scores, dtypes=("i32",), shape=(R,))
    _need(err_flag, "err_flag", scores, dtypes=("i32",), optional=True)


def sa_select_topk(scores, idx, cnt, *, k: int = 0, ratio=None, n_sink: int = 0, n_local: int = 0,
                   causal: bool = False, causal_period: int = 1, causal_offset: int = 0, ncand=None,
                   err_flag=None):
    """Row-wise top-k over scores [R, ld] float; idx [R, kmax], cnt [R] int32."""
    lib = load()
    _select_outputs(scores, idx, cnt, err_flag)
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
    _select_outputs(scores, idx, cnt, err_flag)
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
    _need(q, "q", dtypes=FP, ndim=4)
    B, Hq, N, d = q.shape
    nb, nh = N // 64, Hq if heads is None else len(heads)
    _need(k, "k", q, dtypes=("bf16",) if _dt(q) == F.SA_BF16 else ("f32",), shape=(B, None, N, d))
    _need(idx, "idx", q, dtypes=("i32",), shape=(B, nh, nb, None))
    _need(cnt, "cnt", q, dtypes=("i32",), shape=(B, nh, nb))
    _need(pooled_q, "pooled_q", q, dtypes=("f32",), shape=(B, nh, nb, d), optional=True)
    _need(pooled_k, "pooled_k", q, dtypes=("f32",), shape=(B, k.shape[1], nb, d), optional=True)
    _need(err_flag, "err_flag", q, dtypes=("i32",), optional=True)
    a = F.EstimateTopkArgs()
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
    ws, n = _ws(lib.sa_estimate_topk_workspace_bytes, a, q, workspace)
    F.check(lib.sa_estimate_topk(C.byref(a), _p(ws) if n else None, n, _stream()))
    return ws


def sa_estimate_topk_centroid(q, centroids, sel, cnt, *, k: int, scale=None, err_flag=None, mass=None,
                              k_min: int = 0):
    """Centroid scores and top-k clusters in one call: q [T,Hq,d],
    centroids [Hkv,C,d] float; sel [T,Hq,kmax], cnt [T,Hq] int32.  With
    ``mass``, the adaptive budget of sa_select_mass (k_min .. k clusters)."""
    lib = load()
    _need(q, "q", dtypes=FP, ndim=3)
    T, Hq, d = q.shape
    _need(centroids, "centroids", q, dtypes=("f32",), ndim=3)
    _need(centroids, "centroids", shape=(None, None, d))
    _need(sel, "sel", q, dtypes=("i32",), shape=(T, Hq, None))
    _need(cnt, "cnt", q, dtypes=("i32",), shape=(T, Hq))
    _need(err_flag, "err_flag", q, dtypes=("i32",), optional=True)
    a = F.EstimateTopkArgs()
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
    _need(qi, "qi", dtypes=("bf16",), ndim=3)
    T, Hi, di = qi.shape
    _need(ki, "ki", qi, dtypes=("bf16",), ndim=2)
    _need(ki, "ki", shape=(None, di))
    _need(weights, "weights", qi, dtypes=("f32",), shape=(Hi,))
    _need(idx, "idx", qi, dtypes=("i32",), shape=(T, None))
    _need(cnt, "cnt", qi, dtypes=("i32",), shape=(T,))
    _need(err_flag, "err_flag", qi, dtypes=("i32",), optional=True)
    a = F.IndexerTopkArgs()
    a.seq_q, a.seq_k, a.q_pos0 = T, ki.shape[0], q_pos0
    a.heads, a.head_dim, a.k, a.kmax = Hi, di, k, idx.shape[-1]
    a.q, a.k_ptr, a.weights = _p(qi), _p(ki), _p(weights)
    a.idx, a.cnt, a.err_flag = _p(idx), _p(cnt), _p(err_flag)
    ws, n = _ws(lib.sa_indexer_topk_workspace_bytes, a, qi, workspace)
    F.check(lib.sa_indexer_topk(C.byref(a), _p(ws) if n else None, n, _stream()))
    return ws


def sa_vs_build(vert, vert_cnt, slash, slash_cnt, iv, iv_cnt, col, col_cnt, seq: int, block_size: int = 64):
    """Per-query-block interval and column tables from vertical / slash selections."""
    lib = load()
    _need(vert, "vert", dtypes=("i32",), ndim=2)
    R, nv = vert.shape
    nqb = seq // block_size
    _need(vert_cnt, "vert_cnt", vert, dtypes=("i32",), shape=(R,))
    _need(slash, "slash", vert, dtypes=("i32",), shape=(R, None))
    ns = slash.shape[1]
    _need(slash_cnt, "slash_cnt", vert, dtypes=("i32",), shape=(R,))
    _need(iv, "iv", vert, dtypes=("i32",), shape=(R, nqb * ns * 2))
    _need(iv_cnt, "iv_cnt", vert, dtypes=("i32",), shape=(R, nqb))
    _need(col, "col", vert, dtypes=("i32",), shape=(R, nqb * nv))
    _need(col_cnt, "col_cnt", vert, dtypes=("i32",), shape=(R, nqb))
    a = F.VsBuildArgs()
    a.rows, a.seq, a.block_size = R, seq, block_size
    a.n_vert, a.n_slash = nv, ns
    a.vert, a.vert_cnt, a.slash, a.slash_cnt = _p(vert), _p(vert_cnt), _p(slash), _p(slash_cnt)
    a.iv, a.iv_cnt, a.col, a.col_cnt = _p(iv), _p(iv_cnt), _p(col), _p(col_cnt)
    F.check(lib.sa_vs_build(C.byref(a), _stream()))


def sa_block_sparse_fwd(q, k, v, out, *, block_idx=None, block_cnt=None, iv=None, iv_cnt=None, col=None,
                        col_cnt=None, ashape=None, lse=None, scale=None, block_size: int = 64, heads=None):
    """Sparse attention forward; q [B,Hq,N,d], k/v [B,Hkv,N,d], out [B,Hq,N,d].
    Keys from block tables, vertical-slash tables, or ashape=(n_sink, n_local)
    blocks; heads: optional sequence of query heads (tables compact over them)."""
    lib = load()
    _need(q, "q", dtypes=FP, ndim=4)
    B, Hq, N, d = q.shape
    qt = ("bf16",) if _dt(q) == F.SA_BF16 else ("f32",)
    _need(k, "k", q, dtypes=qt, shape=(B, None, N, d))
    _need(v, "v", q, dtypes=qt, shape=tuple(k.shape))
    _need(out, "out", q, dtypes=FP, shape=(B, Hq, N, d))
    _need(lse, "lse", q, dtypes=("f32",), shape=(B, Hq, N), optional=True)
    nh, nqb = (Hq if heads is None else len(heads)), N // block_size
    a = F.FwdArgs()
    if ashape is not None:
        a.mode = F.SA_FWD_ASHAPE
        a.n_sink, a.n_local = ashape
    else:
        a.mode = F.SA_FWD_BLOCK if block_idx is not None else F.SA_FWD_VSLASH
    if a.mode == F.SA_FWD_BLOCK:
        _need(block_idx, "block_idx", q, dtypes=("i32",), shape=(B, nh, nqb, None))
        _need(block_cnt, "block_cnt", q, dtypes=("i32",), shape=(B, nh, nqb))
    elif a.mode == F.SA_FWD_VSLASH:
        _need(iv, "iv", q, dtypes=("i32",), shape=(B, nh, nqb, None, 2))
        _need(iv_cnt, "iv_cnt", q, dtypes=("i32",), shape=(B, nh, nqb))
        _need(col, "col", q, dtypes=("i32",), shape=(B, nh, nqb, None))
        _need(col_cnt, "col_cnt", q, dtypes=("i32",), shape=(B, nh, nqb))
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


def _gather_args(q, k, v, out, cluster_ptr, sel, tok_idx, lse, scale, q_pos, perm):
    _need(q, "q", dtypes=("bf16",), ndim=3)
    T, Hq, d = q.shape
    _need(k, "k", q, dtypes=("bf16",), ndim=3)
    _need(k, "k", shape=(None, None, d))
    Hkv, Nctx = k.shape[0], k.shape[1]
    _need(v, "v", q, dtypes=("bf16",), shape=tuple(k.shape))
    _need(out, "out", q, dtypes=FP, shape=(T, Hq, d))
    _need(lse, "lse", q, dtypes=("f32",), shape=(T, Hq), optional=True)
    _need(q_pos, "q_pos", q, dtypes=("i32",), shape=(T,), optional=True)
    a = F.GatherArgs()
    a.mode = F.SA_GATHER_CLUSTER if sel is not None else F.SA_GATHER_TOKEN
    if a.mode == F.SA_GATHER_CLUSTER:
        _need(cluster_ptr, "cluster_ptr", q, dtypes=("i32",), ndim=2)
        _need(cluster_ptr, "cluster_ptr", shape=(Hkv, None))
        _need(sel, "sel", q, dtypes=("i32",), shape=(T, Hq, None))
        _need(perm, "perm", q, dtypes=("i32",), shape=(Hkv, Nctx), optional=q_pos is None)
        a.cluster_ptr, a.sel = _p(cluster_ptr), _p(sel)
        a.n_clusters, a.n_sel = cluster_ptr.shape[1] - 1, sel.shape[-1]
        a.perm = _p(perm)
    else:
        _need(tok_idx, "tok_idx", q, dtypes=("i32",))
        if tok_idx.dim() == 3:
            _need(tok_idx, "tok_idx", shape=(T, Hq, None))
            a.tok_per_head = 1
        else:
            _need(tok_idx, "tok_idx", shape=(T, None))
        a.tok_idx, a.n_tok = _p(tok_idx), tok_idx.shape[-1]
    a.dtype, a.out_dtype = _dt(q), _dt(out)
    a.n_q, a.heads_q, a.heads_kv, a.n_ctx, a.head_dim = T, Hq, Hkv, Nctx, d
    a.scale = (1.0 / math.sqrt(d)) if scale is None else scale
    a.q, a.k, a.v, a.out, a.lse = _p(q), _p(k), _p(v), _p(out), _p(lse)
    a.q_pos = _p(q_pos)
    return a


def sa_gather_decode(q, k, v, out, *, cluster_ptr=None, sel=None, tok_idx=None, lse=None, scale=None,
                     q_pos=None, perm=None, workspace=None):
    """Gathered attention: cluster mode (cluster_ptr + sel) or token mode
    (tok_idx [T,n_tok] shared by a token's heads, or [T,Hq,n_tok] per head).
    q [T,Hq,d], k/v [Hkv,Nctx,d], out [T,Hq,d].  q_pos: optional [T] int32
    causal bound (cluster mode then also needs perm [Hkv,Nctx] of the pack).
    Returns the workspace (reusable by later calls)."""
    lib = load()
    a = _gather_args(q, k, v, out, cluster_ptr, sel, tok_idx, lse, scale, q_pos, perm)
    ws, n = _ws(lib.sa_gather_decode_workspace_bytes, a, q, workspace)
    F.check(lib.sa_gather_decode(C.byref(a), _p(ws) if n else None, n, _stream()))
    return ws


def sa_gather_decode_static(q, k, v, out, *, cluster_ptr=None, sel=None, tok_idx=None, lse=None, scale=None,
                            q_pos=None, perm=None):
    """sa_gather_decode with its scratch in the library's static device array:
    no workspace and no allocation (usable under graph capture).  Calls that
    overlap on one GPU race; see sa.h."""
    lib = load()
    a = _gather_args(q, k, v, out, cluster_ptr, sel, tok_idx, lse, scale, q_pos, perm)
    F.check(lib.sa_gather_decode_static(C.byref(a), _stream()))


def sa_cluster_pack(labels, cluster_ptr, perm, n_clusters: int, *, k=None, v=None, k_packed=None,
                    v_packed=None, err_flag=None, workspace=None):
    """Stable cluster-major order of a fixed context; optionally copies K/V rows.
    Returns the workspace."""
    lib = load()
    _need(labels, "labels", dtypes=("i32",), ndim=2)
    Hkv, N = labels.shape
    _need(cluster_ptr, "cluster_ptr", labels, dtypes=("i32",), shape=(Hkv, n_clusters + 1))
    _need(perm, "perm", labels, dtypes=("i32",), shape=(Hkv, N))
    _need(err_flag, "err_flag", labels, dtypes=("i32",), optional=True)
    a = F.ClusterPackArgs()
    a.heads_kv, a.n_ctx, a.n_clusters = Hkv, N, n_clusters
    a.labels, a.cluster_ptr, a.perm = _p(labels), _p(cluster_ptr), _p(perm)
    if k is not None:
        _need(k, "k", labels, dtypes=FP, ndim=3)
        _need(k, "k", shape=(Hkv, N, None))
        for name, t in (("v", v), ("k_packed", k_packed), ("v_packed", v_packed)):
            _need(t, name, labels, dtypes=("bf16",) if _dt(k) == F.SA_BF16 else ("f32",), shape=tuple(k.shape))
        a.head_dim, a.dtype = k.shape[-1], _dt(k)
        a.k, a.v, a.k_packed, a.v_packed = _p(k), _p(v), _p(k_packed), _p(v_packed)
    a.err_flag = _p(err_flag)
    ws, n = _ws(lib.sa_cluster_pack_workspace_bytes, a, labels, workspace)
    F.check(lib.sa_cluster_pack(C.byref(a), _p(ws) if n else None, n, _stream()))
    return ws


def sa_kmeans(k, centroids, labels, *, iters: int, cluster_ptr=None, perm=None, workspace=None):
    """Lloyd iterations per KV head: k [Hkv,N,d], centroids [Hkv,C,d] float
    (in: initial, out: final), labels [Hkv,N] int32; optional cluster_ptr
    [Hkv,C+1] and perm [Hkv,N] of the final labels.  Returns the workspace."""
    lib = load()
    _need(k, "k", dtypes=FP, ndim=3)
    Hkv, N, d = k.shape
    _need(centroids, "centroids", k, dtypes=("f32",), shape=(Hkv, None, d))
    C_ = centroids.shape[1]
    _need(labels, "labels", k, dtypes=("i32",), shape=(Hkv, N))
    _need(cluster_ptr, "cluster_ptr", k, dtypes=("i32",), shape=(Hkv, C_ + 1), optional=True)
    _need(perm, "perm", k, dtypes=("i32",), shape=(Hkv, N), optional=True)
    a = F.KmeansArgs()
    a.heads_kv, a.n_ctx, a.head_dim, a.n_clusters, a.iters, a.dtype = Hkv, N, d, C_, iters, _dt(k)
    a.k, a.centroids, a.labels = _p(k), _p(centroids), _p(labels)
    a.cluster_ptr, a.perm = _p(cluster_ptr), _p(perm)
    ws, n = _ws(lib.sa_kmeans_workspace_bytes, a, k, workspace)
    F.check(lib.sa_kmeans(C.byref(a), _p(ws) if n else None, n, _stream()))
    return ws
