"""Chained calls of the libsa entry points for the workload families.

Each class allocates its device buffers once (torch is the allocator) and
exposes the steps of its path as methods that only enqueue libsa calls on
torch's current stream.  No arithmetic happens here.
"""
from __future__ import annotations

import math

from . import (BLOCK_MEANPOOL, CENTROID, INDEXER, VSLASH, sa_block_sparse_fwd, sa_cluster_pack, sa_estimate,
               sa_estimate_topk, sa_estimate_topk_centroid, sa_gather_decode, sa_indexer_topk, sa_select_mass,
               sa_select_topk, sa_vs_build)


def _t():
    import torch
    return torch


def max_kept_blocks(nb: int, n_sink: int, n_local: int, k=None, ratio=None) -> int:
    """Capacity of a block table row: forced members plus the largest budget."""
    best = 0
    for i in range(nb):
        n = i + 1
        forced = len(set(range(min(n_sink, n))) | set(range(max(0, n - n_local), n)))
        kb = k if ratio is None else -((-ratio[0] * n) // ratio[1])
        best = max(best, forced + max(0, min(kb, n - forced)))
    return best


def _out_buffers(q, out_dtype, with_lse, out=None, lse=None):
    torch = _t()
    B, Hq, N, _ = q.shape
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or q.dtype, device=q.device)
    if lse is None and with_lse:
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    return out, lse


class BlockSparseLayer:
    """Block-sparse prefill: pooled estimate -> top-k with sink/local -> forward.
    ``heads`` restricts the layer to those query heads (tables compact over
    them); ``out``/``lse`` may be shared with other layers of the same heads'
    tensor.  ``fused``: estimate and select in one call that never writes the
    score matrix (sa_estimate_topk); ``estimate`` then does both and
    ``select`` nothing."""

    def __init__(self, q, k, v, *, n_sink: int, n_local: int, ratio=None, k_fixed=None, out_dtype=None,
                 scale=None, with_lse=False, heads=None, out=None, lse=None, fused=False):
        torch = _t()
        self.q, self.k, self.v = q, k, v
        B, Hq, N, d = q.shape
        self.heads = None if heads is None else [int(h) for h in heads]
        nh = Hq if heads is None else len(self.heads)
        self.nb = N // 64
        self.scale = 1.0 / math.sqrt(d) if scale is None else scale
        self.n_sink, self.n_local, self.ratio, self.k_fixed = n_sink, n_local, ratio, k_fixed
        self.kmax = max_kept_blocks(self.nb, n_sink, n_local, k_fixed, ratio)
        dev = q.device
        self.fused = fused
        self.scores = None if fused else torch.empty((B, nh, self.nb, self.nb), dtype=torch.float32, device=dev)
        self.pooled_q = torch.empty((B, nh, self.nb, d), dtype=torch.float32, device=dev)
        self.pooled_k = torch.empty((B, k.shape[1], self.nb, d), dtype=torch.float32, device=dev)
        self.idx = torch.empty((B, nh, self.nb, self.kmax), dtype=torch.int32, device=dev)
        self.cnt = torch.empty((B, nh, self.nb), dtype=torch.int32, device=dev)
        self.out, self.lse = _out_buffers(q, out_dtype, with_lse, out, lse)
        self.err = torch.zeros(1, dtype=torch.int32, device=dev)

    def estimate(self):
        if self.fused:
            budget = dict(ratio=self.ratio) if self.ratio is not None else dict(k_fixed=self.k_fixed)
            sa_estimate_topk(self.q, self.k, self.idx, self.cnt, n_sink=self.n_sink, n_local=self.n_local,
                             scale=self.scale, pooled_q=self.pooled_q, pooled_k=self.pooled_k, heads=self.heads,
                             err_flag=self.err, **budget)
            return
        sa_estimate(BLOCK_MEANPOOL, self.q, self.k, self.scores, scale=self.scale, pooled_q=self.pooled_q,
                    pooled_k=self.pooled_k, heads=self.heads, err_flag=self.err)

    def select(self):
        if self.fused:
            return
        kw = dict(n_sink=self.n_sink, n_local=self.n_local, causal=True, causal_period=self.nb,
                  err_flag=self.err)
        if self.ratio is not None:
            kw["ratio"] = self.ratio
        else:
            kw["k"] = self.k_fixed
        sa_select_topk(self.scores.view(-1, self.nb), self.idx.view(-1, self.kmax), self.cnt.view(-1), **kw)

    def forward(self):
        sa_block_sparse_fwd(self.q, self.k, self.v, self.out, block_idx=self.idx, block_cnt=self.cnt,
                            lse=self.lse, scale=self.scale, heads=self.heads)

    def step(self):
        self.estimate()
        self.select()
        self.forward()


class VerticalSlashLayer:
    """Vertical-slash prefill: last-64-query estimate -> top columns and top
    offsets -> per-block tables -> forward."""

    def __init__(self, q, k, v, *, n_vert: int, n_slash: int, out_dtype=None, scale=None, with_lse=False,
                 heads=None, out=None, lse=None):
        torch = _t()
        self.q, self.k, self.v = q, k, v
        B, Hq, N, d = q.shape
        self.heads = None if heads is None else [int(h) for h in heads]
        nh = Hq if heads is None else len(self.heads)
        self.N, self.R = N, B * nh
        self.nb = N // 64
        self.scale = 1.0 / math.sqrt(d) if scale is None else scale
        self.n_vert, self.n_slash = min(n_vert, N), min(n_slash, N)
        dev = q.device
        self.a_v = torch.empty((B, nh, N), dtype=torch.float32, device=dev)
        self.a_s = torch.empty((B, nh, N), dtype=torch.float32, device=dev)
        self.vert = torch.empty((self.R, self.n_vert), dtype=torch.int32, device=dev)
        self.vert_cnt = torch.empty(self.R, dtype=torch.int32, device=dev)
        self.slash = torch.empty((self.R, self.n_slash), dtype=torch.int32, device=dev)
        self.slash_cnt = torch.empty(self.R, dtype=torch.int32, device=dev)
        self.iv = torch.empty((B, nh, self.nb, self.n_slash, 2), dtype=torch.int32, device=dev)
        self.iv_cnt = torch.empty((B, nh, self.nb), dtype=torch.int32, device=dev)
        self.col = torch.empty((B, nh, self.nb, self.n_vert), dtype=torch.int32, device=dev)
        self.col_cnt = torch.empty((B, nh, self.nb), dtype=torch.int32, device=dev)
        self.out, self.lse = _out_buffers(q, out_dtype, with_lse, out, lse)
        self.ws = None
        self.side = torch.cuda.Stream(device=dev)  # default priority

    def estimate(self):
        self.ws = sa_estimate(VSLASH, self.q, self.k, self.a_v, scores2=self.a_s, scale=self.scale,
                              heads=self.heads, workspace=self.ws)

    def select(self):
        # the two selections run side by side: each has one workgroup per row,
        # too few to fill the GPU alone
        torch = _t()
        cur = torch.cuda.current_stream(self.a_v.device)
        self.side.wait_stream(cur)
        with torch.cuda.stream(self.side):
            sa_select_topk(self.a_s.view(self.R, self.N), self.slash, self.slash_cnt, k=self.n_slash)
        sa_select_topk(self.a_v.view(self.R, self.N), self.vert, self.vert_cnt, k=self.n_vert)
        cur.wait_stream(self.side)
        sa_vs_build(self.vert, self.vert_cnt, self.slash, self.slash_cnt, self.iv.view(self.R, -1),
                    self.iv_cnt.view(self.R, -1), self.col.view(self.R, -1), self.col_cnt.view(self.R, -1),
                    seq=self.N)

    def forward(self):
        sa_block_sparse_fwd(self.q, self.k, self.v, self.out, iv=self.iv, iv_cnt=self.iv_cnt, col=self.col,
                            col_cnt=self.col_cnt, lse=self.lse, scale=self.scale, heads=self.heads)

    def step(self):
        self.estimate()
        self.select()
        self.forward()


class AShapeLayer:
    """A-shape prefill: sink blocks plus a local window of blocks, no estimate."""

    def __init__(self, q, k, v, *, n_sink: int, n_local: int, out_dtype=None, scale=None, with_lse=False,
                 heads=None, out=None, lse=None):
        self.q, self.k, self.v = q, k, v
        self.heads = None if heads is None else [int(h) for h in heads]
        self.n_sink, self.n_local = n_sink, n_local
        self.scale = 1.0 / math.sqrt(q.shape[-1]) if scale is None else scale
        self.out, self.lse = _out_buffers(q, out_dtype, with_lse, out, lse)

    def estimate(self):
        pass

    def select(self):
        pass

    def forward(self):
        sa_block_sparse_fwd(self.q, self.k, self.v, self.out, ashape=(self.n_sink, self.n_local), lse=self.lse,
                            scale=self.scale, heads=self.heads)

    def step(self):
        self.forward()


class MixedPatternLayer:
    """One prefill layer whose query heads follow different patterns, from a
    given head -> pattern assignment ("A", "VS" or "BS").  Each pattern's heads
    run as one group: its estimate, selection and forward launch cover only
    those heads, writing into the shared output."""

    def __init__(self, q, k, v, patterns, *, a_shape=(1, 4), block=None, vslash=None, out_dtype=None,
                 scale=None, with_lse=False):
        Hq = q.shape[1]
        if len(patterns) != Hq:
            raise ValueError("one pattern per query head")
        self.out, self.lse = _out_buffers(q, out_dtype, with_lse)
        groups = {p: [h for h in range(Hq) if patterns[h] == p] for p in ("A", "VS", "BS")}
        unknown = set(patterns) - set(groups)
        if unknown:
            raise ValueError(f"unknown patterns {sorted(unknown)}")
        share = dict(out=self.out, lse=self.lse, scale=scale)
        self.parts = []
        if groups["BS"]:
            self.parts.append(BlockSparseLayer(q, k, v, heads=groups["BS"], **(block or {}), **share))
        if groups["VS"]:
            n_vert, n_slash = vslash
            self.parts.append(VerticalSlashLayer(q, k, v, n_vert=n_vert, n_slash=n_slash, heads=groups["VS"],
                                                 **share))
        if groups["A"]:
            self.parts.append(AShapeLayer(q, k, v, n_sink=a_shape[0], n_local=a_shape[1], heads=groups["A"],
                                          **share))
        self.groups = groups

    def estimate(self):
        for p in self.parts:
            p.estimate()

    def select(self):
        for p in self.parts:
            p.select()

    def forward(self):
        for p in self.parts:
            p.forward()

    def step(self):
        self.estimate()
        self.select()
        self.forward()


class ClusterDecode:
    """Clustered fixed-context decode: offline pack, then per step
    centroid scores -> top clusters -> gathered attention."""

    def __init__(self, q, k, v, labels, centroids, *, n_sel: int, mass=None, k_min: int = 1, out_dtype=None,
                 scale=None, with_lse=False, fused=False):
        """n_sel clusters per query head, or, with ``mass`` set, the fewest
        clusters holding that share of the softmax of the centroid scores,
        between k_min and n_sel (sa_select_mass).  ``fused``: scores and the
        selection in one call, ``estimate`` doing both."""
        torch = _t()
        T, Hq, d = q.shape
        Hkv, N, _ = k.shape
        C = centroids.shape[1]
        dev = q.device
        self.q, self.centroids, self.C, self.n_sel = q, centroids, C, n_sel
        self.mass, self.k_min = mass, k_min
        self.fused = fused
        self.scale = 1.0 / math.sqrt(d) if scale is None else scale
        self.ptr = torch.empty((Hkv, C + 1), dtype=torch.int32, device=dev)
        self.perm = torch.empty((Hkv, N), dtype=torch.int32, device=dev)
        self.k = torch.empty_like(k)
        self.v = torch.empty_like(v)
        self.err = torch.zeros(1, dtype=torch.int32, device=dev)
        sa_cluster_pack(labels, self.ptr, self.perm, C, k=k, v=v, k_packed=self.k, v_packed=self.v,
                        err_flag=self.err)
        self.scores = torch.empty((T, Hq, C), dtype=torch.float32, device=dev)
        self.sel = torch.empty((T, Hq, n_sel), dtype=torch.int32, device=dev)
        self.sel_cnt = torch.empty(T * Hq, dtype=torch.int32, device=dev)
        self.out = torch.empty((T, Hq, d), dtype=out_dtype or torch.float32, device=dev)
        self.lse = torch.empty((T, Hq), dtype=torch.float32, device=dev) if with_lse else None
        self.ws = None

    def estimate(self):
        if self.fused:
            sa_estimate_topk_centroid(self.q, self.centroids, self.sel, self.sel_cnt.view(self.sel.shape[0], -1),
                                      k=self.n_sel, scale=self.scale, mass=self.mass, k_min=self.k_min,
                                      err_flag=self.err)
            return
        sa_estimate(CENTROID, self.q, self.k, self.scores, centroids=self.centroids, scale=self.scale)

    def select(self):
        if self.fused:
            return
        if self.mass is None:
            sa_select_topk(self.scores.view(-1, self.C), self.sel.view(-1, self.n_sel), self.sel_cnt, k=self.n_sel)
        else:
            sa_select_mass(self.scores.view(-1, self.C), self.sel.view(-1, self.n_sel), self.sel_cnt, mass=self.mass,
                           k_min=self.k_min, k_max=self.n_sel)

    def forward(self):
        self.ws = sa_gather_decode(self.q, self.k, self.v, self.out, cluster_ptr=self.ptr, sel=self.sel,
                                   lse=self.lse, scale=self.scale, workspace=self.ws)

    def step(self):
        self.estimate()
        self.select()
        self.forward()


class IndexerPrefill:
    """Token-level sparse prefill with a shared-layer index cache: the full
    layer runs the indexer and top-k and stores the indices; the shared layers
    attend through the same index buffer."""

    def __init__(self, qi, ki, w, pos0: int, layers, *, k_sel: int, full_layers=(0,), out_dtype=None,
                 scale=None, fused: bool = False):
        torch = _t()
        T = qi.shape[0]
        N = ki.shape[0]
        dev = qi.device
        self.qi, self.ki, self.w, self.pos0, self.T, self.N = qi, ki, w, pos0, T, N
        self.layers = layers                      # list of (q [T,Hq,d], k [Hkv,N,d], v)
        self.full = set(full_layers)
        self.k_sel = k_sel
        self.fused = fused
        d = layers[0][0].shape[-1]
        self.scale = 1.0 / math.sqrt(d) if scale is None else scale
        # the score matrix only for the two-call index (or a fused call's fallback)
        self.scores = None if fused else torch.empty((T, N), dtype=torch.float32, device=dev)
        self.idx = torch.empty((T, k_sel), dtype=torch.int32, device=dev)   # the index cache
        self.cnt = torch.empty(T, dtype=torch.int32, device=dev)
        self.err = torch.zeros(1, dtype=torch.int32, device=dev)
        self.outs = [torch.empty(L[0].shape, dtype=out_dtype or torch.float32, device=dev) for L in layers]
        self.ws = None
        self.ws_index = None

    def index_two_call(self):
        """Indexer scores into [T, N], then the causal top-k of every row."""
        if self.scores is None:
            self.scores = _t().empty((self.T, self.N), dtype=_t().float32, device=self.qi.device)
        sa_estimate(INDEXER, self.qi, self.ki, self.scores, weights=self.w, q_pos0=self.pos0)
        sa_select_topk(self.scores, self.idx, self.cnt, k=self.k_sel, causal=True, causal_period=self.T,
                       causal_offset=self.pos0, err_flag=self.err)

    def index(self, check: bool = True):
        """The index of the full layer.  Fused: one call without the score
        matrix.  With check=True (the default) the host reads the error flag
        (one device sync): rows whose sampled threshold failed (flag value 2,
        cnt = -1) make the whole chunk be recomputed with two calls, and a NaN
        among the scores (flag value 1) raises.  check=False leaves reading
        the flag to the caller."""
        if not self.fused:
            self.index_two_call()
        else:
            self.ws_index = sa_indexer_topk(self.qi, self.ki, self.idx, self.cnt, weights=self.w,
                                            q_pos0=self.pos0, k=self.k_sel, err_flag=self.err,
                                            workspace=self.ws_index)
            if check and int(self.err.item()) & 2:
                self.err.bitwise_and_(~2)   # keep bit 0 (NaN) if the fused call set it
                self.index_two_call()
        if check and int(self.err.item()) & 1:
            raise FloatingPointError("indexer: NaN among the scores; the index is unspecified")

    def attend(self, layer: int):
        q, k, v = self.layers[layer]
        self.ws = sa_gather_decode(q, k, v, self.outs[layer], tok_idx=self.idx, scale=self.scale,
                                   workspace=self.ws)

    def step(self, reuse: bool = True, check: bool = True):
        """Every layer: full layers (or all of them without reuse) build the
        index, checked as in index(); each layer then attends through it."""
        for layer in range(len(self.layers)):
            if layer in self.full or not reuse:
                self.index(check=check)
            self.attend(layer)
