"""Per-head sparse patterns, A-shape included (oracle; test infrastructure only).

"MInference 1.0" article, §方法介紹: attention heads follow one of three
patterns — A-shape, vertical-slash and block-sparse; the pattern of each head
is chosen offline, and at inference each head's sparse indices are
approximated according to its own pattern.  The offline search is not part of
this oracle: the head -> pattern assignment is an input.

A-shape: global plus local-window attention ("稀疏注意力机制解析" explainer,
§1.2), taken at the granularity of the article's 64-token blocks
(§延遲和內核中的稀疏模式, Fig. 4).  Reading: query block i keeps blocks
0 .. n_sink-1 and the n_local blocks i-n_local+1 .. i (clipped at 0, each
once), the same sink/local rule as the forced members of the block-sparse
pattern, with no estimated blocks; row r attends those keys up to r.
"""
from __future__ import annotations

import numpy as np

from .attention import gqa_group
from .blocksparse import block_scores, block_select, block_sparse_attention
from .select import forced_set
from .vslash import vs_attention, vs_estimate, vs_select

A_SHAPE, VERTICAL_SLASH, BLOCK_SPARSE = "A", "VS", "BS"


def ashape_blocks(nb: int, n_sink: int, n_local: int):
    """Kept block list of every query block (ascending)."""
    return [forced_set(i + 1, n_sink, n_local) for i in range(nb)]


def ashape_attention(Q, K, V, n_sink: int, n_local: int, bs: int, scale: float, heads=None, blocks=None):
    """O [B,Hq,N,d], lse [B,Hq,N] of the A-shape pattern on every head."""
    B, Hq, N, _ = Q.shape
    table = ashape_blocks(N // bs, n_sink, n_local)
    kept = [[table] * Hq for _ in range(B)]
    return block_sparse_attention(Q, K, V, kept, bs, scale, heads, blocks)


def mixed_layer(Q, K, V, patterns, *, bs: int, scale: float, a_shape=(1, 4), block=None, vslash=None,
                last_q: int = 64):
    """One layer whose query head h runs patterns[h].

    a_shape = (n_sink, n_local) blocks; block = dict(n_sink, n_local, k or
    ratio) for block-sparse heads; vslash = (n_vert, n_slash) for
    vertical-slash heads.  Returns (O, lse, sel) with sel[b][h] the head's
    selection: the kept block lists (A, BS) or the (columns, offsets) pair (VS).
    Each head uses its own KV head g(h) and the single-pattern steps above."""
    B, Hq, N, d = Q.shape
    Hkv = K.shape[1]
    nb = N // bs
    O = np.zeros((B, Hq, N, V.shape[-1]))
    L = np.full((B, Hq, N), -np.inf)
    sel = [[None] * Hq for _ in range(B)]
    for h, pat in enumerate(patterns):
        g = gqa_group(h, Hq, Hkv)
        q1, k1, v1 = Q[:, h:h + 1], K[:, g:g + 1], V[:, g:g + 1]
        if pat == A_SHAPE:
            o, l = ashape_attention(q1, k1, v1, a_shape[0], a_shape[1], bs, scale)
            for b in range(B):
                sel[b][h] = ashape_blocks(nb, *a_shape)
        elif pat == BLOCK_SPARSE:
            kept = block_select(block_scores(q1, k1, bs, scale), **block)
            o, l = block_sparse_attention(q1, k1, v1, kept, bs, scale)
            for b in range(B):
                sel[b][h] = kept[b][0]
        elif pat == VERTICAL_SLASH:
            vs_sel = []
            for b in range(B):
                a_v, a_s = vs_estimate(q1[b, 0, N - last_q:], k1[b, 0], np.arange(N - last_q, N), scale)
                vs_sel.append([vs_select(a_v, a_s, *vslash)])
                sel[b][h] = vs_sel[b][0]
            o, l = vs_attention(q1, k1, v1, vs_sel, bs, scale)
        else:
            raise ValueError(f"unknown pattern {pat!r}")
        O[:, h] = o[:, 0]
        L[:, h] = l[:, 0]
    return O, L, sel
