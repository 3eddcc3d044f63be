"""Block-sparse estimate, selection and attention (oracle; test infrastructure only).

"MInference 1.0" article, §方法介紹: for the block-sparse pattern the block
indices are estimated from mean-pooled Q and K, using the fact that mean
pooling commutes with the matrix product, and a block-sparse FlashAttention
then runs over the chosen blocks.  Blocks are 64 tokens
(§延遲和內核中的稀疏模式, Fig. 4, block-level attention in 64x64 blocks).

Steps, in the order the method takes them:
  1. Qbar[h,i] = mean of the 64 query rows of block i; Kbar[g,j] likewise.
  2. S[h,i,j] = Qbar[h,i] . Kbar[g(h),j] * scale for causal pairs j <= i
     (-inf otherwise).
  3. per query-block row: forced blocks (sink + local ending at the diagonal)
     plus the top-k of the remaining causal blocks by S.
  4. each query row r of block i attends the keys of its kept blocks, keys
     c <= r only (token-causal inside the diagonal block).
"""
from __future__ import annotations

import numpy as np

from .attention import attend_rows, gqa_group
from .select import select_rows


def mean_pool(x: np.ndarray, bs: int) -> np.ndarray:
    """Mean over consecutive groups of bs rows: [N, d] -> [N/bs, d] (fp64)."""
    x = np.asarray(x, np.float64)
    n, d = x.shape
    return x.reshape(n // bs, bs, d).mean(axis=1)


def block_scores(Q: np.ndarray, K: np.ndarray, bs: int, scale: float) -> np.ndarray:
    """S [B,Hq,nb,nb]: pooled-query . pooled-key * scale on causal block pairs
    (j <= i), -inf above the diagonal.  Q [B,Hq,N,d], K [B,Hkv,N,d]."""
    B, Hq, N, d = Q.shape
    Hkv = K.shape[1]
    nb = N // bs
    S = np.full((B, Hq, nb, nb), -np.inf)
    tri = np.tril(np.ones((nb, nb), bool))
    for b in range(B):
        kbar = [mean_pool(K[b, g], bs) for g in range(Hkv)]
        for h in range(Hq):
            qbar = mean_pool(Q[b, h], bs)
            full = (qbar @ kbar[gqa_group(h, Hq, Hkv)].T) * scale
            S[b, h][tri] = full[tri]
    return S


def block_select(S: np.ndarray, *, n_sink: int, n_local: int, k: int | None = None,
                 ratio: tuple[int, int] | None = None):
    """Kept block lists per (b, h, i): forced sink/local blocks plus the top-k
    other causal blocks (ascending)."""
    B, Hq, nb, _ = S.shape
    kept = [[None] * Hq for _ in range(B)]
    for b in range(B):
        for h in range(Hq):
            kept[b][h] = select_rows(S[b, h], causal=True, period=nb, offset=0,
                                     n_sink=n_sink, n_local=n_local, k=k, ratio=ratio)
    return kept


def block_sparse_attention(Q, K, V, kept, bs: int, scale: float, heads=None, blocks=None):
    """O [B,Hq,N,d], lse [B,Hq,N]: each query row attends the union of its
    block's kept key blocks, token-causal.  ``heads``/``blocks`` restrict the
    rows computed (others stay 0 / -inf) for bounded samples."""
    B, Hq, N, d = Q.shape
    Hkv = K.shape[1]
    nb = N // bs
    O = np.zeros((B, Hq, N, V.shape[-1]))
    L = np.full((B, Hq, N), -np.inf)
    for b in range(B):
        for h in (range(Hq) if heads is None else heads):
            g = gqa_group(h, Hq, Hkv)
            Kg = np.asarray(K[b, g], np.float64)
            Vg = np.asarray(V[b, g], np.float64)
            for i in (range(nb) if blocks is None else blocks):
                blk = np.asarray(kept[b][h][i], np.int64)
                keys = (blk[:, None] * bs + np.arange(bs)[None, :]).reshape(-1)
                rows = np.arange(i * bs, (i + 1) * bs)
                o, l = attend_rows(Q[b, h, rows], Kg, Vg, keys, scale, row_pos=rows)
                O[b, h, rows] = o
                L[b, h, rows] = l
    return O, L
