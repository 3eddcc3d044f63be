"""Exact softmax attention restricted to a key set (oracle; test infrastructure only).

Every sparse variant on the pages ends in ordinary softmax attention over the
selected keys: block-sparse FlashAttention over the estimated blocks
("MInference 1.0" article, §方法介紹), attention only over the chosen
clusters' keys (Squeezed Attention page, §技术方案), attention over the
indexer's token subset (IndexCache article, §长文本的算力困境).  Restricting a
query to a subset changes only which keys enter the softmax, so the oracle is
the plain definition evaluated on that subset, in fp64.

Readings: a row whose admissible set is empty returns o = 0 and lse = -inf
(the pages never meet that case).  Grouped-query heads: query head h reads KV
head floor(h*Hkv/Hq) (the pages are silent; contiguous grouping).
"""
from __future__ import annotations

import numpy as np


def gqa_group(h: int, Hq: int, Hkv: int) -> int:
    return (h * Hkv) // Hq


def attend_rows(q: np.ndarray, K: np.ndarray, V: np.ndarray, keys: np.ndarray,
                scale: float, row_pos: np.ndarray | None = None):
    """Softmax attention of each row of q over K[keys], V[keys].

    q: [R, d]; K, V: [N, d]; keys: 1-D array of distinct key indices.
    row_pos: absolute position of each query row; key c is admissible for
    row r only when c <= row_pos[r] (token-causal).  None: no causal mask.
    Returns (o [R, d], lse [R]) in float64."""
    q = np.asarray(q, np.float64)
    keys = np.asarray(keys, np.int64)
    R, d = q.shape
    if keys.shape[0] == 0:
        return np.zeros((R, V.shape[1])), np.full(R, -np.inf)
    Kk = np.asarray(K[keys], np.float64)
    Vk = np.asarray(V[keys], np.float64)
    s = (q @ Kk.T) * scale
    if row_pos is not None:
        s[keys[None, :] > np.asarray(row_pos)[:, None]] = -np.inf
    m = s.max(axis=1)
    empty = ~np.isfinite(m)
    m0 = np.where(empty, 0.0, m)
    p = np.exp(s - m0[:, None])
    l = p.sum(axis=1)
    o = np.zeros((R, Vk.shape[1]))
    nz = l > 0
    o[nz] = (p[nz] @ Vk) / l[nz, None]
    lse = np.where(nz, m0 + np.log(np.where(nz, l, 1.0)), -np.inf)
    return o, lse
