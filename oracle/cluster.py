"""Clustered-context decode (oracle; test infrastructure only).

Squeezed Attention page, §技术方案: offline, the fixed context's keys are
clustered (centroid per cluster, key -> cluster index); online, each query is
compared with every centroid, the top-K clusters are chosen, and attention
runs only over the key/value pairs of those clusters.  §部署建议: K = sqrt(N)
clusters, select 1/4 to 1/2 of them.

Readings: scores are q . centroid * scale; the selection is made per query
head; there is no causal mask (the fixed context precedes the query).
"""
from __future__ import annotations

import numpy as np

from .attention import attend_rows, gqa_group
from .select import topk_row, mass_row


def centroid_scores(q: np.ndarray, centroids: np.ndarray, scale: float) -> np.ndarray:
    """s [T,Hq,C] = q[t,h] . centroid[g(h),c] * scale."""
    q = np.asarray(q, np.float64)
    mu = np.asarray(centroids, np.float64)
    T, Hq, d = q.shape
    Hkv = mu.shape[0]
    s = np.empty((T, Hq, mu.shape[1]))
    for h in range(Hq):
        s[:, h] = (q[:, h] @ mu[gqa_group(h, Hq, Hkv)].T) * scale
    return s


def cluster_select(s: np.ndarray, k: int):
    """Top-k cluster ids per (t, h), ascending: list[T][Hq]."""
    none = np.zeros(0, np.int64)
    return [[topk_row(s[t, h], k, none) for h in range(s.shape[1])] for t in range(s.shape[0])]


def cluster_select_mass(s: np.ndarray, mass: float, k_min: int = 0, k_max: int | None = None):
    """Adaptive cluster choice per (t, h), ascending: list[T][Hq].  The count
    follows the softmax of the row's centroid scores (Squeezed Attention page,
    §技术方案, adaptive cluster selection); the rule is mass_row's."""
    return [[mass_row(s[t, h], mass, k_min, k_max) for h in range(s.shape[1])] for t in range(s.shape[0])]


def cluster_pack(labels: np.ndarray, C: int):
    """Cluster-major order of the context, stable in token order.

    Returns (ptr [Hkv, C+1], perm [Hkv, N]): the tokens of cluster c are
    perm[g, ptr[g,c]:ptr[g,c+1]], ascending.  Written as an explicit counting
    sort so that a reader can check it line by line."""
    labels = np.asarray(labels, np.int64)
    Hkv, N = labels.shape
    ptr = np.zeros((Hkv, C + 1), np.int64)
    perm = np.empty((Hkv, N), np.int64)
    for g in range(Hkv):
        count = np.zeros(C, np.int64)
        for c in labels[g]:
            count[c] += 1
        ptr[g, 1:] = np.cumsum(count)
        fill = ptr[g, :C].copy()
        for t, c in enumerate(labels[g]):
            perm[g, fill[c]] = t
            fill[c] += 1
    return ptr, perm


def cluster_decode(q, K, V, labels, sel, scale: float):
    """O [T,Hq,d], lse [T,Hq]: q[t,h] attends the context tokens whose label
    is among sel[t][h].  K, V: [Hkv, N, d] in context order."""
    q = np.asarray(q, np.float64)
    T, Hq, d = q.shape
    Hkv = K.shape[0]
    O = np.zeros((T, Hq, V.shape[-1]))
    L = np.full((T, Hq), -np.inf)
    for t in range(T):
        for h in range(Hq):
            g = gqa_group(h, Hq, Hkv)
            keys = np.nonzero(np.isin(labels[g], sel[t][h]))[0]
            o, l = attend_rows(q[t, h][None, :], K[g], V[g], keys, scale)
            O[t, h], L[t, h] = o[0], l[0]
    return O, L
