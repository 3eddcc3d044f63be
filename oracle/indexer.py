"""Token-level indexer selection, gathered attention and index reuse
(oracle; test infrastructure only).

IndexCache article, §长文本的算力困境: a light "lightning indexer" picks, for
every layer, the most relevant token subset that attention then runs over; the
indexer's own cost is quadratic.  §"偷懒"的艺术: layers are split into full
layers, which run the indexer and store the selected token indices, and shared
layers, which copy the nearest full layer's indices and skip the indexer.

The pages give no indexer formula; the synthetic workload defines
I[t,s] = sum_h w_h * ReLU(qI[t,h] . kI[s]) over causal pairs s <= pos0 + t,
with a single indexer key head and one weight per indexer head (reading: the
weight carries no token index, so it is shared by all tokens).

Readings: the attention layers are MQA (all query heads read KV head 0, or
floor(h*Hkv/Hq) in general); layers carry independent inputs; every layer
after a full layer reuses that layer's indices unchanged.
"""
from __future__ import annotations

import numpy as np

from .attention import attend_rows, gqa_group
from .select import candidate_count, topk_row


def indexer_scores(qi: np.ndarray, ki: np.ndarray, w: np.ndarray, pos0: int, rows=None):
    """I [len(rows), N]: weighted sum over indexer heads of ReLU(q . k);
    -inf for s > pos0 + t.  qi [T,Hi,di], ki [N,di], w [Hi]."""
    T, Hi, di = qi.shape
    N = ki.shape[0]
    rows = np.arange(T) if rows is None else np.asarray(rows)
    kf = np.asarray(ki, np.float64)
    wf = np.asarray(w, np.float64)
    out = np.empty((rows.shape[0], N))
    for n, t in enumerate(rows):
        dots = np.asarray(qi[t], np.float64) @ kf.T       # [Hi, N]
        out[n] = wf @ np.maximum(dots, 0.0)
        out[n, pos0 + t + 1:] = -np.inf
    return out


def indexer_select(I: np.ndarray, rows, pos0: int, k: int):
    """Top-k causal keys per query row (ascending)."""
    none = np.zeros(0, np.int64)
    res = []
    for n, t in enumerate(rows):
        cnt = candidate_count(int(t), I.shape[1], True, 1 << 62, pos0)
        res.append(topk_row(I[n, :cnt], k, none))
    return res


def gathered_attention(Q, K, V, idx, scale: float, rows=None):
    """O [len(rows),Hq,d], lse [len(rows),Hq]: query token t, every head h,
    attends K[g(h)][idx[t]].  Q [T,Hq,d]; K, V [Hkv,N,d]; idx: per-row index
    arrays (entries < 0 are padding)."""
    T, Hq, d = Q.shape
    Hkv = K.shape[0]
    rows = np.arange(T) if rows is None else np.asarray(rows)
    O = np.zeros((rows.shape[0], Hq, V.shape[-1]))
    L = np.full((rows.shape[0], Hq), -np.inf)
    for n, t in enumerate(rows):
        keys = np.asarray(idx[n], np.int64)
        keys = keys[keys >= 0]
        for h in range(Hq):
            g = gqa_group(h, Hq, Hkv)
            o, l = attend_rows(np.asarray(Q[t, h], np.float64)[None, :], K[g], V[g], keys, scale)
            O[n, h], L[n, h] = o[0], l[0]
    return O, L


def index_cache_forward(layers, full_layers, qi, ki, w, pos0: int, k: int, scale: float, rows=None):
    """Multi-layer sparse attention with index reuse.

    layers: list of (Q, K, V); full_layers: set of layer numbers that run the
    indexer (layer 0 must be one).  Shared layers reuse the indices of the
    nearest preceding full layer.  Returns ([O_l], [idx_l]) where idx_l is the
    index list each layer attended."""
    T = layers[0][0].shape[0]
    rows = np.arange(T) if rows is None else np.asarray(rows)
    assert 0 in full_layers
    outs, used = [], []
    cur = None
    for l, (Q, K, V) in enumerate(layers):
        if l in full_layers:
            I = indexer_scores(qi, ki, w, pos0, rows)
            cur = indexer_select(I, rows, pos0, k)
        O, _ = gathered_attention(Q, K, V, cur, scale, rows)
        outs.append(O)
        used.append(cur)
    return outs, used
