"""Vertical-slash estimate, index build and attention (oracle; test infrastructure only).

"MInference 1.0" article, §方法介紹: for the vertical-slash pattern the best
vertical-line and slash-line indices are estimated from the attention between
the last queries and all keys.  §延遲和內核中的稀疏模式, Fig. 4: vertical
lines are computed in 1x64 pieces, slash lines with block-level attention in
64x64 blocks.

Steps:
  1. per query head h, the last L queries (positions N-L..N-1) attend all
     keys causally: A = softmax(Q_last K^T * scale) (L x N).
  2. vertical score a_v[c] = sum_r A[r, c]; slash score
     a_s[o] = sum_r A[r, pos_r - o] (offset o = query position - key index).
  3. keep the top n_v columns and the top n_s offsets (select.py order).
  4. query block i (rows 64i..64i+63): each kept offset o covers the
     contiguous 64-key tile [64i-o, 64i-o+64) clipped at 0 — the square tile
     whose main diagonal is the slash line (reading; the page says only
     "64x64 blocks").  Tiles are united into disjoint intervals.  The block's
     vertical set is the kept columns c <= 64i+63 outside those intervals.
  5. row r attends (intervals ∪ verticals) ∩ [0, r].

Readings: nothing is forced (the page keeps only the top columns and
offsets), so an early row can have no key and yields o = 0, lse = -inf.
Mean pooling is not used for this pattern (the page's sentence that mentions
pooling for all three patterns then concludes with block-sparse indices
only).  Parity unpinned for the choice of slash-tile reading: no printed
example on the page distinguishes it; it is pinned only by the brute-force
dense-mask cross-check of the same reading.
"""
from __future__ import annotations

import numpy as np

from .attention import attend_rows, gqa_group
from .select import topk_row


def vs_estimate(q_last: np.ndarray, K: np.ndarray, q_pos: np.ndarray, scale: float):
    """(a_v [N], a_s [N]) for one head: q_last [L, d], K [N, d]; q_pos holds the
    absolute position of each of the L query rows."""
    q_last = np.asarray(q_last, np.float64)
    K = np.asarray(K, np.float64)
    N = K.shape[0]
    s = (q_last @ K.T) * scale
    cols = np.arange(N)
    s[cols[None, :] > np.asarray(q_pos)[:, None]] = -np.inf
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    a = p / p.sum(axis=1, keepdims=True)
    a_v = a.sum(axis=0)
    a_s = np.zeros(N)
    for r, pr in enumerate(q_pos):
        c = np.arange(pr + 1)
        a_s[pr - c] += a[r, c]          # offsets pr - c are distinct within a row
    return a_v, a_s


def vs_select(a_v: np.ndarray, a_s: np.ndarray, n_v: int, n_s: int):
    """Top n_v columns and top n_s offsets, ascending."""
    none = np.zeros(0, np.int64)
    return topk_row(a_v, n_v, none), topk_row(a_s, n_s, none)


def vs_block_keys(cols: np.ndarray, offs: np.ndarray, i: int, bs: int):
    """(intervals [(start, end_exclusive)], verticals) for query block i."""
    tiles = []
    for o in np.sort(np.asarray(offs, np.int64)):
        lo, hi = i * bs - int(o), i * bs - int(o) + bs
        lo = max(lo, 0)
        if hi > lo:
            tiles.append((lo, hi))
    tiles.sort()
    merged: list[list[int]] = []
    for lo, hi in tiles:
        if merged and lo <= merged[-1][1]:
            merged[-1][1] = max(merged[-1][1], hi)
        else:
            merged.append([lo, hi])
    ivs = [(a, b) for a, b in merged]
    last = i * bs + bs - 1
    vert = []
    for c in np.sort(np.asarray(cols, np.int64)):
        c = int(c)
        if c > last:
            break
        if not any(a <= c < b for a, b in ivs):
            vert.append(c)
    return ivs, np.array(vert, np.int64)


def vs_block_tables(cols: np.ndarray, offs: np.ndarray, N: int, bs: int):
    """Per query block: list of (intervals, verticals)."""
    return [vs_block_keys(cols, offs, i, bs) for i in range(N // bs)]


def vs_attention(Q, K, V, sel, bs: int, scale: float, heads=None, blocks=None):
    """O [B,Hq,N,d], lse [B,Hq,N]; sel[b][h] = (cols, offs) for head h."""
    B, Hq, N, d = Q.shape
    Hkv = K.shape[1]
    O = np.zeros((B, Hq, N, V.shape[-1]))
    L = np.full((B, Hq, N), -np.inf)
    for b in range(B):
        for h in (range(Hq) if heads is None else heads):
            g = gqa_group(h, Hq, Hkv)
            cols, offs = sel[b][h]
            for i in (range(N // bs) if blocks is None else blocks):
                ivs, vert = vs_block_keys(cols, offs, i, bs)
                parts = [np.arange(a, e) for a, e in ivs] + [vert]
                keys = np.unique(np.concatenate(parts)) if parts else np.zeros(0, np.int64)
                rows = np.arange(i * bs, (i + 1) * bs)
                o, l = attend_rows(Q[b, h, rows], K[b, g], V[b, g], keys, scale, row_pos=rows)
                O[b, h, rows] = o
                L[b, h, rows] = l
    return O, L
