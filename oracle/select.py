"""Per-row top-k selection with forced members (oracle; test infrastructure only).

What the pages fix: a cheap score ranks keys, blocks or clusters and the top
subset is kept ("MInference 1.0" article, §方法介紹; Squeezed Attention page,
§技术方案, "select the Top-K most relevant clusters"; IndexCache article,
§长文本的算力困境, the indexer keeps the most relevant token subset).  Local
and global members are always attended ("稀疏注意力机制解析", §1.2).

Readings (the pages are silent):
  * order: higher score first, equal scores -> lower index first; -0 == +0;
    NaN is an error.  Selected indices are reported in ascending order.
  * forced members (n_sink leading candidates, n_local trailing candidates
    ending at the causal diagonal) are always kept and not counted in k.
  * ratio budget: k_r = ceil(num * n_r / den) over the row's n_r causal
    candidates, capped at the non-forced candidates.
"""
from __future__ import annotations

import numpy as np


def candidate_count(r: int, ncand: int, causal: bool, period: int = 1, offset: int = 0) -> int:
    """Number of candidates of row r: all ncand, or the causal prefix
    0..(r mod period)+offset."""
    if not causal:
        return ncand
    return min(ncand, (r % period) + offset + 1)


def forced_set(n: int, n_sink: int, n_local: int) -> np.ndarray:
    """Leading n_sink and trailing n_local candidates of a row with n candidates."""
    s = set(range(min(n_sink, n))) | set(range(max(0, n - n_local), n))
    return np.array(sorted(s), dtype=np.int64)


def ratio_budget(n: int, num: int, den: int) -> int:
    """ceil(num*n/den) in integer arithmetic."""
    return -((-num * n) // den)


def budget(n: int, n_forced: int, k: int | None, ratio: tuple[int, int] | None) -> int:
    kb = k if ratio is None else ratio_budget(n, ratio[0], ratio[1])
    return max(0, min(kb, n - n_forced))


def topk_row(scores: np.ndarray, k: int, forced: np.ndarray) -> np.ndarray:
    """Ascending indices of forced ∪ (top-k of the remaining candidates).

    ``scores`` holds one value per candidate 0..n-1.  The rank uses the total
    order stated in the module docstring; the sort is a library primitive
    (np.lexsort) over (-score, index)."""
    s = np.asarray(scores, dtype=np.float64)
    if np.isnan(s).any():
        raise ValueError("NaN score")
    n = s.shape[0]
    pool = np.setdiff1d(np.arange(n, dtype=np.int64), forced)
    k = min(k, pool.shape[0])
    order = np.lexsort((pool, -s[pool]))   # primary key is the last one
    chosen = pool[order[:k]]
    return np.sort(np.concatenate([np.asarray(forced, np.int64), chosen]))


def select_rows(scores: np.ndarray, *, causal: bool, period: int = 1, offset: int = 0,
                n_sink: int = 0, n_local: int = 0, k: int | None = None,
                ratio: tuple[int, int] | None = None, ncand: int | None = None):
    """Row-wise selection over a [R, ncand] score matrix.

    Returns a list of ascending index arrays, one per row."""
    R = scores.shape[0]
    nc = scores.shape[1] if ncand is None else ncand
    out = []
    for r in range(R):
        n = candidate_count(r, nc, causal, period, offset)
        f = forced_set(n, n_sink, n_local)
        kr = budget(n, f.shape[0], k, ratio)
        out.append(topk_row(scores[r, :n], kr, f))
    return out


def certified_row(scores: np.ndarray, k: int, forced: np.ndarray, rel: float = 1e-3) -> bool:
    """True when the k-th and (k+1)-th best non-forced scores differ by more
    than rel * max|score| over the non-forced candidates, so that any score
    perturbation below half that gap selects the same set."""
    s = np.asarray(scores, dtype=np.float64)
    pool = np.setdiff1d(np.arange(s.shape[0]), forced)
    if k <= 0 or k >= pool.shape[0]:
        return True
    v = np.sort(s[pool])[::-1]
    scale = np.max(np.abs(s[pool]))
    return bool(v[k - 1] - v[k] > rel * scale)


# ---------------------------------------------------------------------------
# Adaptive budget (Squeezed Attention page, §技术方案, key technical points:
# the number of clusters kept follows the distribution of the query's centroid
# similarities).  The page gives no formula; the reading taken here:
#   * a row's scores are logits; candidate j weighs w_j = exp(s_j - m) with m
#     the row maximum, and an entry equal to m weighs exactly 1 (so +inf
#     entries share all the mass and an all -inf row weighs uniformly);
#   * in the order of topk_row (higher score first, lower index on ties) the
#     row keeps the shortest prefix whose weight reaches mass * sum(w);
#   * that count is clamped to [k_min, k_max] and to the row length.
# ---------------------------------------------------------------------------
def mass_weights(scores: np.ndarray) -> np.ndarray:
    """w_j = exp(s_j - max s), with entries equal to the maximum weighing 1."""
    s = np.asarray(scores, dtype=np.float64)
    if np.isnan(s).any():
        raise ValueError("NaN score")
    m = s.max()
    with np.errstate(invalid="ignore"):
        return np.where(s == m, 1.0, np.exp(s - m))


def mass_count(scores: np.ndarray, mass: float, k_min: int = 0, k_max: int | None = None) -> int:
    """Shortest prefix (in selection order) holding at least ``mass`` of the
    softmax weight, clamped to [k_min, k_max] and to the row length."""
    s = np.asarray(scores, dtype=np.float64)
    n = s.shape[0]
    w = mass_weights(s)
    order = np.lexsort((np.arange(n), -s))
    ws = w[order]
    before = np.concatenate([[0.0], np.cumsum(ws)[:-1]])   # weight ahead of each position
    c = int(np.count_nonzero(before < mass * ws.sum()))
    c = max(c, k_min)
    if k_max is not None:
        c = min(c, k_max)
    return min(c, n)


def mass_row(scores: np.ndarray, mass: float, k_min: int = 0, k_max: int | None = None) -> np.ndarray:
    """Ascending indices of the adaptive selection of one row."""
    c = mass_count(scores, mass, k_min, k_max)
    return topk_row(scores, c, np.zeros(0, np.int64))


def mass_margin(scores: np.ndarray, mass: float) -> float:
    """Distance, relative to the total weight, between mass and the nearest
    share that the count rule compares with it (the weight ahead of each
    position; the full sum is never compared).  When it exceeds the arithmetic
    error of a caller's summation, that caller must find the same count."""
    s = np.asarray(scores, dtype=np.float64)
    w = mass_weights(s)
    order = np.lexsort((np.arange(s.shape[0]), -s))
    ws = w[order]
    before = np.concatenate([[0.0], np.cumsum(ws)[:-1]])
    return float(np.min(np.abs(before / ws.sum() - mass)))
