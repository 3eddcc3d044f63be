"""Shared helpers for the GPU parity tests: device uploads, tolerance checks,
tie-tolerant validity of selected sets, and certification redraws (which ask
the CPU oracle whether a row's k-th/(k+1)-th gap exceeds 1e-3 of its scale)."""
from __future__ import annotations

import numpy as np

import oracle
import workloads as W

DEV = "cuda:0"

# attention tolerances: fp32 inputs, bf16 inputs with fp32 accumulation
TOL_F32_MAX = 1e-4
TOL_BF16_MAX = 2e-2
TOL_BF16_MEAN = 2e-3
# estimator scores: below half the 1e-3 certification gap
TOL_SCORE_REL = 1e-4


def torch():
    import torch as t
    return t


def dev_bf16(bits: np.ndarray):
    t = torch()
    return t.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(t.bfloat16).to(DEV)


def dev_f32(x: np.ndarray):
    return torch().from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV)


def dev_i32(x: np.ndarray):
    return torch().from_numpy(np.ascontiguousarray(x, dtype=np.int32)).to(DEV)


def host(t) -> np.ndarray:
    tt = torch()
    if t.dtype == tt.bfloat16:
        t = t.float()
    return t.detach().cpu().numpy()


def lower_triangle(S: np.ndarray) -> np.ndarray:
    """Block scores as the oracle states them: the library leaves entries
    above the diagonal (j > i) unwritten, the oracle holds -inf there."""
    S = np.array(S, copy=True)
    nb = S.shape[-1]
    S[..., np.triu(np.ones((nb, nb), bool), 1)] = -np.inf
    return S


def pad_table(lists, kmax: int):
    """list of index arrays -> (idx [R,kmax] int32 padded with -1, cnt [R])."""
    R = len(lists)
    idx = np.full((R, kmax), -1, np.int32)
    cnt = np.zeros(R, np.int32)
    for r, a in enumerate(lists):
        idx[r, :len(a)] = a
        cnt[r] = len(a)
    return idx, cnt


def assert_attention_close(got: np.ndarray, want: np.ndarray, bf16: bool, what: str = ""):
    err = np.abs(np.asarray(got, np.float64) - np.asarray(want, np.float64))
    mx, mean = float(err.max()), float(err.mean())
    if bf16:
        assert mx <= TOL_BF16_MAX and mean <= TOL_BF16_MEAN, f"{what}: max {mx:.3e} mean {mean:.3e}"
    else:
        assert mx <= TOL_F32_MAX, f"{what}: max {mx:.3e}"
    return mx, mean


def assert_scores_close(got: np.ndarray, want: np.ndarray, what: str = ""):
    """Row-wise |got - want| <= 1e-4 * max|want| over the finite entries; -inf must match."""
    g = np.asarray(got, np.float64)
    w = np.asarray(want, np.float64)
    assert np.array_equal(np.isneginf(g), np.isneginf(w)), f"{what}: -inf pattern differs"
    fin = np.isfinite(w)
    g0 = np.where(fin, g, 0.0)
    w0 = np.where(fin, w, 0.0)
    scale = np.max(np.abs(w0), axis=-1, keepdims=True)
    bad = np.abs(g0 - w0) > TOL_SCORE_REL * np.maximum(scale, 1e-30)
    assert not bad.any(), f"{what}: {int(bad.sum())} scores outside 1e-4*row scale"


def tie_tolerant_valid(sel: np.ndarray, scores: np.ndarray, k: int, forced: np.ndarray, rel: float = 1e-3):
    """True when sel (ascending) holds all forced members, exactly k pool
    members, and every chosen pool member scores at least every unchosen one
    minus rel * max|pool score|."""
    sel = np.asarray(sel, np.int64)
    n = scores.shape[0]
    forced = np.asarray(forced, np.int64)
    if not set(forced.tolist()) <= set(sel.tolist()):
        return False
    pool = np.setdiff1d(np.arange(n), forced)
    chosen = np.intersect1d(sel, pool)
    if chosen.shape[0] != min(k, pool.shape[0]) or np.any(np.diff(sel) <= 0):
        return False
    if chosen.shape[0] in (0, pool.shape[0]):
        return True
    rest = np.setdiff1d(pool, chosen)
    tol = rel * np.max(np.abs(scores[pool]))
    return bool(scores[chosen].min() >= scores[rest].max() - tol)


# ---------------------------------------------------------------- certification
def block_row_rule(i: int, n_sink: int, n_local: int, k=None, ratio=None):
    n = i + 1
    f = oracle.forced_set(n, n_sink, n_local)
    return f, oracle.budget(n, f.shape[0], k, ratio)


def certify_prefill(inp: W.PrefillInputs, seed: int, bs: int, scale: float, n_sink: int, n_local: int,
                    k=None, ratio=None, q_shift: float = 1.0, max_attempts: int = 64):
    """Redraw query blocks until every (b, h, i) row's pooled-score selection is
    certified.  Mutates inp.q; returns the number of redrawn blocks."""
    B, Hq, N, d = inp.q.shape
    Hkv = inp.k.shape[1]
    nb = N // bs
    redrawn = 0
    for b in range(B):
        kbar = [oracle.mean_pool(inp.f32("k")[b, g], bs) for g in range(Hkv)]
        for h in range(Hq):
            g = oracle.gqa_group(h, Hq, Hkv)
            for i in range(nb):
                f, kr = block_row_rule(i, n_sink, n_local, k, ratio)
                attempt = 0
                while True:
                    rows = inp.q[b, h, i * bs:(i + 1) * bs]
                    rf = rows if inp.dtype == "f32" else W.bf16_to_f32(rows)
                    qbar = np.asarray(rf, np.float64).mean(axis=0)
                    s = (kbar[g][:i + 1] @ qbar) * scale
                    if oracle.certified_row(s, kr, f):
                        break
                    attempt += 1
                    assert attempt < max_attempts, f"cannot certify row {(b, h, i)}"
                    inp.q[b, h, i * bs:(i + 1) * bs] = W.redraw_query_block(
                        seed, b, h, i, attempt, bs, d, inp.u, q_shift, inp.dtype)
                    redrawn += 1
    return redrawn


# ---------------------------------------------------------------- forward on the oracle's own sets
def fwd_on_oracle_blocks(sa, q, k, v, h: int, rows: dict, kmax: int):
    """Run the bf16 forward for query head h alone (head-list launch) on block
    lists chosen by the oracle: rows maps query block -> ascending blocks; all
    other rows are empty.  Returns out [N, d] (float32) of head h."""
    t = torch()
    B, Hq, N, d = q.shape
    nb = N // 64
    lists = [np.asarray(rows.get(i, np.zeros(0, np.int64))) for i in range(nb)]
    idx, cnt = pad_table(lists, kmax)
    out = t.zeros((B, Hq, N, d), dtype=t.float32, device=q.device)
    sa.sa_block_sparse_fwd(q, k, v, out, block_idx=dev_i32(idx.reshape(1, 1, nb, kmax)),
                           block_cnt=dev_i32(cnt.reshape(1, 1, nb)), heads=[h])
    t.cuda.synchronize()
    return host(out[0, h])


def fwd_on_oracle_vs(sa, q, k, v, h: int, cols: np.ndarray, offs: np.ndarray, max_iv: int, max_col: int):
    """Run the bf16 forward for query head h alone on the vertical-slash tables
    the oracle builds from its own (cols, offs).  Returns out [N, d] of head h."""
    t = torch()
    B, Hq, N, d = q.shape
    nb = N // 64
    iv = np.zeros((nb, max_iv, 2), np.int32)
    ivc = np.zeros(nb, np.int32)
    col = np.zeros((nb, max_col), np.int32)
    colc = np.zeros(nb, np.int32)
    for i, (ivs, vert) in enumerate(oracle.vs_block_tables(cols, offs, N, 64)):
        ivc[i] = len(ivs)
        for j, (a, e) in enumerate(ivs):
            iv[i, j] = (a, e)
        colc[i] = len(vert)
        col[i, :len(vert)] = vert
    out = t.zeros((B, Hq, N, d), dtype=t.float32, device=q.device)
    sa.sa_block_sparse_fwd(q, k, v, out, iv=dev_i32(iv[None, None]), iv_cnt=dev_i32(ivc[None, None]),
                           col=dev_i32(col[None, None]), col_cnt=dev_i32(colc[None, None]), heads=[h])
    t.cuda.synchronize()
    return host(out[0, h])
