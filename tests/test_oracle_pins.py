"""Pins of the CPU oracle against facts fixed outside the oracle itself:
closed forms, brute force on tiny inputs, algebraic invariants stated on the
pages, and the numbers the pages print (tests/golden/).  CPU only."""
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle
import workloads as W

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ------------------------------------------------------------------ naive references (loops)
def naive_masked_attention(q, K, V, allowed, scale):
    """Row-by-row softmax written with Python loops over a boolean mask."""
    R, N = allowed.shape
    V = np.asarray(V, np.float64)
    d = V.shape[1]
    out = np.zeros((R, d))
    lse = np.full(R, -math.inf)
    for r in range(R):
        s = [(c, scale * sum(float(q[r, x]) * float(K[c, x]) for x in range(q.shape[1])))
             for c in range(N) if allowed[r, c]]
        if not s:
            continue
        m = max(v for _, v in s)
        w = [(c, math.exp(v - m)) for c, v in s]
        tot = sum(x for _, x in w)
        for c, x in w:
            out[r] += (x / tot) * V[c]
        lse[r] = m + math.log(tot)
    return out, lse


def rnd(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


# ------------------------------------------------------------------ softmax attention
def test_softmax_worked_example():
    g = gold("softmax_worked.json")
    K = np.array(g["k"])[:, None]
    V = np.array(g["v"])[:, None]
    o, lse = oracle.attend_rows(np.array([g["q"]]), K, V, np.arange(3), 1.0)
    assert abs(o[0, 0] - g["out"]) < 1e-12
    assert abs(lse[0] - g["lse"]) < 1e-12


def test_all_blocks_kept_equals_dense_causal():
    bs, nb, d = 64, 3, 8
    N = bs * nb
    Q, K, V = rnd(1, 1, 1, N, d), rnd(2, 1, 1, N, d), rnd(3, 1, 1, N, d)
    kept = [[[np.arange(i + 1) for i in range(nb)]]]
    O, L = oracle.block_sparse_attention(Q, K, V, kept, bs, 0.3)
    causal = np.tril(np.ones((N, N), bool))
    On, Ln = naive_masked_attention(Q[0, 0], K[0, 0], V[0, 0], causal, 0.3)
    assert np.max(np.abs(O[0, 0] - On)) < 1e-12
    assert np.max(np.abs(L[0, 0] - Ln)) < 1e-12


def test_block_sparse_matches_brute_force_dense_mask():
    bs, nb, d = 64, 4, 6
    N = bs * nb
    Q, K, V = rnd(4, 1, 1, N, d), rnd(5, 1, 1, N, d), rnd(6, 1, 1, N, d)
    r = np.random.default_rng(7)
    kept_rows = []
    for i in range(nb):
        cand = np.arange(i + 1)
        kept_rows.append(np.sort(r.choice(cand, size=r.integers(1, i + 2), replace=False)))
    allowed = np.zeros((N, N), bool)
    for i, blks in enumerate(kept_rows):
        for rr in range(i * bs, (i + 1) * bs):
            for j in blks:
                for c in range(j * bs, (j + 1) * bs):
                    if c <= rr:
                        allowed[rr, c] = True
    O, L = oracle.block_sparse_attention(Q, K, V, [[kept_rows]], bs, 0.5)
    On, Ln = naive_masked_attention(Q[0, 0], K[0, 0], V[0, 0], allowed, 0.5)
    assert np.max(np.abs(O[0, 0] - On)) < 1e-12
    assert np.allclose(L[0, 0], Ln, atol=1e-12)


def test_closed_forms_zero_query_constant_value_single_key():
    N, d = 128, 5
    K, V = rnd(8, N, d), rnd(9, N, d)
    keys = np.array([0, 3, 17, 64, 100])
    # q = 0: uniform weights -> mean of the admissible values
    o, lse = oracle.attend_rows(np.zeros((2, d)), K, V, keys, 0.7, row_pos=np.array([20, 127]))
    assert np.allclose(o[0], V[[0, 3, 17]].mean(0), atol=1e-14)
    assert np.allclose(o[1], V[keys].mean(0), atol=1e-14)
    assert abs(lse[0] - math.log(3)) < 1e-14
    # constant values -> that constant, whatever the weights
    Vc = np.tile(np.arange(d, dtype=float), (N, 1))
    o, _ = oracle.attend_rows(rnd(10, 3, d), K, Vc, keys, 0.7)
    assert np.allclose(o, np.arange(d)[None, :], atol=1e-13)
    # a single admissible key -> its value exactly
    o, lse = oracle.attend_rows(rnd(11, 1, d), K, V, keys, 0.7, row_pos=np.array([2]))
    assert np.array_equal(o[0], V[0])
    # no admissible key -> zero output, lse = -inf (reading)
    o, lse = oracle.attend_rows(rnd(12, 1, d), K, V, np.array([5, 9]), 0.7, row_pos=np.array([1]))
    assert np.all(o == 0) and lse[0] == -np.inf


def test_softmax_rows_sum_to_one_via_value_indicator():
    # with V = I the output row is the softmax weight vector itself
    N, d = 40, 7
    K = rnd(13, N, d)
    V = np.eye(N)
    o, _ = oracle.attend_rows(rnd(14, 6, d), K, V, np.arange(N), 1.3, row_pos=np.arange(6) * 7)
    assert np.allclose(o.sum(1), 1.0, atol=1e-12)
    assert np.all(o >= 0)
    for r in range(6):
        assert np.all(o[r, r * 7 + 1:] == 0)


# ------------------------------------------------------------------ block estimate
def test_pooled_score_is_mean_of_block_of_full_scores():
    """Mean pooling commutes with the product ("MInference 1.0" article,
    §方法介紹): Qbar_i . Kbar_j = mean over the 64x64 block of Q K^T."""
    bs, nb, d = 64, 3, 16
    N = bs * nb
    Hq, Hkv = 4, 2
    Q, K = rnd(15, 1, Hq, N, d), rnd(16, 1, Hkv, N, d)
    S = oracle.block_scores(Q, K, bs, 0.25)
    for h in range(Hq):
        g = h * Hkv // Hq
        full = Q[0, h] @ K[0, g].T * 0.25
        for i in range(nb):
            for j in range(nb):
                if j > i:
                    assert S[0, h, i, j] == -np.inf
                else:
                    blk = full[i * bs:(i + 1) * bs, j * bs:(j + 1) * bs].mean()
                    assert abs(S[0, h, i, j] - blk) < 1e-12


def test_sink_diag_top2_block_count_matches_page_fact():
    g = gold("page_facts.json")["block_grid_sink_diag_top2"]
    nb = g["n_blocks"]
    S = np.random.default_rng(17).standard_normal((1, 1, nb, nb))
    kept = oracle.block_select(S, n_sink=1, n_local=1, k=2)
    counts = [len(x) for x in kept[0][0]]
    assert counts == g["kept_per_row"]
    assert sum(counts) == g["kept_total"]
    for i, blks in enumerate(kept[0][0]):
        assert 0 in blks and i in blks
        assert list(blks) == sorted(blks)


def test_ratio_budget_is_ceiling():
    for n in range(1, 300):
        for num, den in [(10, 100), (5, 100), (1, 4), (1, 3)]:
            assert oracle.ratio_budget(n, num, den) == math.ceil(n * num / den - 1e-12)


# ------------------------------------------------------------------ top-k
def brute_topk(s, k, forced):
    pool = [i for i in range(len(s)) if i not in set(forced)]
    k = min(k, len(pool))
    best = None
    for comb in itertools.combinations(pool, k):   # lexicographic order
        tot = sum(s[i] for i in comb)
        if best is None or tot > best[0]:
            best = (tot, comb)
    return sorted(list(forced) + list(best[1]))


@pytest.mark.parametrize("kind", ["normal", "ties"])
def test_topk_equals_bruteforce_max_sum_lexicographic(kind):
    r = np.random.default_rng(18)
    for trial in range(60):
        n = int(r.integers(1, 12))
        s = W.score_rows(100 + trial, 1, n, kind)[0].astype(np.float64)
        if kind == "ties":
            s = np.round(s)          # integers: sums are exact, ties stay ties
        k = int(r.integers(0, n + 1))
        nf = int(r.integers(0, min(3, n) + 1))
        forced = np.sort(r.choice(n, size=nf, replace=False))
        got = oracle.topk_row(s, k, forced)
        assert list(got) == brute_topk(list(s), k, list(forced))


def test_topk_signed_zero_and_nan():
    s = np.array([0.0, -0.0, 0.0, -0.0])
    assert list(oracle.topk_row(s, 2, np.zeros(0, np.int64))) == [0, 1]
    with pytest.raises(ValueError):
        oracle.topk_row(np.array([1.0, np.nan]), 1, np.zeros(0, np.int64))


def test_forced_set_and_budget_rules():
    assert list(oracle.forced_set(10, 1, 4)) == [0, 6, 7, 8, 9]
    assert list(oracle.forced_set(3, 1, 4)) == [0, 1, 2]
    assert oracle.budget(10, 5, None, (10, 100)) == 1
    assert oracle.budget(3, 3, None, (10, 100)) == 0
    assert oracle.candidate_count(5, 100, True, 4, 10) == 12
    assert oracle.candidate_count(5, 100, False) == 100


def test_certified_gap():
    s = np.array([5.0, 4.0, 3.0, 2.999])
    none = np.zeros(0, np.int64)
    assert oracle.certified_row(s, 2, none)           # gap 1 > 1e-3*5
    assert not oracle.certified_row(s, 3, none)       # gap 0.001 < 0.005
    assert oracle.certified_row(s, 4, none)           # keeps everything


# ------------------------------------------------------------------ vertical-slash
def test_vs_scores_sum_to_number_of_rows_and_match_loops():
    N, d, L = 96, 6, 8
    K = rnd(19, N, d)
    q = rnd(20, L, d)
    pos = np.arange(N - L, N)
    a_v, a_s = oracle.vs_estimate(q, K, pos, 0.4)
    assert abs(a_v.sum() - L) < 1e-12 and abs(a_s.sum() - L) < 1e-12
    assert np.all(a_v >= 0) and np.all(a_s >= 0)
    # independent loop: softmax weights per (row, column), then bin by offset
    av2, as2 = np.zeros(N), np.zeros(N)
    for r in range(L):
        s = [0.4 * sum(q[r, x] * K[c, x] for x in range(d)) for c in range(pos[r] + 1)]
        m = max(s)
        e = [math.exp(v - m) for v in s]
        z = sum(e)
        for c in range(pos[r] + 1):
            av2[c] += e[c] / z
            as2[pos[r] - c] += e[c] / z
    assert np.max(np.abs(a_v - av2)) < 1e-12
    assert np.max(np.abs(a_s - as2)) < 1e-12


def test_vs_block_keys_match_definition_by_brute_force():
    bs, N = 64, 512
    r = np.random.default_rng(21)
    for trial in range(5):
        cols = np.sort(r.choice(N, size=20, replace=False))
        offs = np.sort(r.choice(N, size=6, replace=False))
        for i in range(N // bs):
            ivs, vert = oracle.vs_block_keys(cols, offs, i, bs)
            # intervals are disjoint, sorted, non-adjacent after merging
            for (a0, b0), (a1, b1) in zip(ivs, ivs[1:]):
                assert b0 < a1
            got = set(vert.tolist()) | {c for a, b in ivs for c in range(a, b)}
            want = set()
            for c in range(N):
                on_slash = any(i * bs - o <= c < i * bs - o + bs for o in offs)
                on_vert = c in set(cols.tolist()) and c <= i * bs + bs - 1
                if on_slash or on_vert:
                    want.add(c)
            assert got == want
            assert not (set(vert.tolist()) & {c for a, b in ivs for c in range(a, b)})


def test_vs_everything_kept_equals_dense_causal():
    bs, N, d = 64, 192, 5
    Q, K, V = rnd(22, 1, 1, N, d), rnd(23, 1, 1, N, d), rnd(24, 1, 1, N, d)
    sel = [[(np.arange(N), np.arange(N))]]
    O, L = oracle.vs_attention(Q, K, V, sel, bs, 0.5)
    On, Ln = naive_masked_attention(Q[0, 0], K[0, 0], V[0, 0], np.tril(np.ones((N, N), bool)), 0.5)
    assert np.max(np.abs(O[0, 0] - On)) < 1e-12


def test_vs_slash_only_offset_zero_is_block_diagonal():
    # offset 0 alone gives each block its own diagonal tile
    bs, N, d = 64, 128, 4
    Q, K, V = rnd(25, 1, 1, N, d), rnd(26, 1, 1, N, d), rnd(27, 1, 1, N, d)
    O, _ = oracle.vs_attention(Q, K, V, [[(np.zeros(0, np.int64), np.array([0]))]], bs, 1.0)
    kept = [[[np.array([0]), np.array([1])]]]
    Ob, _ = oracle.block_sparse_attention(Q, K, V, kept, bs, 1.0)
    assert np.max(np.abs(O - Ob)) < 1e-13



# ------------------------------------------------------------------ adaptive budget
def brute_mass_count(s, mass):
    """Fewest candidates of ANY subset whose softmax share reaches ``mass``,
    by enumerating subsets; shares are exactly rounded sums (math.fsum) of
    math.exp over the row.  Returns (count, best share of that size)."""
    n = len(s)
    m = max(s)
    e = [math.exp(x - m) for x in s]
    tot = math.fsum(e)
    for c in range(1, n + 1):
        best = max(math.fsum(e[i] for i in comb) for comb in itertools.combinations(range(n), c))
        if best >= mass * tot:
            return c, best / tot
    return n, 1.0


def test_mass_count_equals_bruteforce_fewest_subset():
    r = np.random.default_rng(41)
    checked = 0
    for trial in range(150):
        n = int(r.integers(1, 11))
        s = r.normal(0.0, float(r.choice([0.3, 1.0, 3.0])), n)
        mass = float(r.uniform(0.05, 1.0))
        if oracle.mass_margin(s, mass) < 1e-9:
            continue
        c = oracle.mass_count(s, mass)
        bc, share = brute_mass_count(list(s), mass)
        assert c == bc
        sel = oracle.mass_row(s, mass)
        assert list(sel) == list(oracle.topk_row(s, c, np.zeros(0, np.int64)))
        w = np.exp(s - s.max())
        assert abs(w[sel].sum() / w.sum() - share) < 1e-12    # the kept prefix is a best subset
        checked += 1
    assert checked > 120


def test_mass_count_uniform_row_is_ceiling():
    for n in range(1, 41):
        for j in range(1, 9):
            s = np.full(n, 0.7)
            assert oracle.mass_count(s, j / 8) == math.ceil(j * n / 8)
            assert list(oracle.mass_row(s, j / 8)) == list(range(math.ceil(j * n / 8)))


def test_mass_count_geometric_closed_form():
    # weights 2^-j (scores -j ln 2): the first c hold (1 - 2^-c)/(1 - 2^-n) of the mass
    r = np.random.default_rng(42)
    for n in (1, 2, 5, 17, 30):
        for c in range(1, n + 1):
            mass = (1.0 - 1.5 * 2.0 ** -c) / (1.0 - 2.0 ** -n)
            perm = r.permutation(n)
            s = np.empty(n)
            s[perm] = -np.arange(n) * math.log(2.0)
            assert oracle.mass_count(s, mass) == c
            assert list(oracle.mass_row(s, mass)) == sorted(perm[:c])


def test_mass_count_invariants_and_special_rows():
    r = np.random.default_rng(43)
    for trial in range(40):
        n = int(r.integers(2, 200))
        s = r.normal(0, 2, n)
        prev = 0
        for mass in (0.1, 0.3, 0.5, 0.7, 0.9, 1.0):
            c = oracle.mass_count(s, mass)
            assert prev <= c <= n                      # monotone in the mass
            prev = c
            if oracle.mass_margin(s, mass) > 1e-9:      # a common shift leaves the softmax alone
                assert oracle.mass_count(s + 1000.25, mass) == c
        assert oracle.mass_count(s, 1.0) == n          # moderate range: every weight is positive
        assert oracle.mass_count(s, 0.9, k_min=n) == n
        assert oracle.mass_count(s, 0.9, k_max=1) == 1
    dom = np.zeros(16)
    dom[5] = 60.0
    assert list(oracle.mass_row(dom, 0.99)) == [5]
    inf2 = np.array([0.0, np.inf, 3.0, np.inf])        # the +inf entries share everything
    assert list(oracle.mass_row(inf2, 0.5)) == [1]
    assert list(oracle.mass_row(inf2, 0.51)) == [1, 3]
    assert list(oracle.mass_row(np.full(6, -np.inf), 0.5)) == [0, 1, 2]   # uniform
    assert list(oracle.mass_row(np.array([1.0, -np.inf, 1.0]), 1.0)) == [0, 2]
    with pytest.raises(ValueError):
        oracle.mass_count(np.array([1.0, np.nan]), 0.5)


# ------------------------------------------------------------------ A-shape and per-head patterns
def ashape_mask(N, bs, n_sink, n_local):
    """Token-level A-shape mask from its definition: key c is visible to row
    r when c <= r and c lies in the first n_sink blocks or in the n_local
    blocks ending at r's block."""
    m = np.zeros((N, N), bool)
    for r in range(N):
        for c in range(r + 1):
            m[r, c] = c < bs * n_sink or c >= bs * (r // bs - n_local + 1)
    return m


@pytest.mark.parametrize("n_sink,n_local", [(1, 2), (0, 1), (2, 3), (1, 100), (0, 0)])
def test_ashape_matches_token_mask(n_sink, n_local):
    bs, N, d = 4, 32, 5
    Q, K, V = rnd(71, 1, 2, N, d), rnd(72, 1, 1, N, d), rnd(73, 1, 1, N, d)
    O, L = oracle.ashape_attention(Q, K, V, n_sink, n_local, bs, 0.6)
    mask = ashape_mask(N, bs, n_sink, n_local)
    for h in range(2):
        On, Ln = naive_masked_attention(Q[0, h], K[0, 0], V[0, 0], mask, 0.6)
        assert np.max(np.abs(O[0, h] - On)) < 1e-12
        assert np.array_equal(np.isneginf(L[0, h]), np.isneginf(Ln))
        fin = np.isfinite(Ln)
        assert np.max(np.abs(L[0, h][fin] - Ln[fin]), initial=0.0) < 1e-12
    if n_local >= N // bs:                      # the window covers every causal block: dense causal
        Od, _ = naive_masked_attention(Q[0, 0], K[0, 0], V[0, 0], np.tril(np.ones((N, N), bool)), 0.6)
        assert np.max(np.abs(O[0, 0] - Od)) < 1e-12


def test_mixed_layer_heads_match_single_pattern_layers():
    """Each head of a mixed layer equals the same head of a layer that runs
    its pattern on every head (independent slicing and KV-head mapping)."""
    bs, N, d, Hq, Hkv = 8, 64, 6, 4, 2
    Q, K, V = rnd(81, 1, Hq, N, d), rnd(82, 1, Hkv, N, d), rnd(83, 1, Hkv, N, d)
    scale = 0.5
    block = dict(n_sink=1, n_local=1, k=2)
    pats = ["BS", "A", "VS", "BS"]
    O, L, sel = oracle.mixed_layer(Q, K, V, pats, bs=bs, scale=scale, a_shape=(1, 2), block=block,
                                   vslash=(9, 5), last_q=8)
    Ob, _ = oracle.block_sparse_attention(Q, K, V, oracle.block_select(oracle.block_scores(Q, K, bs, scale),
                                                                         **block), bs, scale)
    Oa, _ = oracle.ashape_attention(Q, K, V, 1, 2, bs, scale)
    vsel = [[oracle.vs_select(*oracle.vs_estimate(Q[0, h, N - 8:], K[0, h * Hkv // Hq], np.arange(N - 8, N), scale),
                              9, 5) for h in range(Hq)]]
    Ov, _ = oracle.vs_attention(Q, K, V, vsel, bs, scale)
    ref = {"BS": Ob, "A": Oa, "VS": Ov}
    for h, p in enumerate(pats):
        assert np.max(np.abs(O[0, h] - ref[p][0, h])) < 1e-12, (h, p)
    assert list(sel[0][1][5]) == [0, 4, 5]


# ------------------------------------------------------------------ offline k-means
def test_kmeans_equals_scipy_lloyd():
    from scipy.cluster.vq import kmeans2
    r = np.random.default_rng(61)
    for trial in range(6):
        C, d, N = int(r.integers(2, 9)), int(r.integers(2, 12)), int(r.integers(20, 300))
        X = np.concatenate([r.normal(r.normal(0, 3, d), 1.0, (N // C + 1, d)) for _ in range(C)])[:N]
        mu0 = X[r.choice(N, C, replace=False)] + 0.01
        it = int(r.integers(1, 6))
        mu, lab, margins = oracle.kmeans(X, mu0, it)
        if margins.min() < 1e-9:
            continue
        with np.errstate(all="ignore"):
            import warnings
            with warnings.catch_warnings():
                warnings.simplefilter("ignore")
                smu, slab = kmeans2(X, mu0.copy(), iter=it, minit="matrix", missing="warn")
        assert np.array_equal(lab, slab)
        assert np.max(np.abs(mu - smu)) < 1e-12


def test_kmeans_separated_mixture_closed_form_and_fixed_point():
    r = np.random.default_rng(62)
    C, d, N = 6, 16, 600
    means = r.normal(0, 1, (C, d)) * 10
    true = r.integers(0, C, N)
    X = means[true] + r.normal(0, 0.3, (N, d))
    mu, lab, _ = oracle.kmeans(X, means + 0.5, 1)
    assert np.array_equal(lab, true)
    for c in range(C):
        assert np.max(np.abs(mu[c] - X[true == c].mean(axis=0))) < 1e-12
    mu2, lab2, _ = oracle.kmeans(X, mu, 3)
    assert np.array_equal(lab2, true) and np.max(np.abs(mu2 - mu)) < 1e-12


def test_kmeans_objective_never_increases_and_empty_and_tied_clusters():
    r = np.random.default_rng(63)
    X = r.normal(0, 1, (400, 5))
    mu = X[:7].copy()
    prev = np.inf
    for _ in range(6):
        mu_next, lab, _ = oracle.kmeans(X, mu, 1)
        obj = oracle.kmeans_objective(X, mu_next, lab)
        assert obj <= prev + 1e-9
        prev, mu = obj, mu_next
    far = np.vstack([X[:3], np.full((1, 5), 1e6)])            # a centroid no key is near
    mu_f, lab_f, _ = oracle.kmeans(X, far, 2)
    assert np.all(lab_f != 3) and np.array_equal(mu_f[3], far[3])
    dup = np.vstack([X[:1], X[:1], X[1:2]])                   # equal centroids: the lower index wins
    _, lab_d, _ = oracle.kmeans(X, dup, 1)
    assert not np.any(lab_d == 1)

# ------------------------------------------------------------------ clustered decode
def test_cluster_rule_from_page():
    g = gold("page_facts.json")["squeezed_cluster_rule"]
    assert math.isqrt(g["context_len"]) == g["clusters"]
    assert g["clusters"] // 4 == g["select_min"] and g["clusters"] // 2 == g["select_max"]


def test_all_clusters_equal_dense_decode():
    inp = W.decode_clustered(31, T=2, Hq=4, Hkv=2, Nctx=80, d=6, C=5)
    q = W.bf16_to_f32(inp.q).astype(np.float64)
    K = W.bf16_to_f32(inp.k).astype(np.float64)
    V = W.bf16_to_f32(inp.v).astype(np.float64)
    sel = [[np.arange(5) for _ in range(4)] for _ in range(2)]
    O, L = oracle.cluster_decode(q, K, V, inp.labels, sel, 0.4)
    for t in range(2):
        for h in range(4):
            g = h * 2 // 4
            On, Ln = naive_masked_attention(q[t, h][None], K[g], V[g], np.ones((1, 80), bool), 0.4)
            assert np.max(np.abs(O[t, h] - On[0])) < 1e-12
            assert abs(L[t, h] - Ln[0]) < 1e-12


def test_cluster_subset_equals_masked_dense_decode():
    inp = W.decode_clustered(32, T=1, Hq=2, Hkv=1, Nctx=60, d=4, C=6)
    q = W.bf16_to_f32(inp.q).astype(np.float64)
    K = W.bf16_to_f32(inp.k).astype(np.float64)
    V = W.bf16_to_f32(inp.v).astype(np.float64)
    s = oracle.centroid_scores(q, inp.centroids, 0.5)
    sel = oracle.cluster_select(s, 2)
    O, _ = oracle.cluster_decode(q, K, V, inp.labels, sel, 0.5)
    for h in range(2):
        # brute force: best two clusters by loop over all pairs
        sc = [0.5 * sum(float(q[0, h, x]) * float(inp.centroids[0, c, x]) for x in range(4)) for c in range(6)]
        best = max(itertools.combinations(range(6), 2), key=lambda p: (sc[p[0]] + sc[p[1]], [-p[0], -p[1]]))
        assert list(sel[0][h]) == sorted(best)
        mask = np.array([[inp.labels[0, t] in best for t in range(60)]])
        On, _ = naive_masked_attention(q[0, h][None], K[0], V[0], mask, 0.5)
        assert np.max(np.abs(O[0, h] - On[0])) < 1e-12


def test_cluster_pack_is_stable_cluster_major_permutation():
    r = np.random.default_rng(33)
    labels = r.integers(0, 7, size=(2, 200))
    ptr, perm = oracle.cluster_pack(labels, 7)
    for g in range(2):
        assert sorted(perm[g].tolist()) == list(range(200))
        lab = labels[g][perm[g]]
        assert all(lab[i] <= lab[i + 1] for i in range(199))
        for c in range(7):
            seg = perm[g, ptr[g, c]:ptr[g, c + 1]]
            assert list(seg) == [t for t in range(200) if labels[g, t] == c]


# ------------------------------------------------------------------ indexer + index cache
def test_indexer_matches_loops_and_is_nonnegative():
    T, Hi, di, N = 3, 2, 4, 10
    qi = W.integer_bf16(40, (T, Hi, di), -4, 4, 0)
    ki = W.integer_bf16(40, (N, di), -4, 4, 1)
    w = np.array([0.25, 0.75], np.float32)
    qf, kf = W.bf16_to_f32(qi), W.bf16_to_f32(ki)
    pos0 = N - T
    I = oracle.indexer_scores(qf, kf, w, pos0)
    for t in range(T):
        for s in range(N):
            if s > pos0 + t:
                assert I[t, s] == -np.inf
                continue
            want = 0.0
            for h in range(Hi):
                dot = sum(float(qf[t, h, x]) * float(kf[s, x]) for x in range(di))
                want += float(w[h]) * max(0.0, dot)
            assert I[t, s] == want           # integer inputs, w = m/4: exact
            assert I[t, s] >= 0


def test_indexer_one_hot_weight_is_relu_of_one_head():
    T, Hi, di, N = 4, 3, 8, 20
    qi = np.random.default_rng(41).standard_normal((T, Hi, di))
    ki = np.random.default_rng(42).standard_normal((N, di))
    w = np.array([0.0, 1.0, 0.0])
    I = oracle.indexer_scores(qi, ki, w, N - T)
    ref = np.maximum(qi[:, 1, :] @ ki.T, 0.0)
    for t in range(T):
        n = N - T + t + 1
        assert np.allclose(I[t, :n], ref[t, :n], atol=1e-13)


def test_planted_indexer_selects_hot_set_and_is_certified():
    T, Hi, di, N, k = 32, 4, 32, 4096, 64
    inp = W.indexer_planted(43, T, Hi, di, N, k, n_dir=8)
    I = oracle.indexer_scores(W.bf16_to_f32(inp.qi), W.bf16_to_f32(inp.ki), inp.w, inp.pos0)
    sel = oracle.indexer_select(I, np.arange(T), inp.pos0, k)
    kf = W.bf16_to_f32(inp.ki)
    for t in range(T):
        g = t % 8
        hot = np.nonzero(kf[:, g] > 2.0)[0]
        assert list(sel[t]) == list(hot)
        assert oracle.certified_row(I[t, :inp.pos0 + t + 1], k, np.zeros(0, np.int64))


def test_index_cache_reuses_full_layer_indices():
    g = gold("page_facts.json")["indexcache_layer_pattern"]
    T, Hi, di, N, k, Hq, d = 4, 2, 8, 64, 8, 3, 6
    ind = W.indexer_random(44, T, Hi, di, N)
    qi, ki = W.bf16_to_f32(ind.qi), W.bf16_to_f32(ind.ki)
    layers = []
    for l in range(g["layers"]):
        L = W.mqa_layer(44, l, T, Hq, 1, N, d)
        layers.append((W.bf16_to_f32(L.q), W.bf16_to_f32(L.k), W.bf16_to_f32(L.v)))
    outs, used = oracle.index_cache_forward(layers, set(g["full_layers"]), qi, ki, ind.w, ind.pos0, k, 0.5)
    for l in range(1, g["layers"]):
        assert all(np.array_equal(a, b) for a, b in zip(used[0], used[l]))
    assert 1 - len(g["full_layers"]) / g["layers"] == g["indexer_work_removed"]
    # each layer equals the plain gathered attention over layer 0's indices
    for l, (Q, K, V) in enumerate(layers):
        for t in range(T):
            keys = used[0][t]
            for h in range(Hq):
                mask = np.zeros((1, N), bool)
                mask[0, keys] = True
                On, _ = naive_masked_attention(Q[t, h][None], K[0], V[0], mask, 0.5)
                assert np.max(np.abs(outs[l][t, h] - On[0])) < 1e-12


def test_quadratic_cost_fact():
    g = gold("page_facts.json")["indexcache_quadratic_cost"]
    assert (g["n_large"] / g["n_small"]) ** 2 == g["ratio"]


# ------------------------------------------------------------------ generators
def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 3.0e38, 1.0 + 2 ** -7], np.float32)
    b = W.f32_to_bf16(x)
    assert b.tolist() == [0x3F80, 0x3F80, 0x3F82, 0xC020, 0x7F62, 0x3F81]
    y = W.bf16_to_f32(b)
    assert y[3] == -2.5


def test_substreams_are_addressable():
    a = W.prefill_bf16(50, 1, 4, 2, 128, 8)
    b = W.prefill_bf16(50, 1, 4, 2, 128, 8, heads=[2])
    assert np.array_equal(a.q[0, 2], b.q[0, 2])
    assert np.array_equal(a.k, b.k)
    assert len(a.shift_pos) == 1 and abs(np.linalg.norm(a.u) - 1) < 1e-6
