"""GPU parity of the adaptive cluster budget (sa_select_mass) and of the
clustered decode that uses it, against the CPU oracle.

The count is an integer decided by fp32 weights (summed exactly in fixed
point) on the GPU and fp64 weights and sums in the oracle.  Where the oracle's prefix shares keep more than MARGIN away from the
requested mass, both must find the same count; elsewhere the GPU's count must
be one the oracle finds for a mass within MARGIN, and its set must be exactly
the oracle's top-c for that count (the order itself is exact on both sides)."""
import math

import numpy as np
import pytest

import oracle
import workloads as W
from gpu_helpers import assert_attention_close, dev_bf16, dev_f32, dev_i32, host, torch

pytestmark = pytest.mark.gpu

MARGIN = 1e-5   # fp32 exponentials (a few 1e-7 relative) plus 2^-40 rounding per weight


@pytest.fixture(scope="module")
def sa():
    import dynamic_sparse_attention_pool_amd as m
    m.load()
    return m


def run_mass(sa, scores, mass, k_min, k_max, kmax=None, ncand=None):
    t = torch()
    R = scores.shape[0]
    n = scores.shape[1] if ncand is None else ncand
    kmax = min(k_max, n) if kmax is None else kmax
    idx = t.full((R, kmax), 7, dtype=t.int32, device="cuda:0")
    cnt = t.full((R,), -5, dtype=t.int32, device="cuda:0")
    err = t.zeros(1, dtype=t.int32, device="cuda:0")
    sa.sa_select_mass(dev_f32(scores), idx, cnt, mass=mass, k_min=k_min, k_max=k_max, ncand=ncand, err_flag=err)
    t.cuda.synchronize()
    return host(idx), host(cnt), int(host(err)[0])


def check_rows(scores, idx, cnt, mass, k_min, k_max, ncand=None):
    n = scores.shape[1] if ncand is None else ncand
    exact = 0
    for r in range(scores.shape[0]):
        s = scores[r, :n].astype(np.float64)
        c = int(cnt[r])
        assert np.all(idx[r, c:] == -1), r
        got = idx[r, :c]
        if oracle.mass_margin(s, mass) > MARGIN:
            assert list(got) == list(oracle.mass_row(s, mass, k_min, k_max)), r
            exact += 1
        else:
            lo = oracle.mass_count(s, max(mass - MARGIN, 1e-12), k_min, k_max)
            hi = oracle.mass_count(s, mass + MARGIN, k_min, k_max)   # above 1: every weight counts
            assert lo <= c <= hi, (r, c, lo, hi)
            assert list(got) == list(oracle.topk_row(s, c, np.zeros(0, np.int64))), r
    return exact


@pytest.mark.parametrize("R,n", [(64, 1), (64, 7), (300, 64), (256, 256), (33, 257), (40, 1000), (16, 4096)])
@pytest.mark.parametrize("kind", ["normal", "ties", "coarse"])
def test_select_mass_matches_oracle(sa, R, n, kind):
    print(f"mass R{R} n{n} {kind}", flush=True)
    for j, (mass, k_min, k_max) in enumerate([(0.5, 1, 64), (0.9, 0, n), (0.3, 4, 16), (1.0, 1, n)]):
        s = W.score_rows(600 + j, R, n, kind) * np.float32(1.0 + 2 * j)
        idx, cnt, err = run_mass(sa, s, mass, k_min, k_max)
        assert err == 0
        exact = check_rows(s, idx, cnt, mass, k_min, k_max)
        if kind == "normal" and mass < 1.0:     # at mass 1 the last weights are below MARGIN
            assert exact >= 0.9 * R


def test_select_mass_special_rows(sa):
    inf = np.inf
    rows = [
        ([0.0, inf, 3.0, inf], 0.5, [1]),           # +inf entries share all the weight
        ([0.0, inf, 3.0, inf], 0.51, [1, 3]),
        ([-inf] * 6, 0.5, [0, 1, 2]),               # all -inf: uniform
        ([1.0, -inf, 1.0, -inf], 1.0, [0, 2]),      # -inf weighs nothing
        ([0.0] * 5 + [60.0] + [0.0] * 2, 0.99, [5]),
        ([-0.0, 0.0, -0.0, 0.0], 0.5, [0, 1]),      # signed zeros tie; lower index first
    ]
    for vals, mass, want in rows:
        s = np.array([vals], np.float32)
        idx, cnt, err = run_mass(sa, s, mass, 0, len(vals))
        assert err == 0 and int(cnt[0]) == len(want) and list(idx[0, :len(want)]) == want, (vals, mass)
    # clamps, ld wider than the candidate range, and a wider output table
    s = W.score_rows(700, 50, 300, "normal")
    for k_min, k_max in [(0, 1), (20, 20), (200, 300)]:
        idx, cnt, _ = run_mass(sa, s, 0.4, k_min, k_max, kmax=k_max + 3, ncand=250)
        check_rows(s, idx, cnt, 0.4, k_min, k_max, ncand=250)
        assert np.all((cnt >= min(k_min, 250)) & (cnt <= k_max))
    # NaN is flagged
    s = W.score_rows(701, 4, 100, "normal")
    s[2, 17] = np.nan
    _, _, err = run_mass(sa, s, 0.5, 1, 10)
    assert err == 1


def test_select_mass_no_rows_is_a_noop(sa):
    t = torch()
    idx = t.full((0, 4), 7, dtype=t.int32, device="cuda:0")
    cnt = t.zeros(0, dtype=t.int32, device="cuda:0")
    sa.sa_select_mass(t.zeros((0, 10), dtype=t.float32, device="cuda:0"), idx, cnt, mass=0.5, k_max=4)
    t.cuda.synchronize()


def mass_certified(s, mass, k_min, k_max, gap_rel=1e-3):
    """The count stays put for masses within 1e-4 and the score gap at the
    cut exceeds gap_rel of the row scale: scores perturbed by the estimator's
    error (far below both) select the same clusters."""
    c = oracle.mass_count(s, mass, k_min, k_max)
    if oracle.mass_count(s, mass - 1e-4, k_min, k_max) != c or oracle.mass_count(s, mass + 1e-4, k_min, k_max) != c:
        return False
    return oracle.certified_row(s, c, np.zeros(0, np.int64), gap_rel)


@pytest.mark.parametrize("T,Hq,Hkv,C,d,k_min,k_max,mass,dt", [(3, 8, 2, 256, 128, 1, 64, 0.5, "bf16"),
                                                                (2, 4, 4, 100, 64, 0, 100, 0.9, "f32"),
                                                                (2, 16, 2, 1024, 128, 3, 200, 0.2, "bf16"),
                                                                (1, 8, 1, 37, 128, 37, 37, 0.5, "bf16")])
def test_fused_centroid_mass_matches_separate_path_and_oracle(sa, T, Hq, Hkv, C, d, k_min, k_max, mass, dt):
    """sa_estimate_topk(CENTROID) with a mass: the same clusters and counts as
    sa_estimate(CENTROID) + sa_select_mass, bit for bit (same score
    arithmetic), and the oracle's counts and sets up to the margin."""
    t = torch()
    r = np.random.default_rng(95 + C)
    qf = r.standard_normal((T, Hq, d)).astype(np.float32)
    cent = (r.standard_normal((Hkv, C, d)) * 0.7).astype(np.float32)
    q = dev_bf16(W.f32_to_bf16(qf)) if dt == "bf16" else dev_f32(qf)
    qh = W.bf16_to_f32(W.f32_to_bf16(qf)) if dt == "bf16" else qf
    scale = 1 / math.sqrt(d)
    kmax = min(k_max, C)
    sel = t.full((T, Hq, kmax), 9, dtype=t.int32, device="cuda:0")
    cnt = t.full((T, Hq), -3, dtype=t.int32, device="cuda:0")
    err = t.zeros(1, dtype=t.int32, device="cuda:0")
    sa.sa_estimate_topk_centroid(q, dev_f32(cent), sel, cnt, k=k_max, scale=scale, mass=mass, k_min=k_min,
                                 err_flag=err)
    scores = t.empty((T, Hq, C), dtype=t.float32, device="cuda:0")
    sa.sa_estimate(sa.CENTROID, q, q, scores, centroids=dev_f32(cent), scale=scale)
    sel2 = t.full((T * Hq, kmax), 9, dtype=t.int32, device="cuda:0")
    cnt2 = t.full((T * Hq,), -3, dtype=t.int32, device="cuda:0")
    sa.sa_select_mass(scores.view(-1, C), sel2, cnt2, mass=mass, k_min=k_min, k_max=k_max)
    t.cuda.synchronize()
    assert int(host(err)[0]) == 0
    assert np.array_equal(host(sel).reshape(T * Hq, kmax), host(sel2)) and np.array_equal(host(cnt).ravel(), host(cnt2))
    s = oracle.centroid_scores(qh, cent, scale).reshape(T * Hq, C)
    check_rows(s, host(sel).reshape(T * Hq, kmax), host(cnt).ravel(), mass, k_min, k_max)


@pytest.mark.parametrize("fused", [False, True])
def test_adaptive_decode_full_size_certified(sa, fused):
    """8 queries x 32/8 heads over 65536 clustered keys, 256 centroids: the
    clusters holding half of the softmax weight of the centroid scores, at
    least 1 and at most 64, then the gathered attention over them (scores and
    selection as two calls, or in one)."""
    from dynamic_sparse_attention_pool_amd.pipelines import ClusterDecode
    seed = W.CONFIG_SEEDS[4]
    T, Hq, Hkv, N, d, C, kcap, mass = 8, 32, 8, 65536, 128, 256, 64, 0.5
    inp = W.decode_clustered(seed, T, Hq, Hkv, N, d, C)
    scale = 1 / math.sqrt(d)
    for t in range(T):
        for h in range(Hq):
            g = h * Hkv // Hq
            a = 0
            while not mass_certified(oracle.centroid_scores(W.bf16_to_f32(inp.q[t:t + 1, h:h + 1]),
                                                            inp.centroids[g:g + 1], scale)[0, 0], mass, 1, kcap):
                a += 1
                assert a < 200
                inp.q[t, h] = W.redraw_decode_query(seed, t, h, 1000 + a, d)
    dc = ClusterDecode(dev_bf16(inp.q), dev_bf16(inp.k), dev_bf16(inp.v), dev_i32(inp.labels),
                       dev_f32(inp.centroids), n_sel=kcap, mass=mass, k_min=1, with_lse=True, fused=fused)
    dc.step()
    torch().cuda.synchronize()
    s = oracle.centroid_scores(W.bf16_to_f32(inp.q), inp.centroids, scale)
    sel = oracle.cluster_select_mass(s, mass, 1, kcap)
    got, cnt = host(dc.sel), host(dc.sel_cnt).reshape(T, Hq)
    counts = []
    for t in range(T):
        for h in range(Hq):
            c = len(sel[t][h])
            counts.append(c)
            assert cnt[t, h] == c and np.array_equal(got[t, h, :c], sel[t][h]), (t, h)
            assert np.all(got[t, h, c:] == -1)
    assert min(counts) < max(counts)          # the budget does adapt across heads
    wo, wl = oracle.cluster_decode(W.bf16_to_f32(inp.q), W.bf16_to_f32(inp.k), W.bf16_to_f32(inp.v), inp.labels,
                                   sel, scale)
    assert_attention_close(host(dc.out), wo, bf16=True, what="adaptive decode")
    assert np.max(np.abs(host(dc.lse) - wl)) < 1e-3
