"""GPU parity of the fused indexer top-k (sa_indexer_topk) against the CPU
oracle, and against the two-call path (sa_estimate INDEXER + sa_select_topk).

The fused call keeps every key of a row of at most 8192 keys; for a longer
row it scores every 16th key first, takes the 256th largest causal sampled
score as a threshold, keeps the keys at or above it in per-chunk runs and
selects exactly among them.  On inputs whose scores are
exact in fp32 (small integers, weights m/64) the GPU scores equal the oracle's,
so the outcome of that bracket is known in advance: `predict_failed` applies
the same rule to the oracle's scores, and rows must fail exactly where it says
and equal the oracle's top-k everywhere else."""
import math

import numpy as np
import pytest

import oracle
import workloads as W
from gpu_helpers import dev_bf16, dev_f32, host, tie_tolerant_valid, torch

pytestmark = pytest.mark.gpu

STRIDE, CHUNK, SEL_CAP, RANK = 16, 8192, 8192, 256
EXPECT = STRIDE * RANK


@pytest.fixture(scope="module")
def sa():
    import dynamic_sparse_attention_pool_amd as m
    m.load()
    return m


def run_fused(sa, qi, ki, w, pos0, k, kmax=None):
    t = torch()
    T, N = qi.shape[0], ki.shape[0]
    kmax = kmax or min(k, N)
    idx = t.full((T, kmax), -7, dtype=t.int32, device="cuda:0")
    cnt = t.full((T,), -7, dtype=t.int32, device="cuda:0")
    err = t.zeros(1, dtype=t.int32, device="cuda:0")
    sa.sa_indexer_topk(dev_bf16(qi), dev_bf16(ki), idx, cnt, weights=dev_f32(w), q_pos0=pos0, k=k, err_flag=err)
    t.cuda.synchronize()
    return host(idx), host(cnt), int(host(err)[0])


def run_two_call(sa, qi, ki, w, pos0, k, kmax=None):
    t = torch()
    T, N = qi.shape[0], ki.shape[0]
    kmax = kmax or min(k, N)
    scores = t.empty((T, N), dtype=t.float32, device="cuda:0")
    sa.sa_estimate(sa.INDEXER, dev_bf16(qi), dev_bf16(ki), scores, weights=dev_f32(w), q_pos0=pos0)
    idx = t.empty((T, kmax), dtype=t.int32, device="cuda:0")
    cnt = t.empty((T,), dtype=t.int32, device="cuda:0")
    sa.sa_select_topk(scores, idx, cnt, k=k, causal=True, causal_period=T, causal_offset=pos0)
    t.cuda.synchronize()
    return host(idx), host(cnt)


def slots(n, c):
    """Slots of chunk c of a row with n causal keys (twice its share of the
    4096 expected kept keys, plus 64, rounded up to 64, at most the chunk's
    keys)."""
    ln = min(CHUNK, n - c * CHUNK)
    share = -(-2 * EXPECT * ln // n)
    return min(ln, -(-share // 64) * 64 + 64)


def predict_failed(I_row, n, k):
    """Whether the bracket of a row with exact scores I_row[:n] fails."""
    if k >= n or n <= SEL_CAP:
        return False
    smp = I_row[:n:STRIDE]
    thr = np.sort(smp)[::-1][RANK - 1]
    kept = I_row[:n] >= thr
    total = 0
    for c in range(-(-n // CHUNK)):
        fc = int(kept[c * CHUNK:(c + 1) * CHUNK].sum())
        if fc > slots(n, c):
            return True
        total += fc
    return total > SEL_CAP or total < k


def check_exact(qi, ki, w, pos0, k, idx, cnt, expect_fail=None):
    """Every row against the oracle's exact top-k or the predicted failure."""
    T, N = qi.shape[0], ki.shape[0]
    I = oracle.indexer_scores(W.bf16_to_f32(qi), W.bf16_to_f32(ki), w, pos0)
    sel = oracle.indexer_select(I, np.arange(T), pos0, k)
    failed = 0
    for t in range(T):
        n = min(N, pos0 + t + 1)
        if predict_failed(I[t], n, k):
            assert cnt[t] == -1 and np.all(idx[t] == -1), t
            failed += 1
            continue
        kr = min(k, n)
        assert cnt[t] == kr, (t, cnt[t], kr)
        assert np.array_equal(idx[t, :kr], sel[t]), t
        assert np.all(idx[t, kr:] == -1), t
    if expect_fail is not None:
        assert (failed > 0) == expect_fail, failed
    return failed


@pytest.mark.parametrize("T,Hi,N,back,k,span,unit_w", [(61, 64, 20000, 50, 2048, 4, False),
                                                        (61, 64, 20000, 50, 300, 4, False),
                                                        (50, 32, 9000, 0, 1, 4, False),
                                                        (40, 64, 8192 * 2, 7, 777, 4, False),
                                                        (40, 32, 12000, 0, 500, 1, True),     # ~56 ties at the k-th
                                                        (40, 32, 12000, 0, 1500, 1, True)])   # ~126 ties
def test_indexer_topk_exact_integer_inputs(sa, T, Hi, N, back, k, span, unit_w):
    """Integers in [-span,span] and weights m/64 or 1 (scores exact in fp32;
    with span 1 and unit weights about 120 distinct values, so many keys tie
    at the k-th score): the fused result equals the oracle's top-k row for row
    (ties to the lower index), with the predicted bracket failures only, and
    the two-call path's output bit for bit."""
    qi = W.integer_bf16(91, (T, Hi, 64), -span, span, 0)
    ki = W.integer_bf16(91, (N, 64), -span, span, 1)
    w = (np.ones(Hi) if unit_w else np.random.default_rng(91).integers(0, 65, size=Hi) / 64.0).astype(np.float32)
    pos0 = N - T - back
    idx, cnt, err = run_fused(sa, qi, ki, w, pos0, k)
    failed = check_exact(qi, ki, w, pos0, k, idx, cnt)
    assert (err & 2 != 0) == (failed > 0) and err & 1 == 0
    ridx, rcnt = run_two_call(sa, qi, ki, w, pos0, k)
    ok = cnt >= 0
    assert np.array_equal(idx[ok], ridx[ok]) and np.array_equal(cnt[ok], rcnt[ok])


@pytest.mark.parametrize("T,Hi,N,pos0,k", [(3000, 64, 12000, 6000, 2048),  # every-key and sampled rows
                                           (2500, 32, 2500, 0, 2048),      # prefill from 0: short rows
                                           (100, 64, 50004, 49000, 512),   # ragged last chunk
                                           (64, 64, 40000, 30000, 1)])     # k = 1
def test_indexer_topk_random(sa, T, Hi, N, pos0, k):
    """Random indexer inputs: no row fails; every row equals the two-call
    path's bit for bit; sampled rows against the oracle (certified rows
    exactly, the others as a valid top-k up to near-ties)."""
    ind = W.indexer_random(92, T, Hi, 64, N)
    idx, cnt, err = run_fused(sa, ind.qi, ind.ki, ind.w, pos0, k)
    assert err == 0
    n_rows = np.minimum(N, pos0 + np.arange(T) + 1)
    assert np.array_equal(cnt, np.minimum(k, n_rows))
    ridx, rcnt = run_two_call(sa, ind.qi, ind.ki, ind.w, pos0, k)
    assert np.array_equal(idx, ridx) and np.array_equal(cnt, rcnt)
    # evenly spread rows and the rows on both sides of the every-key / sampled boundary
    edge = np.nonzero(np.diff(n_rows > SEL_CAP))[0]
    rows = np.unique(np.concatenate([np.linspace(0, T - 1, 12).astype(np.int64), edge, edge + 1]))
    I = oracle.indexer_scores(W.bf16_to_f32(ind.qi), W.bf16_to_f32(ind.ki), ind.w, pos0, rows)
    sel = oracle.indexer_select(I, rows, pos0, k)
    none = np.zeros(0, np.int64)
    for r, t in enumerate(rows):
        n = int(n_rows[t])
        got = idx[t, :cnt[t]]
        if oracle.certified_row(I[r, :n], k, none):
            assert np.array_equal(got, sel[r]), t
        else:
            assert tie_tolerant_valid(got, I[r, :n], k, none), t


@pytest.mark.parametrize("T,Hi,N,pos0,k", [(1, 64, 1, 0, 1),          # one key
                                           (5, 32, 17, 12, 16),      # rows of 13..17 keys around k
                                           (3, 64, 40, 0, 2048),     # k above every row
                                           (7, 64, 8200, 8190, 2048),  # rows of 8191..8197 keys: both rules
                                           (9, 32, 8195, 8180, 100)])
def test_indexer_topk_small_and_boundary_rows(sa, T, Hi, N, pos0, k):
    """Exact integer inputs on tiny contexts and on rows around the 8192-key
    boundary between keeping every key and the sampled threshold: every row
    equals the oracle's top-k."""
    qi = W.integer_bf16(97, (T, Hi, 64), -4, 4, 0)
    ki = W.integer_bf16(97, (N, 64), -4, 4, 1)
    w = (np.random.default_rng(97).integers(0, 65, size=Hi) / 64.0).astype(np.float32)
    idx, cnt, err = run_fused(sa, qi, ki, w, pos0, k)
    assert check_exact(qi, ki, w, pos0, k, idx, cnt) == 0 and err == 0


def test_indexer_topk_kmax_padding(sa):
    T, Hi, N, k = 30, 64, 9000, 100
    ind = W.indexer_random(93, T, Hi, 64, N)
    idx, cnt, _ = run_fused(sa, ind.qi, ind.ki, ind.w, ind.pos0, k, kmax=k + 13)
    assert np.all(cnt == k) and np.all(idx[:, k:] == -1)
    ridx, _ = run_two_call(sa, ind.qi, ind.ki, ind.w, ind.pos0, k, kmax=k + 13)
    assert np.array_equal(idx, ridx)


def planted_stride(seed, T, Hi, N, sampled_hot: bool):
    """Exact integer inputs whose scores depend on the key's position modulo
    16: dimension 0 of every query is 4; keys at multiples of 16 get 4 (or 0)
    there and the others 0 (or 4), plus integer noise in [-1,1] elsewhere."""
    qi = W.bf16_to_f32(W.integer_bf16(seed, (T, Hi, 64), -1, 1, 0))
    ki = W.bf16_to_f32(W.integer_bf16(seed, (N, 64), -1, 1, 1))
    qi[:, :, 0] = 4.0
    on = (np.arange(N) % STRIDE == 0) == sampled_hot
    ki[:, 0] = np.where(on, 4.0, 0.0)
    w = (np.random.default_rng(seed).integers(1, 65, size=Hi) / 64.0).astype(np.float32)
    return W.f32_to_bf16(qi), W.f32_to_bf16(ki), w


@pytest.mark.parametrize("sampled_hot", [True, False])
def test_indexer_topk_bracket_failure_is_flagged(sa, sampled_hot):
    """Scores with structure at the sampling period: hot sampled keys leave
    fewer than k keys above the threshold; cold sampled keys put almost every
    key above it and overflow the runs.  The failing rows are exactly the
    predicted ones and carry cnt = -1; err_flag gets 2; the pipeline's checked
    index redoes the chunk with two calls and equals the oracle."""
    from dynamic_sparse_attention_pool_amd.pipelines import IndexerPrefill
    T, Hi, N, k = 48, 64, 24000, 1024
    qi, ki, w = planted_stride(94, T, Hi, N, sampled_hot)
    pos0 = N - T
    idx, cnt, err = run_fused(sa, qi, ki, w, pos0, k)
    failed = check_exact(qi, ki, w, pos0, k, idx, cnt, expect_fail=True)
    assert failed == T and err & 2
    L = W.mqa_layer(94, 0, T, 16, 1, N, 128)
    layers = [(dev_bf16(L.q), dev_bf16(L.k), dev_bf16(L.v))]
    ip = IndexerPrefill(dev_bf16(qi), dev_bf16(ki), dev_f32(w), pos0, layers, k_sel=k, fused=True)
    ip.index(check=True)
    torch().cuda.synchronize()
    I = oracle.indexer_scores(W.bf16_to_f32(qi), W.bf16_to_f32(ki), w, pos0)
    sel = oracle.indexer_select(I, np.arange(T), pos0, k)
    got = host(ip.idx)
    for t in range(T):
        assert np.array_equal(got[t], sel[t]), t
    assert int(ip.err.item()) == 0  # the redo cleared bit 1 and raised nothing else
    # a whole step takes the same checked path: both layers (the second one
    # reusing the index) attend through the redone index, exactly as the
    # two-call pipeline's layers do
    L2 = W.mqa_layer(94, 1, T, 16, 1, N, 128)
    layers2 = layers + [(dev_bf16(L2.q), dev_bf16(L2.k), dev_bf16(L2.v))]
    fu = IndexerPrefill(dev_bf16(qi), dev_bf16(ki), dev_f32(w), pos0, layers2, k_sel=k, fused=True)
    tc = IndexerPrefill(dev_bf16(qi), dev_bf16(ki), dev_f32(w), pos0, layers2, k_sel=k, fused=False)
    fu.step(reuse=True)
    tc.step(reuse=True)
    torch().cuda.synchronize()
    assert np.array_equal(host(fu.idx), host(tc.idx)) and np.array_equal(host(fu.idx), sel)
    for a, b in zip(fu.outs, tc.outs):
        assert np.array_equal(host(a), host(b))
    assert int(fu.err.item()) == 0


def test_indexer_topk_nan_flag(sa):
    T, Hi, N, k = 24, 32, 9000, 64
    ind = W.indexer_random(95, T, Hi, 64, N)
    w = ind.w.copy()
    w[3] = np.nan
    _, _, err = run_fused(sa, ind.qi, ind.ki, w, ind.pos0, k)
    assert err & 1


@pytest.mark.parametrize("fused", [True, False])
def test_indexer_pipeline_nan_raises(sa, fused):
    """A NaN among the indexer scores is reported by the checked index, fused
    or two-call, instead of reaching the layers."""
    from dynamic_sparse_attention_pool_amd.pipelines import IndexerPrefill
    T, Hi, N, k = 24, 32, 9000, 64
    ind = W.indexer_random(95, T, Hi, 64, N)
    w = ind.w.copy()
    w[3] = np.nan
    L = W.mqa_layer(95, 0, T, 16, 1, N, 128)
    ip = IndexerPrefill(dev_bf16(ind.qi), dev_bf16(ind.ki), dev_f32(w), ind.pos0,
                        [(dev_bf16(L.q), dev_bf16(L.k), dev_bf16(L.v))], k_sel=k, fused=fused)
    with pytest.raises(FloatingPointError):
        ip.step()


def test_indexer_topk_full_size(sa):
    """4096 queries at the end of a 131072-token context, 64 heads x 64,
    top-2048: the launch the benchmark times.  Every row equals the two-call
    path bit for bit; sampled rows against the oracle."""
    seed = W.CONFIG_SEEDS[5]
    T, N, Hi, k = 4096, 131072, 64, 2048
    ind = W.indexer_random(seed, T, Hi, 64, N)
    idx, cnt, err = run_fused(sa, ind.qi, ind.ki, ind.w, ind.pos0, k)
    assert err == 0 and np.all(cnt == k)
    ridx, rcnt = run_two_call(sa, ind.qi, ind.ki, ind.w, ind.pos0, k)
    assert np.array_equal(idx, ridx) and np.array_equal(cnt, rcnt)
    rows = np.array([0, 1, 1000, 2047, 3333, 4095])
    I = oracle.indexer_scores(W.bf16_to_f32(ind.qi), W.bf16_to_f32(ind.ki), ind.w, ind.pos0, rows)
    none = np.zeros(0, np.int64)
    sel = oracle.indexer_select(I, rows, ind.pos0, k)
    for r, t in enumerate(rows):
        cand = I[r, :ind.pos0 + t + 1]
        if oracle.certified_row(cand, k, none):
            assert np.array_equal(idx[t], sel[r])
        else:
            assert tie_tolerant_valid(idx[t], cand, k, none)
