"""GPU parity of the token indexer, its top-k and the shared-layer index
cache, against the CPU oracle."""
import math

import numpy as np
import pytest

import oracle
import workloads as W
from gpu_helpers import (assert_attention_close, assert_scores_close, dev_bf16, dev_f32, dev_i32, host,
                         tie_tolerant_valid, torch)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sa():
    import dynamic_sparse_attention_pool_amd as m
    m.load()
    return m


def gpu_indexer(sa, qi, ki, w, pos0):
    t = torch()
    T, N = qi.shape[0], ki.shape[0]
    out = t.empty((T, N), dtype=t.float32, device="cuda:0")
    sa.sa_estimate(sa.INDEXER, dev_bf16(qi), dev_bf16(ki), out, weights=dev_f32(w), q_pos0=pos0)
    t.cuda.synchronize()
    return host(out)


@pytest.mark.parametrize("Hi", [64, 24])
def test_indexer_exact_integer_inputs(sa, Hi):
    """Integers in [-4,4] and weights m/64: every product, ReLU and weighted
    sum is exact in fp32, so the GPU equals the fp64 oracle bit for bit (64
    heads on the matrix-core rows, 24 heads split over eight waves)."""
    T, di, N = 64, 64, 16384 + 512
    qi = W.integer_bf16(41, (T, Hi, di), -4, 4, 0)
    ki = W.integer_bf16(41, (N, di), -4, 4, 1)
    w = (np.random.default_rng(41).integers(0, 65, size=Hi) / 64.0).astype(np.float32)
    pos0 = N - T - 100
    got = gpu_indexer(sa, qi, ki, w, pos0)
    want = oracle.indexer_scores(W.bf16_to_f32(qi), W.bf16_to_f32(ki), w, pos0)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("T,Hi,N", [(80, 64, 20000), (64, 32, 9000), (32, 16, 8192), (7, 8, 4096), (33, 24, 5000),
                                    (20, 40, 4100), (9, 48, 3000), (40, 56, 8200)])
def test_indexer_random(sa, T, Hi, N):
    ind = W.indexer_random(42, T, Hi, 64, N)
    got = gpu_indexer(sa, ind.qi, ind.ki, ind.w, ind.pos0)
    want = oracle.indexer_scores(W.bf16_to_f32(ind.qi), W.bf16_to_f32(ind.ki), ind.w, ind.pos0)
    assert_scores_close(got, want, "indexer")


def test_index_cache_layers_planted_certified(sa):
    """Planted indexer input (certified top-2048), 4 MQA layers: the full
    layer's indices equal the oracle's; shared layers attend through the same
    index buffer and match the oracle run with layer-1 indices."""
    from dynamic_sparse_attention_pool_amd.pipelines import IndexerPrefill
    T, Hi, di, N, k = 64, 64, 64, 40960, 2048
    ind = W.indexer_planted(43, T, Hi, di, N, k, n_dir=16)
    layers_np = [W.mqa_layer(43, l, T, 16, 1, N, 128) for l in range(4)]
    layers = [(dev_bf16(L.q), dev_bf16(L.k), dev_bf16(L.v)) for L in layers_np]
    ip = IndexerPrefill(dev_bf16(ind.qi), dev_bf16(ind.ki), dev_f32(ind.w), ind.pos0, layers, k_sel=k)
    ip.step(reuse=True)
    torch().cuda.synchronize()
    idx = host(ip.idx)
    I = oracle.indexer_scores(W.bf16_to_f32(ind.qi), W.bf16_to_f32(ind.ki), ind.w, ind.pos0)
    sel = oracle.indexer_select(I, np.arange(T), ind.pos0, k)
    for t in range(T):
        assert oracle.certified_row(I[t, :ind.pos0 + t + 1], k, np.zeros(0, np.int64))
        assert np.array_equal(idx[t], sel[t])
    lay = [(W.bf16_to_f32(L.q), W.bf16_to_f32(L.k), W.bf16_to_f32(L.v)) for L in layers_np]
    outs, used = oracle.index_cache_forward(lay, {0}, W.bf16_to_f32(ind.qi), W.bf16_to_f32(ind.ki), ind.w,
                                            ind.pos0, k, 1 / math.sqrt(128))
    for l in range(4):
        assert_attention_close(host(ip.outs[l]), outs[l], bf16=True, what=f"layer {l}")
    # running the indexer on every layer gives the same index buffer, bytewise
    before = host(ip.idx).copy()
    ip.step(reuse=False)
    torch().cuda.synchronize()
    assert np.array_equal(host(ip.idx), before)


def test_indexer_full_size_sampled_rows(sa):
    """4096 queries at the end of a 131072-token context, 64 heads x 64: the
    benchmark's launch; sampled rows checked against the oracle one by one."""
    from dynamic_sparse_attention_pool_amd.pipelines import IndexerPrefill
    seed = W.CONFIG_SEEDS[5]
    T, N, Hi, di, k = 4096, 131072, 64, 64, 2048
    ind = W.indexer_random(seed, T, Hi, di, N)
    L = W.mqa_layer(seed, 0, T, 16, 1, N, 128)
    layers = [(dev_bf16(L.q), dev_bf16(L.k), dev_bf16(L.v))]
    ip = IndexerPrefill(dev_bf16(ind.qi), dev_bf16(ind.ki), dev_f32(ind.w), ind.pos0, layers, k_sel=k)
    # every score (causal ones and the -inf beyond each query's position) and
    # every output row is written: no NaN planted before the launch survives
    ip.scores.fill_(float("nan"))
    ip.outs[0].fill_(float("nan"))
    ip.step()
    torch().cuda.synchronize()
    assert not bool(torch().isnan(ip.scores).any()), "some indexer scores were not written"
    assert bool(torch().isfinite(ip.outs[0]).all()), "some gathered-attention rows were not written"
    rows = np.array([0, 1, 777, 2048, 4000, 4095])
    scores = host(ip.scores[rows.tolist()])
    idx = host(ip.idx)[rows]
    want = oracle.indexer_scores(W.bf16_to_f32(ind.qi), W.bf16_to_f32(ind.ki), ind.w, ind.pos0, rows)
    assert_scores_close(scores, want, "full-size indexer rows")
    none = np.zeros(0, np.int64)
    sel = oracle.indexer_select(want, rows, ind.pos0, k)
    exact = 0
    for n, t in enumerate(rows):
        cand = want[n, :ind.pos0 + t + 1]
        if oracle.certified_row(cand, k, none):
            assert np.array_equal(idx[n], sel[n])
            exact += 1
        else:
            assert tie_tolerant_valid(idx[n], cand, k, none)
    print(f"certified rows: {exact}/{len(rows)}", flush=True)
    wo, _ = oracle.gathered_attention(W.bf16_to_f32(L.q), W.bf16_to_f32(L.k), W.bf16_to_f32(L.v), list(idx),
                                      1 / math.sqrt(128), rows)
    assert_attention_close(host(ip.outs[0])[rows], wo, bf16=True, what="full-size gathered attention")
