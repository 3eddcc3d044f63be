"""Full-size block-sparse layers (32768 and 131072 tokens, GQA 32/8, d128,
bf16) run exactly as the benchmark runs them; sampled heads and query blocks
are checked against the oracle one by one."""
import math

import numpy as np
import pytest

import oracle
import workloads as W
from gpu_helpers import (assert_attention_close, assert_scores_close, dev_bf16, fwd_on_oracle_blocks, host,
                         lower_triangle,
                         tie_tolerant_valid, torch)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sa():
    import dynamic_sparse_attention_pool_amd as m
    m.load()
    return m


@pytest.mark.parametrize("N,ratio,seed", [(32768, (10, 100), W.CONFIG_SEEDS[2]), (131072, (5, 100), W.CONFIG_SEEDS[3])])
def test_block_sparse_layer_full_size(sa, N, ratio, seed):
    from dynamic_sparse_attention_pool_amd.pipelines import BlockSparseLayer
    print(f"full-size layer N={N} ratio={ratio}", flush=True)
    inp = W.prefill_bf16(seed, 1, 32, 8, N, 128)
    layer = BlockSparseLayer(dev_bf16(inp.q), dev_bf16(inp.k), dev_bf16(inp.v), n_sink=1, n_local=4, ratio=ratio,
                             out_dtype=torch().bfloat16, with_lse=True)
    # every (head, query block) of the launch writes its rows, whatever order the
    # workgroups take them in: no NaN planted before the launch may survive
    layer.out.fill_(float("nan"))
    layer.lse.fill_(float("nan"))
    layer.step()
    torch().cuda.synchronize()
    assert int(host(layer.err)[0]) == 0
    assert bool(torch().isfinite(layer.out).all()), "some output rows were not written"
    assert bool(torch().isfinite(layer.lse).all()), "some lse rows were not written"
    nb = N // 64
    scale = 1 / math.sqrt(128)
    idx, cnt = host(layer.idx), host(layer.cnt)
    # kept-block total equals the sum of the per-row budgets (independent of the data)
    per_row = []
    for i in range(nb):
        f = oracle.forced_set(i + 1, 1, 4)
        per_row.append(f.shape[0] + oracle.budget(i + 1, f.shape[0], None, ratio))
    assert int(cnt.sum()) == 32 * sum(per_row)
    S_gpu = lower_triangle(host(layer.scores))
    rng = np.random.default_rng(0)
    certified = total = 0
    for h in [0, 5, 31]:
        g = h * 8 // 32
        qh, kh, vh = inp.f32("q")[:, h:h + 1], inp.f32("k")[:, g:g + 1], inp.f32("v")[:, g:g + 1]
        S = oracle.block_scores(qh, kh, 64, scale)
        rows = np.unique(np.concatenate([[0, 1, 4, 5, nb - 1], rng.integers(0, nb, 12)]))
        assert_scores_close(S_gpu[0, h, rows], S[0, 0, rows], f"pooled scores h{h}")
        kept = [[[None] * nb]]
        differ = {}
        for i in rows:
            f = oracle.forced_set(i + 1, 1, 4)
            kr = oracle.budget(i + 1, f.shape[0], None, ratio)
            got = idx[0, h, i, :cnt[0, h, i]]
            want = oracle.topk_row(S[0, 0, i, :i + 1], kr, f)
            total += 1
            if oracle.certified_row(S[0, 0, i, :i + 1], kr, f):
                certified += 1
                assert np.array_equal(got, want), (h, i)
            else:
                assert tie_tolerant_valid(got, S[0, 0, i, :i + 1], kr, f), (h, i)
            kept[0][0][i] = want
            if not np.array_equal(got, want):
                differ[int(i)] = want
        wo, wl = oracle.block_sparse_attention(qh, kh, vh, kept, 64, scale, blocks=rows)
        o = host(layer.out[0, h])
        lse = host(layer.lse[0, h])
        for i in rows:
            if int(i) in differ:
                continue
            r = slice(64 * i, 64 * i + 64)
            assert_attention_close(o[r], wo[0, 0, r], bf16=True, what=f"h{h} block {i}")
            assert np.max(np.abs(lse[r] - wl[0, 0, r])) < 1e-3
        if differ:   # rows whose near-tied selection differs: the forward on the oracle's own blocks
            oo = fwd_on_oracle_blocks(sa, layer.q, layer.k, layer.v, h, differ, idx.shape[-1])
            for i in differ:
                r = slice(64 * i, 64 * i + 64)
                assert_attention_close(oo[r], wo[0, 0, r], bf16=True, what=f"h{h} block {i} on oracle blocks")
    print(f"certified sampled rows: {certified}/{total}", flush=True)
