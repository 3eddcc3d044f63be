"""Full-size block-sparse layers (32768 and 131072 tokens, GQA 32/8, d128,
bf16) run exactly as the benchmark runs them; sampled heads and query blocks
are checked against the oracle one by one."""
import math

import numpy as np
import pytest

import oracle
import workloads as W
from gpu_helpers import (assert_attention_close, assert_scores_close, dev_bf16, dev_i32, fwd_on_oracle_blocks, host,
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


class _BlockRows:
    """K or V rows held only for the blocks a test filled: K[keys] gathers
    rows by absolute key index, the interface attend_rows reads."""

    def __init__(self, blocks: dict, d: int):
        self.blocks, self.shape = blocks, (None, d)

    def __getitem__(self, keys):
        return np.stack([self.blocks[int(c) // 64][int(c) % 64] for c in np.asarray(keys)])


def test_fwd_bf16_tiles_past_4gib_of_kv(sa):
    """2^24 + 8192 tokens at d = 128: one KV head's K and V span 4.3 GB each,
    so the tiles of blocks >= 262144 start beyond 2^32 bytes from the head's
    base.  The tensors are zero except seeded values in the sampled query
    blocks and in every block they list (several past that point); those rows
    are checked against the oracle, and a zero row against its closed form."""
    t = torch()
    N, d = (1 << 24) + 8192, 128
    nb, scale = N // 64, 1 / math.sqrt(d)
    lists = {nb - 1: [0, 1, 131072, 262143, 262144, 262200, nb - 2, nb - 1],
             nb - 37: [0, 262150, nb - 40, nb - 37],
             262144: [5, 262143, 262144],
             200000: [0, 100000, 199999, 200000]}
    print(f"past-4GiB forward: N={N}, sampled blocks {sorted(lists)}", flush=True)
    q = t.zeros((1, 1, N, d), dtype=t.bfloat16, device="cuda:0")
    k, v = t.zeros_like(q), t.zeros_like(q)
    qb, kb, vb = {}, {}, {}

    def fill(dst, store, j, tag):
        bits = W.f32_to_bf16(W.normal(77, (64, d), tag, j))
        store[j] = W.bf16_to_f32(bits)
        dst[0, 0, 64 * j:64 * j + 64] = dev_bf16(bits)

    for i, blocks in lists.items():
        fill(q, qb, i, 0)
        for j in blocks:
            if j not in kb:
                fill(k, kb, j, 1)
                fill(v, vb, j, 2)
    kmax = 8
    idx = np.full((nb, kmax), -1, np.int32)
    cnt = np.ones(nb, np.int32)
    idx[:, 0] = np.arange(nb)
    for i, blocks in lists.items():
        idx[i, :len(blocks)], cnt[i] = blocks, len(blocks)
    out = t.empty((1, 1, N, d), dtype=t.float32, device="cuda:0")
    lse = t.empty((1, 1, N), dtype=t.float32, device="cuda:0")
    sa.sa_block_sparse_fwd(q, k, v, out, block_idx=dev_i32(idx.reshape(1, 1, nb, kmax)),
                           block_cnt=dev_i32(cnt.reshape(1, 1, nb)), lse=lse)
    t.cuda.synchronize()
    K, V = _BlockRows(kb, d), _BlockRows(vb, d)
    for i, blocks in lists.items():
        rows = np.arange(64 * i, 64 * i + 64)
        keys = (np.asarray(blocks)[:, None] * 64 + np.arange(64)[None, :]).reshape(-1)
        wo, wl = oracle.attend_rows(qb[i], K, V, keys, scale, row_pos=rows)
        assert_attention_close(host(out[0, 0, 64 * i:64 * i + 64]), wo, bf16=True, what=f"block {i}")
        assert np.max(np.abs(host(lse[0, 0, 64 * i:64 * i + 64]) - wl)) < 1e-3
    # a zero row over its own diagonal block: every admissible score is 0, so
    # o = 0 and lse = log(number of admissible keys)
    z = 1000
    assert np.all(host(out[0, 0, 64 * z:64 * z + 64]) == 0)
    assert np.allclose(host(lse[0, 0, 64 * z:64 * z + 64]), np.log(np.arange(1, 65)), atol=1e-5)

