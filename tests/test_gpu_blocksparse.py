"""GPU parity of the block-sparse path: selection, pooled estimate and the
sparse forward, each against the CPU oracle on the same seeded inputs."""
import math

import numpy as np
import pytest

import oracle
import workloads as W
from gpu_helpers import (assert_attention_close, assert_scores_close, certify_prefill, dev_bf16, dev_f32,
                         dev_i32, host, lower_triangle, pad_table, tie_tolerant_valid, torch)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sa():
    import dynamic_sparse_attention_pool_amd as m
    m.load()
    return m


def gpu_select(sa, scores_np, kmax, **kw):
    t = torch()
    s = dev_f32(scores_np)
    idx = t.empty((scores_np.shape[0], kmax), dtype=t.int32, device=s.device)
    cnt = t.empty(scores_np.shape[0], dtype=t.int32, device=s.device)
    err = t.zeros(1, dtype=t.int32, device=s.device)
    sa.sa_select_topk(s, idx, cnt, err_flag=err, **kw)
    t.cuda.synchronize()
    return host(idx), host(cnt), int(host(err)[0])


def oracle_select(scores_np, **kw):
    ratio = kw.get("ratio")
    return oracle.select_rows(scores_np.astype(np.float64), causal=kw.get("causal", False),
                              period=kw.get("causal_period", 1), offset=kw.get("causal_offset", 0),
                              n_sink=kw.get("n_sink", 0), n_local=kw.get("n_local", 0),
                              k=None if ratio else kw.get("k", 0), ratio=ratio)


SELECT_CASES = [
    # (rows, ncand, kind, kwargs, kmax)
    (16, 16, "normal", dict(k=2, n_sink=1, n_local=1, causal=True, causal_period=16), 4),
    (64, 512, "normal", dict(ratio=(10, 100), n_sink=1, n_local=4, causal=True, causal_period=512), 57),
    (48, 2048, "ties", dict(ratio=(5, 100), n_sink=1, n_local=4, causal=True, causal_period=2048), 108),
    (40, 256, "ties", dict(k=64), 64),
    (8, 300, "normal", dict(k=0, n_sink=3), 3),
    (8, 300, "normal", dict(k=500, n_local=7), 300),
    (5, 4096, "ties", dict(k=1000), 1000),
    # one wave per row (257..2048 candidates): a row count that leaves a partial workgroup
    (7, 1000, "coarse", dict(k=37, n_sink=2, n_local=3), 42),
    (13, 2000, "ties", dict(ratio=(7, 100), n_sink=1, n_local=2, causal=True, causal_period=13,
                            causal_offset=1987), 143),
]


@pytest.mark.parametrize("case", range(len(SELECT_CASES)))
def test_select_bit_exact_lds_rows(sa, case):
    R, n, kind, kw, kmax = SELECT_CASES[case]
    print(f"select case {case}: rows {R} ncand {n} {kind} {kw}", flush=True)
    s = W.score_rows(7, R, n, kind, case)
    idx, cnt, err = gpu_select(sa, s, kmax, **kw)
    want = oracle_select(s, **kw)
    assert err == 0
    for r in range(R):
        assert cnt[r] == len(want[r]), r
        assert np.array_equal(idx[r, :cnt[r]], want[r]), r
        assert np.all(idx[r, cnt[r]:] == -1)


@pytest.mark.parametrize("kind", ["normal", "ties", "coarse"])
def test_select_bit_exact_long_rows(sa, kind):
    # indexer-like causal rows (ragged lengths) and vertical/slash-like full rows
    R, n = 6, 131072
    print(f"long select {kind}", flush=True)
    s = W.score_rows(8, R, n, kind)
    for kw, kmax in [(dict(k=2048, causal=True, causal_period=R, causal_offset=n - R), 2048),
                     (dict(k=1000), 1000), (dict(k=64, n_sink=2, n_local=2), 68)]:
        idx, cnt, err = gpu_select(sa, s, kmax, **kw)
        want = oracle_select(s, **kw)
        assert err == 0
        for r in range(R):
            assert cnt[r] == len(want[r])
            assert np.array_equal(idx[r, :cnt[r]], want[r])


@pytest.mark.parametrize("kind", ["normal", "ties"])
def test_select_rows_longer_than_one_bitmap(sa, kind):
    # past 131072 candidates the two-pass kernel takes over
    R, n = 3, 140000
    print(f"select beyond bitmap {kind}", flush=True)
    s = W.score_rows(10, R, n, kind)
    for kw, kmax in [(dict(k=500), 500), (dict(k=2048, causal=True, causal_period=R, causal_offset=n - R), 2048)]:
        idx, cnt, err = gpu_select(sa, s, kmax, **kw)
        want = oracle_select(s, **kw)
        assert err == 0
        for r in range(R):
            assert cnt[r] == len(want[r]) and np.array_equal(idx[r, :cnt[r]], want[r])


def test_select_ragged_long_rows_and_nan_flag(sa):
    s = W.score_rows(9, 3, 5000, "normal")
    idx, cnt, err = gpu_select(sa, s, 300, k=300)
    want = oracle_select(s, k=300)
    assert err == 0 and all(np.array_equal(idx[r, :cnt[r]], want[r]) for r in range(3))
    s[1, 17] = np.nan
    _, _, err = gpu_select(sa, s, 300, k=300)
    assert err == 1
    s = W.score_rows(10, 5, 1500, "normal")     # one wave per row
    s[3, 1499] = np.nan
    _, _, err = gpu_select(sa, s, 64, k=60, n_local=4)
    assert err == 1


def run_block_estimate(sa, q, k, scale):
    """Pooled scores with the upper triangle checked untouched (the buffer is
    pre-filled with a sentinel) and then stated as -inf, like the oracle's."""
    t = torch()
    B, Hq, N, d = q.shape
    nb = N // 64
    scores = t.full((B, Hq, nb, nb), 7777.0, dtype=t.float32, device=q.device)
    pq = t.empty((B, Hq, nb, d), dtype=t.float32, device=q.device)
    pk = t.empty((B, k.shape[1], nb, d), dtype=t.float32, device=q.device)
    err = t.zeros(1, dtype=t.int32, device=q.device)
    sa.sa_estimate(sa.BLOCK_MEANPOOL, q, k, scores, scale=scale, pooled_q=pq, pooled_k=pk, err_flag=err)
    t.cuda.synchronize()
    s = host(scores)
    upper = np.triu(np.ones((nb, nb), bool), 1)
    assert np.all(s[..., upper] == 7777.0), "entries above the diagonal were written"
    assert int(host(err)[0]) == 0
    return lower_triangle(s), host(pq), host(pk)


def test_block_estimate_exact_integer_inputs(sa):
    """bf16 integers in [-2,2] with scale 1: block sums, /64 and the 128-term
    dot products are exact in fp32, so the GPU equals the fp64 oracle bit for bit."""
    B, Hq, Hkv, N, d = 1, 4, 2, 640, 128
    q = W.integer_bf16(11, (B, Hq, N, d), -2, 2, 0)
    k = W.integer_bf16(11, (B, Hkv, N, d), -2, 2, 1)
    s, pq, pk = run_block_estimate(sa, dev_bf16(q), dev_bf16(k), 1.0)
    want = oracle.block_scores(W.bf16_to_f32(q), W.bf16_to_f32(k), 64, 1.0)
    assert np.array_equal(s, want)
    assert np.array_equal(pq[0, 1], oracle.mean_pool(W.bf16_to_f32(q)[0, 1], 64))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_block_estimate_random(sa, dtype):
    if dtype == "f32":
        inp = W.prefill_fp32(12, 1, 2, 1024, 64)
        q, k = dev_f32(inp.q), dev_f32(inp.k)
        d = 64
    else:
        inp = W.prefill_bf16(12, 2, 4, 2, 1024, 128)
        q, k = dev_bf16(inp.q), dev_bf16(inp.k)
        d = 128
    scale = 1 / math.sqrt(d)
    s, _, _ = run_block_estimate(sa, q, k, scale)
    want = oracle.block_scores(inp.f32("q"), inp.f32("k"), 64, scale)
    assert_scores_close(s, want, f"block scores {dtype}")


def run_fwd(sa, q, k, v, kept_lists, kmax, out_bf16=False, scale=None):
    t = torch()
    B, Hq, N, d = q.shape
    nb = N // 64
    flat = [kept_lists[b][h][i] for b in range(B) for h in range(Hq) for i in range(nb)]
    idx, cnt = pad_table(flat, kmax)
    out = t.empty((B, Hq, N, d), dtype=t.bfloat16 if out_bf16 else t.float32, device=q.device)
    lse = t.empty((B, Hq, N), dtype=t.float32, device=q.device)
    sa.sa_block_sparse_fwd(q, k, v, out, block_idx=dev_i32(idx.reshape(B, Hq, nb, kmax)),
                           block_cnt=dev_i32(cnt.reshape(B, Hq, nb)), lse=lse, scale=scale)
    t.cuda.synchronize()
    return host(out), host(lse)


@pytest.mark.parametrize("d", [64, 128])
def test_fwd_fp32_sink_diag_top2_on_oracle_sets(sa, d):
    inp = W.prefill_fp32(W.CONFIG_SEEDS[1], 1, 1, 1024, d)
    scale = 1 / math.sqrt(d)
    S = oracle.block_scores(inp.q, inp.k, 64, scale)
    kept = oracle.block_select(S, n_sink=1, n_local=1, k=2)
    o, l = run_fwd(sa, dev_f32(inp.q), dev_f32(inp.k), dev_f32(inp.v), kept, 4, scale=scale)
    wo, wl = oracle.block_sparse_attention(inp.q, inp.k, inp.v, kept, 64, scale)
    assert_attention_close(o, wo, bf16=False, what="fp32 fwd")
    assert np.max(np.abs(l - wl)) < 1e-5


@pytest.mark.parametrize("d,out_bf16", [(128, False), (128, True), (64, False), (64, True)])
def test_fwd_bf16_on_oracle_sets(sa, d, out_bf16):
    B, Hq, Hkv, N = 1, 4, 2, 1024
    inp = W.prefill_bf16(13, B, Hq, Hkv, N, d)
    scale = 1 / math.sqrt(d)
    S = oracle.block_scores(inp.f32("q"), inp.f32("k"), 64, scale)
    kept = oracle.block_select(S, n_sink=1, n_local=4, ratio=(30, 100))
    kept[0][1] = [np.arange(i + 1) for i in range(N // 64)]      # head 1 dense causal
    o, l = run_fwd(sa, dev_bf16(inp.q), dev_bf16(inp.k), dev_bf16(inp.v), kept, N // 64, out_bf16=out_bf16)
    wo, wl = oracle.block_sparse_attention(inp.f32("q"), inp.f32("k"), inp.f32("v"), kept, 64, scale)
    assert_attention_close(o, wo, bf16=True, what=f"bf16 fwd d{d}")
    assert np.max(np.abs(l - wl)) < 1e-3


def test_fwd_bf16_row_at_table_capacity(sa):
    """At 131072 tokens a row may list all 2048 blocks, the most the bf16 path
    stages per row: that row, a row of every other block, a half-length dense
    row and diagonal-only rows, sampled against the oracle."""
    B, Hq, Hkv, N, d = 1, 1, 1, 131072, 128
    nb = N // 64
    inp = W.prefill_bf16(15, B, Hq, Hkv, N, d)
    kept = [[[np.array([i]) for i in range(nb)]]]
    kept[0][0][nb - 1] = np.arange(nb)
    kept[0][0][nb - 2] = np.arange(0, nb - 1, 2)
    kept[0][0][1000] = np.arange(1001)
    print(f"capacity row: kmax {nb}, N {N}", flush=True)
    o, l = run_fwd(sa, dev_bf16(inp.q), dev_bf16(inp.k), dev_bf16(inp.v), kept, nb)
    rows = [0, 999, 1000, nb - 2, nb - 1]
    wo, wl = oracle.block_sparse_attention(inp.f32("q"), inp.f32("k"), inp.f32("v"), kept, 64, 1 / math.sqrt(d),
                                           blocks=rows)
    for i in rows:
        r = slice(64 * i, 64 * i + 64)
        assert_attention_close(o[:, :, r], wo[:, :, r], bf16=True, what=f"capacity rows, block {i}")
        assert np.max(np.abs(l[:, :, r] - wl[:, :, r])) < 1e-3


def test_fwd_bf16_empty_and_single_block_rows(sa):
    B, Hq, Hkv, N, d = 1, 2, 1, 512, 128
    inp = W.prefill_bf16(14, B, Hq, Hkv, N, d)
    nb = N // 64
    kept = [[[np.zeros(0, np.int64) if i % 3 == 0 else np.array([i // 2]) for i in range(nb)] for _ in range(Hq)]]
    o, l = run_fwd(sa, dev_bf16(inp.q), dev_bf16(inp.k), dev_bf16(inp.v), kept, 2)
    wo, wl = oracle.block_sparse_attention(inp.f32("q"), inp.f32("k"), inp.f32("v"), kept, 64, 1 / math.sqrt(d))
    assert_attention_close(o, wo, bf16=True, what="empty/single rows")
    assert np.array_equal(np.isneginf(l), np.isneginf(wl))
    assert np.all(o[:, :, 0:64] == 0)


def run_block_layer(sa, q, k, v, n_sink, n_local, kmax, k_fixed=None, ratio=None, out_bf16=False, scale=None):
    """estimate -> select -> forward, as the benchmark chains them."""
    t = torch()
    B, Hq, N, d = q.shape
    nb = N // 64
    scale = 1 / math.sqrt(d) if scale is None else scale
    scores = t.empty((B, Hq, nb, nb), dtype=t.float32, device=q.device)
    sa.sa_estimate(sa.BLOCK_MEANPOOL, q, k, scores, scale=scale)
    idx = t.empty((B * Hq * nb, kmax), dtype=t.int32, device=q.device)
    cnt = t.empty(B * Hq * nb, dtype=t.int32, device=q.device)
    sel = dict(n_sink=n_sink, n_local=n_local, causal=True, causal_period=nb)
    if ratio:
        sel["ratio"] = ratio
    else:
        sel["k"] = k_fixed
    sa.sa_select_topk(scores.view(B * Hq * nb, nb), idx, cnt, **sel)
    out = t.empty((B, Hq, N, d), dtype=t.bfloat16 if out_bf16 else t.float32, device=q.device)
    sa.sa_block_sparse_fwd(q, k, v, out, block_idx=idx.view(B, Hq, nb, kmax), block_cnt=cnt.view(B, Hq, nb),
                           scale=scale)
    t.cuda.synchronize()
    return lower_triangle(host(scores)), host(idx).reshape(B, Hq, nb, kmax), host(cnt).reshape(B, Hq, nb), host(out)


def test_end_to_end_sink_diag_top2_fp32(sa):
    seed = W.CONFIG_SEEDS[1]
    inp = W.prefill_fp32(seed, 1, 1, 1024, 64)
    certify_prefill(inp, seed, 64, 1 / 8.0, 1, 1, k=2)
    S, idx, cnt, o = run_block_layer(sa, dev_f32(inp.q), dev_f32(inp.k), dev_f32(inp.v), 1, 1, 4, k_fixed=2)
    Sw = oracle.block_scores(inp.q, inp.k, 64, 1 / 8.0)
    kept = oracle.block_select(Sw, n_sink=1, n_local=1, k=2)
    assert_scores_close(S, Sw)
    for i in range(16):
        assert np.array_equal(idx[0, 0, i, :cnt[0, 0, i]], kept[0][0][i])
    assert int(cnt.sum()) == 58
    wo, _ = oracle.block_sparse_attention(inp.q, inp.k, inp.v, kept, 64, 1 / 8.0)
    assert_attention_close(o, wo, bf16=False, what="config-1 end to end")


def test_end_to_end_shifted_gqa_prefill_certified(sa):
    """GQA 8/2, d128, N 4096, 1% shifted keys, sink + 4 local + ceil(10%):
    certified rows -> identical kept sets; outputs within the bf16 bounds."""
    seed = 21
    B, Hq, Hkv, N, d = 1, 8, 2, 4096, 128
    inp = W.prefill_bf16(seed, B, Hq, Hkv, N, d)
    scale = 1 / math.sqrt(d)
    nre = certify_prefill(inp, seed, 64, scale, 1, 4, ratio=(10, 100))
    print(f"redrawn blocks: {nre}", flush=True)
    nb = N // 64
    kmax = 5 + math.ceil(0.1 * nb)
    S, idx, cnt, o = run_block_layer(sa, dev_bf16(inp.q), dev_bf16(inp.k), dev_bf16(inp.v), 1, 4, kmax,
                                     ratio=(10, 100))
    Sw = oracle.block_scores(inp.f32("q"), inp.f32("k"), 64, scale)
    assert_scores_close(S, Sw)
    kept = oracle.block_select(Sw, n_sink=1, n_local=4, ratio=(10, 100))
    for h in range(Hq):
        for i in range(nb):
            assert np.array_equal(idx[0, h, i, :cnt[0, h, i]], kept[0][h][i]), (h, i)
    wo, _ = oracle.block_sparse_attention(inp.f32("q"), inp.f32("k"), inp.f32("v"), kept, 64, scale)
    assert_attention_close(o, wo, bf16=True, what="shifted GQA prefill")


def test_determinism_bitwise(sa):
    inp = W.prefill_bf16(22, 1, 4, 2, 2048, 128)
    q, k, v = dev_bf16(inp.q), dev_bf16(inp.k), dev_bf16(inp.v)
    a = run_block_layer(sa, q, k, v, 1, 4, 12, ratio=(10, 100))
    b = run_block_layer(sa, q, k, v, 1, 4, 12, ratio=(10, 100))
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_fwd_out_of_range_block_entries(sa):
    """Table entries the forward cannot use — negative ids, blocks above the
    diagonal, counts above kmax or below 0 — are skipped or clipped: the output
    equals, bit for bit, the forward on the cleaned table, and nothing is read
    outside K and V."""
    t = torch()
    B, Hq, Hkv, N, d = 1, 2, 1, 1024, 128
    nb = N // 64
    inp = W.prefill_bf16(61, B, Hq, Hkv, N, d)
    r = np.random.default_rng(61)
    clean = [[np.unique(np.concatenate([[0, i], r.choice(i + 1, size=min(i + 1, 3), replace=False)]))
              for i in range(nb)] for _ in range(Hq)]
    kmax = 8
    idx_c, cnt_c = pad_table([x for h in clean for x in h], kmax)
    idx_b, cnt_b = idx_c.copy(), cnt_c.copy()
    for row in range(Hq * nb):
        i = row % nb
        n = cnt_b[row]
        junk = [-5, i + 1 + r.integers(0, 50), 10 ** 9, -(10 ** 9)]
        room = kmax - n
        if room > 0:
            idx_b[row, n:n + room] = np.resize(junk, room)   # skipped entries after the kept ones
            cnt_b[row] = kmax if row % 3 else kmax + 100     # count above kmax is clipped to kmax
    cnt_b[5] = -7                                           # a negative count keeps nothing
    cnt_c[5] = 0
    q, k, v = dev_bf16(inp.q), dev_bf16(inp.k), dev_bf16(inp.v)
    outs = []
    for idx, cnt in ((idx_c, cnt_c), (idx_b, cnt_b)):
        o = t.empty(q.shape, dtype=t.float32, device=q.device)
        sa.sa_block_sparse_fwd(q, k, v, o, block_idx=dev_i32(idx).view(B, Hq, nb, kmax),
                               block_cnt=dev_i32(cnt).view(B, Hq, nb))
        outs.append(host(o))
    t.cuda.synchronize()
    assert np.array_equal(outs[0], outs[1])
    assert np.all(outs[1][0, 0, 5 * 64:6 * 64] == 0)


def test_fwd_rows_beyond_2_pow_32_bytes(sa):
    """A 16.8M-token head (K and V above 4 GiB each): the last query block
    attends blocks on both sides of row 2^24, where byte offsets pass 2^32.
    Compared with the oracle on those keys (the other rows are zero and
    unread)."""
    t = torch()
    d = 128
    N = (1 << 24) + 2048
    nb = N // 64
    i = nb - 1
    blocks = np.array([0, (1 << 18) - 1, 1 << 18, (1 << 18) + 26, i], np.int64)
    rows = (blocks[:, None] * 64 + np.arange(64)[None, :]).reshape(-1)
    rg = W.rng(62, 0)
    kq = W.f32_to_bf16(rg.standard_normal((64, d), dtype=np.float32))
    kk = W.f32_to_bf16(rg.standard_normal((rows.size, d), dtype=np.float32))
    kv = W.f32_to_bf16(rg.standard_normal((rows.size, d), dtype=np.float32))
    q = t.zeros((1, 1, N, d), dtype=t.bfloat16, device="cuda:0")
    k = t.zeros_like(q)
    v = t.zeros_like(q)
    q[0, 0, i * 64:] = dev_bf16(kq)
    ridx = t.from_numpy(rows).to("cuda:0")
    k[0, 0].index_copy_(0, ridx, dev_bf16(kk))
    v[0, 0].index_copy_(0, ridx, dev_bf16(kv))
    kmax = 8
    idx = np.full((nb, kmax), -1, np.int32)
    cnt = np.zeros(nb, np.int32)
    idx[i, :blocks.size] = blocks
    cnt[i] = blocks.size
    out = t.empty_like(q)
    sa.sa_block_sparse_fwd(q, k, v, out, block_idx=dev_i32(idx).view(1, 1, nb, kmax),
                           block_cnt=dev_i32(cnt).view(1, 1, nb))
    got = host(out[0, 0, i * 64:])
    t.cuda.synchronize()
    del q, k, v, out
    t.cuda.empty_cache()
    # compact problem: kept keys in ascending order, query positions mapped to
    # the number of kept keys at or before them (the causal relation is kept)
    qpos = i * 64 + np.arange(64)
    want, _ = oracle.attend_rows(W.bf16_to_f32(kq), W.bf16_to_f32(kk), W.bf16_to_f32(kv), np.arange(rows.size),
                                 1 / math.sqrt(d), row_pos=np.searchsorted(rows, qpos, side="right") - 1)
    assert_attention_close(got, want, bf16=True, what="rows beyond 2^32 bytes")
