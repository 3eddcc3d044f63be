"""GPU parity of the boundary options: the estimators' non-finite flag,
per-head and grouped token lists, and the per-query causal bound q_pos of the
gathered attention, each against the CPU oracle's plain attention over the
admissible keys."""
import math

import numpy as np
import pytest

import oracle
import workloads as W
from gpu_helpers import assert_attention_close, dev_bf16, dev_f32, dev_i32, host, torch

pytestmark = pytest.mark.gpu

NAN_BF16 = np.uint16(0x7FC0)


@pytest.fixture(scope="module")
def sa():
    import dynamic_sparse_attention_pool_amd as m
    m.load()
    return m


def _flag(t):
    return t.zeros(1, dtype=t.int32, device="cuda:0")


def run_estimate_flag(sa, kind, q, k, **kw):
    t = torch()
    err = _flag(t)
    sa.sa_estimate(kind, q, k, err_flag=err, **kw)
    t.cuda.synchronize()
    return int(host(err)[0])


def test_estimate_nonfinite_flag_block_and_vslash(sa):
    """Clean inputs leave the flag at 0; a NaN in a query row (block) or a key
    row (vertical-slash), or an input large enough to overflow the pooled sum,
    sets bit 0."""
    t = torch()
    B, Hq, Hkv, N, d = 1, 4, 2, 512, 128
    inp = W.prefill_bf16(71, B, Hq, Hkv, N, d)
    nb = N // 64

    def block(qb, kb):
        s = t.empty((B, Hq, nb, nb), dtype=t.float32, device="cuda:0")
        return run_estimate_flag(sa, sa.BLOCK_MEANPOOL, dev_bf16(qb), dev_bf16(kb), scores=s, scale=0.1)

    def vslash(qb, kb):
        av = t.empty((B, Hq, N), dtype=t.float32, device="cuda:0")
        as_ = t.empty_like(av)
        return run_estimate_flag(sa, sa.VSLASH, dev_bf16(qb), dev_bf16(kb), scores=av, scores2=as_, scale=0.1)

    assert block(inp.q, inp.k) == 0 and vslash(inp.q, inp.k) == 0
    q = inp.q.copy()
    q[0, 1, 70, 5] = NAN_BF16
    assert block(q, inp.k) == 1
    big = inp.q.copy()
    big[0, 2, 128:192] = W.f32_to_bf16(np.full((64, d), 3.0e38, np.float32))   # pooled sum overflows
    assert block(big, inp.k) == 1
    k = inp.k.copy()
    k[0, 0, 100, 3] = NAN_BF16
    assert vslash(inp.q, k) == 1


@pytest.mark.parametrize("Hi", [64, 16])
def test_estimate_nonfinite_flag_indexer_and_centroid(sa, Hi):
    t = torch()
    T, N = 8, 700
    ind = W.indexer_random(72, T, Hi, 64, N)
    scores = t.empty((T, N), dtype=t.float32, device="cuda:0")
    kw = dict(scores=scores, weights=dev_f32(ind.w), q_pos0=N - T)
    assert run_estimate_flag(sa, sa.INDEXER, dev_bf16(ind.qi), dev_bf16(ind.ki), **kw) == 0
    ki = ind.ki.copy()
    ki[50, 3] = NAN_BF16      # a causal key of every query
    assert run_estimate_flag(sa, sa.INDEXER, dev_bf16(ind.qi), dev_bf16(ki), **kw) == 1
    ki = ind.ki.copy()
    ki[N - 1, 3] = NAN_BF16   # only the last query sees it
    assert run_estimate_flag(sa, sa.INDEXER, dev_bf16(ind.qi), dev_bf16(ki), **kw) == 1
    if Hi in (32, 64):  # the fused top-k reports the same inputs
        idx = t.empty((T, 16), dtype=t.int32, device="cuda:0")
        cnt = t.empty(T, dtype=t.int32, device="cuda:0")
        for kk, want in ((ind.ki, 0), (ki, 1)):
            err = _flag(t)
            sa.sa_indexer_topk(dev_bf16(ind.qi), dev_bf16(kk), idx, cnt, weights=dev_f32(ind.w), q_pos0=N - T, k=16,
                               err_flag=err)
            t.cuda.synchronize()
            assert int(host(err)[0]) & 1 == want
    dec = W.decode_clustered(73, 2, 8, 2, 256, 128, 16)
    cs = t.empty((2, 8, 16), dtype=t.float32, device="cuda:0")
    cent = dev_f32(dec.centroids)
    kc = dev_bf16(dec.k)
    assert run_estimate_flag(sa, sa.CENTROID, dev_bf16(dec.q), kc, scores=cs, centroids=cent) == 0
    q = dec.q.copy()
    q[1, 6, 9] = NAN_BF16
    assert run_estimate_flag(sa, sa.CENTROID, dev_bf16(q), kc, scores=cs, centroids=cent) == 1


def gather_ref(q, k, v, lists, per_head, qpos, scale):
    """Oracle: each (token, head) attends the ids of its list that lie in
    [0, N) and at or before q_pos[t]."""
    T, Hq, d = q.shape
    Hkv, N, _ = k.shape
    O = np.zeros((T, Hq, d))
    L = np.full((T, Hq), -np.inf)
    for tt in range(T):
        for h in range(Hq):
            ids = np.asarray(lists[tt, h] if per_head else lists[tt], np.int64)
            lim = N - 1 if qpos is None else qpos[tt]
            ids = ids[(ids >= 0) & (ids < N) & (ids <= lim)]
            g = oracle.gqa_group(h, Hq, Hkv)
            o, l = oracle.attend_rows(q[tt, h][None], k[g], v[g], ids, scale)
            O[tt, h], L[tt, h] = o[0], l[0]
    return O, L


@pytest.mark.parametrize("Hq,Hkv,per_head,causal", [(8, 2, True, False), (8, 2, True, True), (8, 2, False, True),
                                                    (16, 1, False, True), (32, 2, False, False),
                                                    (6, 6, True, True)])
def test_token_gather_lists_and_causal_bound(sa, Hq, Hkv, per_head, causal):
    """Per-head lists [T,Hq,n], shared lists with any head grouping (one wave
    per head) or with 16 heads per KV head (matrix-core path), with and
    without q_pos; lists carry -1 padding, ids >= N and ids past q_pos."""
    t = torch()
    T, N, d, n = 6, 3000, 128, 150
    L = W.mqa_layer(74, 0, T, Hq, Hkv, N, d)
    r = np.random.default_rng(74)
    shape = (T, Hq, n) if per_head else (T, n)
    lists = np.empty(shape, np.int32)
    for pos in np.ndindex(shape[:-1]):
        ids = r.choice(N, size=n, replace=False).astype(np.int32)
        ids[r.random(n) < 0.1] = -1
        ids[r.random(n) < 0.03] = N + 5
        lists[pos] = ids
    qpos = np.array([2999, 1500, 10, 0, 2000, 777], np.int32) if causal else None
    out = t.empty((T, Hq, d), dtype=t.float32, device="cuda:0")
    lse = t.empty((T, Hq), dtype=t.float32, device="cuda:0")
    sa.sa_gather_decode(dev_bf16(L.q), dev_bf16(L.k), dev_bf16(L.v), out, tok_idx=dev_i32(lists), lse=lse,
                        q_pos=None if qpos is None else dev_i32(qpos))
    t.cuda.synchronize()
    scale = 1 / math.sqrt(d)
    wo, wl = gather_ref(W.bf16_to_f32(L.q), W.bf16_to_f32(L.k), W.bf16_to_f32(L.v), lists, per_head, qpos, scale)
    assert_attention_close(host(out), wo, bf16=True, what=f"token gather Hq{Hq}/{Hkv} per_head={per_head}")
    gl = host(lse)
    assert np.array_equal(np.isneginf(gl), np.isneginf(wl))
    fin = np.isfinite(wl)
    assert np.max(np.abs(gl[fin] - wl[fin])) < 1e-3


@pytest.mark.parametrize("T,qpos", [(4, [4095, 2000, 10, 900]),
                                    (12, [4095, 0, 3000, 17, 2048, 4000, 1, 512, 3999, 64, 100, 2500])])
def test_cluster_decode_causal_bound(sa, T, qpos):
    """Cluster mode with q_pos: packed rows map back to context positions
    through the pack's perm; query t attends the tokens of its selected
    clusters at or before q_pos[t] (none for some).  T = 12 puts 48 query
    rows on each KV head (the two-tile form of the gather)."""
    t = torch()
    Hq, Hkv, N, d, C, ks = 8, 2, 4096, 128, 64, 8
    print(f"causal cluster decode T{T}", flush=True)
    dec = W.decode_clustered(75, T, Hq, Hkv, N, d, C)
    ptr = t.empty((Hkv, C + 1), dtype=t.int32, device="cuda:0")
    perm = t.empty((Hkv, N), dtype=t.int32, device="cuda:0")
    kp = t.empty((Hkv, N, d), dtype=t.bfloat16, device="cuda:0")
    vp = t.empty_like(kp)
    sa.sa_cluster_pack(dev_i32(dec.labels), ptr, perm, C, k=dev_bf16(dec.k), v=dev_bf16(dec.v), k_packed=kp,
                       v_packed=vp)
    scale = 1 / math.sqrt(d)
    sel = oracle.cluster_select(oracle.centroid_scores(W.bf16_to_f32(dec.q), dec.centroids, scale), ks)
    sel_np = np.array([[s for s in row] for row in sel], np.int32)
    qpos = np.array(qpos, np.int32)
    out = t.empty((T, Hq, d), dtype=t.float32, device="cuda:0")
    lse = t.empty((T, Hq), dtype=t.float32, device="cuda:0")
    sa.sa_gather_decode(dev_bf16(dec.q), kp, vp, out, cluster_ptr=ptr, sel=dev_i32(sel_np), lse=lse,
                        q_pos=dev_i32(qpos), perm=perm)
    t.cuda.synchronize()
    q, k, v = W.bf16_to_f32(dec.q), W.bf16_to_f32(dec.k), W.bf16_to_f32(dec.v)
    wo = np.zeros((T, Hq, d))
    wl = np.full((T, Hq), -np.inf)
    for tt in range(T):
        for h in range(Hq):
            g = oracle.gqa_group(h, Hq, Hkv)
            ids = np.nonzero(np.isin(dec.labels[g], sel[tt][h]) & (np.arange(N) <= qpos[tt]))[0]
            o, l = oracle.attend_rows(q[tt, h][None], k[g], v[g], ids, scale)
            wo[tt, h], wl[tt, h] = o[0], l[0]
    assert_attention_close(host(out), wo, bf16=True, what="causal cluster decode")
    gl = host(lse)
    assert np.array_equal(np.isneginf(gl), np.isneginf(wl))
    fin = np.isfinite(wl)
    assert np.max(np.abs(gl[fin] - wl[fin])) < 1e-3
