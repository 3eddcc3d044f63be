"""GPU parity of the clustered decode path (pack, centroid scores, selection,
gathered attention) and of the token-gathered attention used by the index
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


def pack(sa, labels, C, k=None, v=None):
    t = torch()
    Hkv, N = labels.shape
    ptr = t.empty((Hkv, C + 1), dtype=t.int32, device="cuda:0")
    perm = t.empty((Hkv, N), dtype=t.int32, device="cuda:0")
    err = t.zeros(1, dtype=t.int32, device="cuda:0")
    kp = vp = None
    if k is not None:
        kp, vp = t.empty_like(k), t.empty_like(v)
    sa.sa_cluster_pack(dev_i32(labels), ptr, perm, C, k=k, v=v, k_packed=kp, v_packed=vp, err_flag=err)
    t.cuda.synchronize()
    return ptr, perm, kp, vp, int(host(err)[0])


def test_cluster_pack_matches_stable_counting_sort(sa):
    r = np.random.default_rng(1)
    labels = r.integers(0, 37, size=(3, 5003)).astype(np.int32)
    k = W.f32_to_bf16(r.standard_normal((3, 5003, 128)).astype(np.float32))
    v = W.f32_to_bf16(r.standard_normal((3, 5003, 128)).astype(np.float32))
    ptr, perm, kp, vp, err = pack(sa, labels, 37, dev_bf16(k), dev_bf16(v))
    wptr, wperm = oracle.cluster_pack(labels, 37)
    assert err == 0
    assert np.array_equal(host(ptr), wptr) and np.array_equal(host(perm), wperm)
    kph = host(kp.view(torch().int16)).view(np.uint16)
    for g in range(3):
        assert np.array_equal(kph[g], k[g][wperm[g]])


def test_cluster_pack_flags_bad_labels(sa):
    labels = np.zeros((1, 100), np.int32)
    labels[0, 7] = 9
    _, _, _, _, err = pack(sa, labels, 4)
    assert err == 1


def test_centroid_scores(sa):
    inp = W.decode_clustered(2, T=8, Hq=32, Hkv=8, Nctx=512, d=128, C=256)
    t = torch()
    s = t.empty((8, 32, 256), dtype=t.float32, device="cuda:0")
    sa.sa_estimate(sa.CENTROID, dev_bf16(inp.q), dev_bf16(inp.k), s, centroids=dev_f32(inp.centroids),
                   scale=1 / math.sqrt(128))
    t.cuda.synchronize()
    want = oracle.centroid_scores(W.bf16_to_f32(inp.q), inp.centroids, 1 / math.sqrt(128))
    assert_scores_close(host(s), want, "centroid scores")


def run_decode(sa, inp, C, sel_np, out_bf16=False):
    t = torch()
    ptr, perm, kp, vp, _ = pack(sa, inp.labels, C, dev_bf16(inp.k), dev_bf16(inp.v))
    T, Hq, d = inp.q.shape
    out = t.empty((T, Hq, d), dtype=t.bfloat16 if out_bf16 else t.float32, device="cuda:0")
    lse = t.empty((T, Hq), dtype=t.float32, device="cuda:0")
    sa.sa_gather_decode(dev_bf16(inp.q), kp, vp, out, cluster_ptr=ptr, sel=dev_i32(sel_np), lse=lse,
                        scale=1 / math.sqrt(d))
    t.cuda.synchronize()
    return host(out), host(lse)


@pytest.mark.parametrize("T,Hq,Hkv,N,C,ksel", [(8, 32, 8, 8192, 64, 16), (2, 8, 2, 3001, 20, 5),
                                               (16, 16, 4, 4096, 32, 8)])
def test_cluster_decode_on_oracle_selection(sa, T, Hq, Hkv, N, C, ksel):
    print(f"decode T{T} Hq{Hq} Hkv{Hkv} N{N} C{C} k{ksel}", flush=True)
    inp = W.decode_clustered(3, T, Hq, Hkv, N, 128, C)
    scale = 1 / math.sqrt(128)
    s = oracle.centroid_scores(W.bf16_to_f32(inp.q), inp.centroids, scale)
    sel = oracle.cluster_select(s, ksel)
    sel_np = np.array([[sel[t][h] for h in range(Hq)] for t in range(T)], np.int32)
    o, l = run_decode(sa, inp, C, sel_np)
    wo, wl = oracle.cluster_decode(W.bf16_to_f32(inp.q), W.bf16_to_f32(inp.k), W.bf16_to_f32(inp.v), inp.labels,
                                   sel, scale)
    assert_attention_close(o, wo, bf16=True, what="cluster decode")
    assert np.max(np.abs(l - wl)) < 1e-3


def test_cluster_decode_all_clusters_is_dense_and_dup_ignored(sa):
    T, Hq, Hkv, N, C = 4, 8, 2, 2048, 16
    inp = W.decode_clustered(4, T, Hq, Hkv, N, 128, C)
    sel_np = np.tile(np.arange(C, dtype=np.int32), (T, Hq, 1))
    sel_np[:, :, -1] = sel_np[:, :, 0]                 # a duplicate: counts once
    sel_np[:, :, -2] = -1                              # padding: ignored
    o, _ = run_decode(sa, inp, C, sel_np)
    keep = [[np.arange(C - 2) for _ in range(Hq)] for _ in range(T)]
    wo, _ = oracle.cluster_decode(W.bf16_to_f32(inp.q), W.bf16_to_f32(inp.k), W.bf16_to_f32(inp.v), inp.labels,
                                  keep, 1 / math.sqrt(128))
    assert_attention_close(o, wo, bf16=True, what="all clusters")


def test_decode_end_to_end_full_size_certified(sa):
    """8 queries x 32/8 heads over 65536 clustered keys, top 64 of 256: the
    pipeline the benchmark times, with certified query redraws."""
    from dynamic_sparse_attention_pool_amd.pipelines import ClusterDecode
    seed = W.CONFIG_SEEDS[4]
    T, Hq, Hkv, N, d, C, ksel = 8, 32, 8, 65536, 128, 256, 64
    inp = W.decode_clustered(seed, T, Hq, Hkv, N, d, C)
    scale = 1 / math.sqrt(d)
    none = np.zeros(0, np.int64)
    for t in range(T):
        for h in range(Hq):
            a = 0
            while not oracle.certified_row(oracle.centroid_scores(W.bf16_to_f32(inp.q[t:t + 1, h:h + 1]),
                                                                  inp.centroids[h * Hkv // Hq:h * Hkv // Hq + 1],
                                                                  scale)[0, 0], ksel, none):
                a += 1
                inp.q[t, h] = W.redraw_decode_query(seed, t, h, a, d)
    dc = ClusterDecode(dev_bf16(inp.q), dev_bf16(inp.k), dev_bf16(inp.v), dev_i32(inp.labels),
                       dev_f32(inp.centroids), n_sel=ksel, with_lse=True)
    dc.step()
    torch().cuda.synchronize()
    s = oracle.centroid_scores(W.bf16_to_f32(inp.q), inp.centroids, scale)
    sel = oracle.cluster_select(s, ksel)
    got = host(dc.sel)
    for t in range(T):
        for h in range(Hq):
            assert np.array_equal(got[t, h], sel[t][h]), (t, h)
    wo, wl = oracle.cluster_decode(W.bf16_to_f32(inp.q), W.bf16_to_f32(inp.k), W.bf16_to_f32(inp.v), inp.labels,
                                   sel, scale)
    assert_attention_close(host(dc.out), wo, bf16=True, what="full-size decode")


@pytest.mark.parametrize("T,N,ntok", [(37, 9000, 2048), (8, 4096, 100), (4, 131072, 2048)])
def test_token_gather_mqa(sa, T, N, ntok):
    print(f"token gather T{T} N{N} ntok{ntok}", flush=True)
    r = np.random.default_rng(5)
    L = W.mqa_layer(6, 0, T, 16, 1, N, 128)
    idx = np.full((T, ntok), -1, np.int32)
    lists = []
    for t in range(T):
        n = ntok if t % 3 else max(1, ntok - 17 * (t + 1))         # ragged rows, -1 padded
        n = min(n, N)
        ids = np.sort(r.choice(N, size=n, replace=False)).astype(np.int32)
        idx[t, :n] = ids
        lists.append(ids)
    tt = torch()
    out = tt.empty((T, 16, 128), dtype=tt.float32, device="cuda:0")
    lse = tt.empty((T, 16), dtype=tt.float32, device="cuda:0")
    sa.sa_gather_decode(dev_bf16(L.q), dev_bf16(L.k), dev_bf16(L.v), out, tok_idx=dev_i32(idx), lse=lse)
    tt.cuda.synchronize()
    wo, wl = oracle.gathered_attention(W.bf16_to_f32(L.q), W.bf16_to_f32(L.k), W.bf16_to_f32(L.v), lists,
                                       1 / math.sqrt(128))
    assert_attention_close(host(out), wo, bf16=True, what="token gather")
    assert np.max(np.abs(host(lse) - wl)) < 1e-3


@pytest.mark.parametrize("T,Hq,Hkv,C,k,dt", [(8, 32, 8, 256, 64, "bf16"), (3, 6, 2, 1000, 37, "f32"),
                                            (2, 8, 1, 300, 400, "bf16"), (5, 4, 4, 17, 5, "f32"),
                                            (4, 8, 2, 1024, 100, "bf16"), (3, 8, 2, 400, 50, "f32")])
def test_fused_centroid_topk_matches_oracle_and_separate_path(sa, T, Hq, Hkv, C, k, dt):
    """sa_estimate_topk(CENTROID) keeps the oracle's clusters on certified rows
    and equals the separate scores + selection bit for bit (same arithmetic)."""
    print(f"fused centroid T{T} Hq{Hq} Hkv{Hkv} C{C} k{k} {dt}", flush=True)
    t = torch()
    inp = W.decode_clustered(61, T, Hq, Hkv, 64, 128, C)
    qf = W.bf16_to_f32(inp.q)
    q = dev_bf16(inp.q) if dt == "bf16" else dev_f32(qf)
    cent = dev_f32(inp.centroids)
    if k == 5:   # tied scores: duplicate centroids
        c2 = inp.centroids.copy()
        c2[:, 1::2] = c2[:, 0::2][:, :c2[:, 1::2].shape[1]]
        cent = dev_f32(c2)
        inp.centroids = c2
    kmax = min(k, C) + 2
    sel = t.full((T, Hq, kmax), 9, dtype=t.int32, device="cuda:0")
    cnt = t.full((T, Hq), -1, dtype=t.int32, device="cuda:0")
    sa.sa_estimate_topk_centroid(q, cent, sel, cnt, k=k, scale=1 / math.sqrt(128))
    s = t.empty((T, Hq, C), dtype=t.float32, device="cuda:0")
    sa.sa_estimate(sa.CENTROID, q, q, s, centroids=cent, scale=1 / math.sqrt(128))
    sel2 = t.full((T * Hq, kmax), 9, dtype=t.int32, device="cuda:0")
    cnt2 = t.full((T * Hq,), -1, dtype=t.int32, device="cuda:0")
    sa.sa_select_topk(s.view(T * Hq, C), sel2, cnt2, k=k)
    t.cuda.synchronize()
    got, gcnt = host(sel), host(cnt)
    assert np.array_equal(got.reshape(T * Hq, kmax), host(sel2)) and np.array_equal(gcnt.reshape(-1), host(cnt2))
    assert np.all(gcnt == min(k, C)) and np.all(got[:, :, min(k, C):] == -1)
    want_s = oracle.centroid_scores(qf, inp.centroids, 1 / math.sqrt(128))
    none = np.zeros(0, np.int64)
    for tt in range(T):
        for h in range(Hq):
            if oracle.certified_row(want_s[tt, h], min(k, C), none):
                assert np.array_equal(got[tt, h, :min(k, C)], oracle.topk_row(want_s[tt, h], k, none)), (tt, h)


def test_fused_centroid_topk_nan_flag(sa):
    t = torch()
    inp = W.decode_clustered(62, 2, 8, 2, 64, 128, 40)
    qf = W.bf16_to_f32(inp.q).copy()
    qf[1, 5, 3] = np.nan
    sel = t.empty((2, 8, 10), dtype=t.int32, device="cuda:0")
    cnt = t.empty((2, 8), dtype=t.int32, device="cuda:0")
    err = t.zeros(1, dtype=t.int32, device="cuda:0")
    sa.sa_estimate_topk_centroid(dev_f32(qf), dev_f32(inp.centroids), sel, cnt, k=10, err_flag=err)
    t.cuda.synchronize()
    assert int(host(err)[0]) == 1


def test_decode_end_to_end_full_size_fused_estimate(sa):
    """The full-size decode step with the fused centroid top-k: same clusters
    as the oracle on certified rows, outputs within the bf16 bounds."""
    from dynamic_sparse_attention_pool_amd.pipelines import ClusterDecode
    seed = W.CONFIG_SEEDS[4]
    T, Hq, Hkv, N, d, C, ksel = 8, 32, 8, 65536, 128, 256, 64
    inp = W.decode_clustered(seed, T, Hq, Hkv, N, d, C)
    scale = 1 / math.sqrt(d)
    dc = ClusterDecode(dev_bf16(inp.q), dev_bf16(inp.k), dev_bf16(inp.v), dev_i32(inp.labels),
                       dev_f32(inp.centroids), n_sel=ksel, with_lse=True, fused=True)
    dc.step()
    torch().cuda.synchronize()
    s = oracle.centroid_scores(W.bf16_to_f32(inp.q), inp.centroids, scale)
    none = np.zeros(0, np.int64)
    got = host(dc.sel)
    rows = [(t, h) for t in range(T) for h in range(Hq) if oracle.certified_row(s[t, h], ksel, none)]
    assert len(rows) > 0.6 * T * Hq
    sel = oracle.cluster_select(s, ksel)
    for t, h in rows:
        assert np.array_equal(got[t, h], sel[t][h]), (t, h)
    # every other row: a valid top-64 up to near-ties of the fp64 scores
    for t in range(T):
        for h in range(Hq):
            assert tie_tolerant_valid(np.sort(got[t, h]), s[t, h], ksel, none), (t, h)
    # all outputs against the oracle's decode over the clusters the GPU chose
    gsel = [[np.sort(got[t, h]) for h in range(Hq)] for t in range(T)]
    wo, _ = oracle.cluster_decode(W.bf16_to_f32(inp.q), W.bf16_to_f32(inp.k), W.bf16_to_f32(inp.v), inp.labels,
                                  gsel, scale)
    assert_attention_close(host(dc.out), wo, bf16=True, what="fused decode")
