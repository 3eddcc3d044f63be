"""GPU parity of the A-shape forward, of head-list launches (estimates and
forward over a subset of query heads with compact tables) and of the layer
that runs a given pattern per head, against the CPU oracle."""
import math

import numpy as np
import pytest

import oracle
import workloads as W
from gpu_helpers import (assert_attention_close, assert_scores_close, dev_bf16, dev_f32, dev_i32, lower_triangle,
                         fwd_on_oracle_blocks, fwd_on_oracle_vs, host, pad_table, tie_tolerant_valid, torch)

pytestmark = pytest.mark.gpu

NONE = np.zeros(0, np.int64)


@pytest.fixture(scope="module")
def sa():
    import dynamic_sparse_attention_pool_amd as m
    m.load()
    return m


def run_ashape(sa, q, k, v, n_sink, n_local, out_dtype, heads=None, fill=None):
    t = torch()
    B, Hq, N, d = q.shape
    out = t.empty((B, Hq, N, d), dtype=out_dtype, device=q.device)
    lse = t.empty((B, Hq, N), dtype=t.float32, device=q.device)
    if fill is not None:
        out.fill_(fill)
        lse.fill_(fill)
    sa.sa_block_sparse_fwd(q, k, v, out, ashape=(n_sink, n_local), lse=lse, heads=heads)
    t.cuda.synchronize()
    return host(out), host(lse)


@pytest.mark.parametrize("n_sink,n_local", [(1, 4), (0, 1), (2, 3), (1, 100), (0, 0), (3, 0)])
@pytest.mark.parametrize("d,out_bf16", [(128, False), (128, True), (64, False)])
def test_ashape_forward_bf16(sa, n_sink, n_local, d, out_bf16):
    print(f"ashape bf16 d{d} sink {n_sink} local {n_local} out_bf16 {out_bf16}", flush=True)
    t = torch()
    inp = W.prefill_bf16(91, 2, 4, 2, 1024, d)
    o, l = run_ashape(sa, dev_bf16(inp.q), dev_bf16(inp.k), dev_bf16(inp.v), n_sink, n_local,
                      t.bfloat16 if out_bf16 else t.float32)
    wo, wl = oracle.ashape_attention(inp.f32("q"), inp.f32("k"), inp.f32("v"), n_sink, n_local, 64, 1 / math.sqrt(d))
    assert_attention_close(o, wo, bf16=True, what="A-shape")
    assert np.array_equal(np.isneginf(l), np.isneginf(wl))
    fin = np.isfinite(wl)
    assert np.max(np.abs(l[fin] - wl[fin]), initial=0.0) < 1e-3
    if n_sink == 0 and n_local == 0:
        assert np.all(o == 0)


@pytest.mark.parametrize("n_sink,n_local", [(1, 2), (0, 3)])
def test_ashape_forward_fp32_with_head_list(sa, n_sink, n_local):
    t = torch()
    inp = W.prefill_fp32(92, 1, 4, 512, 64)
    heads = [3, 1]
    o, l = run_ashape(sa, dev_f32(inp.q), dev_f32(inp.k), dev_f32(inp.v), n_sink, n_local, t.float32,
                      heads=heads, fill=7.0)
    wo, wl = oracle.ashape_attention(inp.q, inp.k, inp.v, n_sink, n_local, 64, 1 / 8.0, heads=heads)
    assert_attention_close(o[:, heads], wo[:, heads], bf16=False, what="A-shape fp32")
    assert np.max(np.abs(l[:, heads] - wl[:, heads])) < 1e-5
    assert np.all(o[:, [0, 2]] == 7.0) and np.all(l[:, [0, 2]] == 7.0)     # unlisted heads untouched


def test_head_list_block_forward_compact_tables(sa):
    """Listed heads in any order read rows b*n + j of compact tables; other
    heads' outputs stay as they were."""
    t = torch()
    B, Hq, Hkv, N, d = 2, 8, 2, 1024, 128
    nb = N // 64
    inp = W.prefill_bf16(93, B, Hq, Hkv, N, d)
    scale = 1 / math.sqrt(d)
    S = oracle.block_scores(inp.f32("q"), inp.f32("k"), 64, scale)
    kept = oracle.block_select(S, n_sink=1, n_local=2, ratio=(25, 100))
    heads = [5, 0, 3]
    flat = [kept[b][h][i] for b in range(B) for h in heads for i in range(nb)]
    kmax = 3 + math.ceil(0.25 * nb)
    idx, cnt = pad_table(flat, kmax)
    out = t.full((B, Hq, N, d), 7.0, dtype=t.float32, device="cuda:0")
    lse = t.full((B, Hq, N), 7.0, dtype=t.float32, device="cuda:0")
    sa.sa_block_sparse_fwd(dev_bf16(inp.q), dev_bf16(inp.k), dev_bf16(inp.v), out,
                           block_idx=dev_i32(idx.reshape(B, 3, nb, kmax)), block_cnt=dev_i32(cnt.reshape(B, 3, nb)),
                           lse=lse, heads=heads)
    t.cuda.synchronize()
    o, l = host(out), host(lse)
    wo, wl = oracle.block_sparse_attention(inp.f32("q"), inp.f32("k"), inp.f32("v"), kept, 64, scale, heads=heads)
    assert_attention_close(o[:, heads], wo[:, heads], bf16=True, what="head-list forward")
    assert np.max(np.abs(l[:, heads] - wl[:, heads])) < 1e-3
    others = [h for h in range(Hq) if h not in heads]
    assert np.all(o[:, others] == 7.0) and np.all(l[:, others] == 7.0)


def test_head_list_estimates_are_compact(sa):
    t = torch()
    B, Hq, Hkv, N, d = 2, 8, 2, 1024, 128
    nb = N // 64
    inp = W.prefill_bf16(94, B, Hq, Hkv, N, d)
    scale = 1 / math.sqrt(d)
    q, k = dev_bf16(inp.q), dev_bf16(inp.k)
    heads = [6, 1, 2]
    s = t.empty((B, 3, nb, nb), dtype=t.float32, device="cuda:0")
    pq = t.empty((B, 3, nb, d), dtype=t.float32, device="cuda:0")
    sa.sa_estimate(sa.BLOCK_MEANPOOL, q, k, s, scale=scale, pooled_q=pq, heads=heads)
    av = t.empty((B, 3, N), dtype=t.float32, device="cuda:0")
    as_ = t.empty((B, 3, N), dtype=t.float32, device="cuda:0")
    sa.sa_estimate(sa.VSLASH, q, k, av, scores2=as_, scale=scale, heads=heads)
    t.cuda.synchronize()
    want = oracle.block_scores(inp.f32("q"), inp.f32("k"), 64, scale)
    assert_scores_close(lower_triangle(host(s)), want[:, heads], "compact block scores")
    pw = np.stack([[oracle.mean_pool(inp.f32("q")[b, h], 64) for h in heads] for b in range(B)])
    assert np.max(np.abs(host(pq) - pw)) < 1e-5
    for b in range(B):
        for j, h in enumerate(heads):
            g = oracle.gqa_group(h, Hq, Hkv)
            wv, ws = oracle.vs_estimate(inp.f32("q")[b, h, N - 64:], inp.f32("k")[b, g], np.arange(N - 64, N), scale)
            assert_scores_close(host(av)[b, j][None], wv[None], f"compact vertical b{b} h{h}")
            assert_scores_close(host(as_)[b, j][None], ws[None], f"compact slash b{b} h{h}")


PATTERNS = ["BS", "A", "VS", "BS", "A", "VS", "VS", "BS"]


def test_mixed_layer_end_to_end(sa):
    """Eight heads over two KV heads with a mixed assignment; every head's
    selection matches the oracle exactly where certified and is tie-tolerant
    valid elsewhere; outputs match wherever the selections are identical."""
    from dynamic_sparse_attention_pool_amd.pipelines import MixedPatternLayer
    B, Hq, Hkv, N, d = 1, 8, 2, 2048, 128
    nb = N // 64
    nv, ns = 100, 16
    scale = 1 / math.sqrt(d)
    base = W.prefill_bf16(95, B, Hq, Hkv, N, d)
    inp, _, _ = W.plant_vertical_slash(base, 95, nv, ns, 100.0, 3.0)
    block = dict(n_sink=1, n_local=4, ratio=(10, 100))
    layer = MixedPatternLayer(dev_bf16(inp.q), dev_bf16(inp.k), dev_bf16(inp.v), PATTERNS, a_shape=(1, 3),
                              block=block, vslash=(nv, ns), out_dtype=torch().float32, with_lse=True)
    layer.step()
    torch().cuda.synchronize()
    o, l = host(layer.out), host(layer.lse)
    wo, wl, wsel = oracle.mixed_layer(inp.f32("q"), inp.f32("k"), inp.f32("v"), PATTERNS, bs=64, scale=scale,
                                      a_shape=(1, 3), block=block, vslash=(nv, ns))
    parts = {type(p).__name__: p for p in layer.parts}
    bsl, vsl = parts["BlockSparseLayer"], parts["VerticalSlashLayer"]
    S = oracle.block_scores(inp.f32("q"), inp.f32("k"), 64, scale)
    same_rows = 0
    for h in range(Hq):
        if PATTERNS[h] == "A":
            assert_attention_close(o[0, h], wo[0, h], bf16=True, what=f"A head {h}")
            assert np.max(np.abs(l[0, h] - wl[0, h])) < 1e-3
        elif PATTERNS[h] == "BS":
            j = bsl.heads.index(h)
            idx, cnt = host(bsl.idx)[0, j], host(bsl.cnt)[0, j]
            differ = {}
            for i in range(nb):
                got = idx[i, :cnt[i]]
                want = wsel[0][h][i]
                f = oracle.forced_set(i + 1, 1, 4)
                kr = oracle.budget(i + 1, len(f), None, (10, 100))
                if np.array_equal(got, want):
                    same_rows += 1
                    rows = slice(64 * i, 64 * i + 64)
                    assert_attention_close(o[0, h, rows], wo[0, h, rows], bf16=True, what=f"BS head {h} block {i}")
                else:
                    assert not oracle.certified_row(S[0, h, i, :i + 1], kr, f), (h, i)
                    assert tie_tolerant_valid(got, S[0, h, i, :i + 1], kr, f), (h, i)
                    differ[i] = want
            if differ:
                oo = fwd_on_oracle_blocks(sa, bsl.q, bsl.k, bsl.v, h, differ, bsl.kmax)
                for i in differ:
                    rows = slice(64 * i, 64 * i + 64)
                    assert_attention_close(oo[rows], wo[0, h, rows], bf16=True, what=f"BS head {h} block {i} (oracle)")
        else:
            j = vsl.heads.index(h)
            vh, sh = host(vsl.vert)[j], host(vsl.slash)[j]
            cols, offs = wsel[0][h]
            if np.array_equal(vh, cols) and np.array_equal(sh, offs):
                assert_attention_close(o[0, h], wo[0, h], bf16=True, what=f"VS head {h}")
            else:
                g = oracle.gqa_group(h, Hq, Hkv)
                wv, ws = oracle.vs_estimate(inp.f32("q")[0, h, N - 64:], inp.f32("k")[0, g], np.arange(N - 64, N),
                                            scale)
                assert tie_tolerant_valid(vh, wv, nv, NONE) and tie_tolerant_valid(sh, ws, ns, NONE), h
                oo = fwd_on_oracle_vs(sa, vsl.q, vsl.k, vsl.v, h, cols, offs, ns, nv)
                assert_attention_close(oo, wo[0, h], bf16=True, what=f"VS head {h} on oracle tables")
    assert same_rows >= 0.8 * 3 * nb


def test_mixed_layer_heads_bitwise_equal_single_pattern_layers(sa):
    """A head computed inside a mixed layer is bit-for-bit the head computed by
    the single-pattern layer over all heads: the head list changes only which
    workgroups run, not their arithmetic."""
    from dynamic_sparse_attention_pool_amd.pipelines import AShapeLayer, BlockSparseLayer, MixedPatternLayer
    inp = W.prefill_bf16(96, 1, 8, 2, 2048, 128)
    q, k, v = dev_bf16(inp.q), dev_bf16(inp.k), dev_bf16(inp.v)
    block = dict(n_sink=1, n_local=4, ratio=(10, 100))
    pats = ["BS", "A"] * 4
    mixed = MixedPatternLayer(q, k, v, pats, a_shape=(2, 2), block=block)
    bs_all = BlockSparseLayer(q, k, v, **block)
    a_all = AShapeLayer(q, k, v, n_sink=2, n_local=2)
    for layer in (mixed, bs_all, a_all):
        layer.step()
    torch().cuda.synchronize()
    m, b, a = host(mixed.out.float()), host(bs_all.out.float()), host(a_all.out.float())
    for h, p in enumerate(pats):
        ref = b if p == "BS" else a
        assert np.array_equal(m[0, h], ref[0, h]), (h, p)


def test_mixed_layer_full_size_sampled(sa):
    """131072 tokens, 32/8 heads, one A, one VS and two BS heads per KV head
    (sink + 4 local + ceil(5%) for BS; 1000 columns and 64 offsets for VS;
    sink + 4 local for A): sampled heads and query blocks against the oracle."""
    from dynamic_sparse_attention_pool_amd.pipelines import MixedPatternLayer
    N, d, Hq, Hkv = 131072, 128, 32, 8
    pats = [("A", "VS", "BS", "BS")[h % 4] for h in range(Hq)]
    sample = [0, 1, 2, 29]
    inp = W.prefill_bf16(W.CONFIG_SEEDS[3], 1, Hq, Hkv, N, d, heads=sample)
    block = dict(n_sink=1, n_local=4, ratio=(5, 100))
    layer = MixedPatternLayer(dev_bf16(inp.q), dev_bf16(inp.k), dev_bf16(inp.v), pats, a_shape=(1, 4),
                              block=block, vslash=(1000, 64), out_dtype=torch().float32)
    layer.out.fill_(float("nan"))   # the three head-list launches together write every row
    layer.step()
    torch().cuda.synchronize()
    assert bool(torch().isfinite(layer.out).all()), "some output rows were not written"
    scale = 1 / math.sqrt(d)
    parts = {type(p).__name__: p for p in layer.parts}
    bsl, vsl = parts["BlockSparseLayer"], parts["VerticalSlashLayer"]
    blocks = [0, 3, 1000, 2047]
    for h in sample:
        g = oracle.gqa_group(h, Hq, Hkv)
        o = host(layer.out[0, h])
        if pats[h] == "A":
            wo, _ = oracle.ashape_attention(inp.f32("q"), inp.f32("k"), inp.f32("v"), 1, 4, 64, scale, heads=[h],
                                            blocks=blocks)
        elif pats[h] == "BS":
            j = bsl.heads.index(h)
            idx, cnt = host(bsl.idx)[0, j], host(bsl.cnt)[0, j]
            qbar = oracle.mean_pool(inp.f32("q")[0, h], 64)
            kbar = oracle.mean_pool(inp.f32("k")[0, g], 64)
            kept = [[[None] * (N // 64) for _ in range(Hq)]]
            for i in blocks:
                s = (kbar[:i + 1] @ qbar[i]) * scale
                f = oracle.forced_set(i + 1, 1, 4)
                kr = oracle.budget(i + 1, len(f), None, (5, 100))
                got = idx[i, :cnt[i]]
                if oracle.certified_row(s, kr, f):
                    assert np.array_equal(got, oracle.topk_row(s, kr, f)), (h, i)
                else:
                    assert tie_tolerant_valid(got, s, kr, f), (h, i)
                kept[0][h][i] = oracle.topk_row(s, kr, f)
            wo, _ = oracle.block_sparse_attention(inp.f32("q"), inp.f32("k"), inp.f32("v"), kept, 64, scale,
                                                  heads=[h], blocks=blocks)
            differ = {i: kept[0][h][i] for i in blocks if not np.array_equal(idx[i, :cnt[i]], kept[0][h][i])}
            if differ:   # near-tied rows: the forward on the oracle's own blocks
                oo = fwd_on_oracle_blocks(sa, layer.q, layer.k, layer.v, h, differ, idx.shape[-1])
                for i in differ:
                    o[64 * i:64 * i + 64] = oo[64 * i:64 * i + 64]
        else:
            j = vsl.heads.index(h)
            wv, ws = oracle.vs_estimate(inp.f32("q")[0, h, N - 64:], inp.f32("k")[0, g], np.arange(N - 64, N), scale)
            vh, sh = host(vsl.vert)[j], host(vsl.slash)[j]
            for got, sc, kk in [(vh, wv, 1000), (sh, ws, 64)]:
                if oracle.certified_row(sc, kk, NONE):
                    assert np.array_equal(got, oracle.topk_row(sc, kk, NONE))
                else:
                    assert tie_tolerant_valid(got, sc, kk, NONE)
            cols, offs = oracle.vs_select(wv, ws, 1000, 64)
            sel = [[None] * Hq]
            sel[0][h] = (cols, offs)
            wo, _ = oracle.vs_attention(inp.f32("q"), inp.f32("k"), inp.f32("v"), sel, 64, scale, heads=[h],
                                        blocks=blocks)
            if not (np.array_equal(vh, cols) and np.array_equal(sh, offs)):
                o = fwd_on_oracle_vs(sa, layer.q, layer.k, layer.v, h, cols, offs, 64, 1000)
        for i in blocks:
            rows = slice(64 * i, 64 * i + 64)
            assert_attention_close(o[rows], wo[0, h, rows], bf16=True, what=f"{pats[h]} head {h} block {i}")
