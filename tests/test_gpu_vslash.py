"""GPU parity of the vertical-slash path: last-query estimate, top columns /
offsets, per-block tables and the forward in tile-list mode."""
import math

import numpy as np
import pytest

import oracle
import workloads as W
from gpu_helpers import (dev_f32, assert_attention_close, assert_scores_close, dev_bf16, dev_i32, fwd_on_oracle_vs, host,
                         tie_tolerant_valid, torch)

pytestmark = pytest.mark.gpu

NONE = np.zeros(0, np.int64)


@pytest.fixture(scope="module")
def sa():
    import dynamic_sparse_attention_pool_amd as m
    m.load()
    return m


def oracle_vs_scores(inp, h, scale):
    B, Hq, N, d = inp.q.shape
    g = oracle.gqa_group(h, Hq, inp.k.shape[1])
    return oracle.vs_estimate(inp.f32("q")[0, h, N - 64:], inp.f32("k")[0, g], np.arange(N - 64, N), scale)


@pytest.mark.parametrize("N,d", [(2048, 128), (1024, 64)])
def test_vs_estimate(sa, N, d):
    inp = W.prefill_bf16(51, 1, 4, 2, N, d)
    t = torch()
    av = t.empty((1, 4, N), dtype=t.float32, device="cuda:0")
    as_ = t.empty((1, 4, N), dtype=t.float32, device="cuda:0")
    scale = 1 / math.sqrt(d)
    sa.sa_estimate(sa.VSLASH, dev_bf16(inp.q), dev_bf16(inp.k), av, scores2=as_, scale=scale)
    t.cuda.synchronize()
    for h in range(4):
        wv, ws = oracle_vs_scores(inp, h, scale)
        assert_scores_close(host(av)[0, h][None], wv[None], "vertical")
        assert_scores_close(host(as_)[0, h][None], ws[None], "slash")
        assert abs(host(av)[0, h].sum() - 64) < 1e-3 and abs(host(as_)[0, h].sum() - 64) < 1e-3


@pytest.mark.parametrize("Hq,Hkv,heads,N,d", [(8, 1, None, 1024, 128), (16, 2, [3, 9, 12, 15, 4], 1024, 128),
                                            (3, 3, None, 1024, 128), (6, 1, [5, 0], 1024, 128),
                                            (4, 1, None, 64, 128), (8, 2, [7], 128, 64), (5, 5, None, 1088, 64)])
def test_vs_estimate_group_shapes(sa, Hq, Hkv, heads, N, d):
    """Query heads per KV head 8, 1, 6 and 4 (workgroups cover up to four of a
    KV head's query heads, so these need two blocks, a partial block or one
    head per block), with and without a head list, batch 2; one- and two-tile
    contexts and a chunk of one tile (17 tiles)."""
    B = 2
    inp = W.prefill_bf16(53, B, Hq, Hkv, N, d)
    lst = list(range(Hq)) if heads is None else heads
    t = torch()
    av = t.empty((B, len(lst), N), dtype=t.float32, device="cuda:0")
    as_ = t.empty_like(av)
    scale = 1 / math.sqrt(d)
    sa.sa_estimate(sa.VSLASH, dev_bf16(inp.q), dev_bf16(inp.k), av, scores2=as_, scale=scale, heads=heads)
    t.cuda.synchronize()
    for b in range(B):
        for j, h in enumerate(lst):
            g = oracle.gqa_group(h, Hq, Hkv)
            wv, ws = oracle.vs_estimate(inp.f32("q")[b, h, N - 64:], inp.f32("k")[b, g], np.arange(N - 64, N), scale)
            assert_scores_close(host(av)[b, j][None], wv[None], f"vertical b{b} h{h}")
            assert_scores_close(host(as_)[b, j][None], ws[None], f"slash b{b} h{h}")


@pytest.mark.parametrize("ns", [40, 64, 100])  # up to 64 offsets: one wave per row; more: one thread per row
def test_vs_build_tables_exact(sa, ns):
    N, R, nv = 4096, 5, 300
    r = np.random.default_rng(52)
    cols = [np.sort(r.choice(N, size=nv, replace=False)) for _ in range(R)]
    offs = [np.sort(r.choice(N, size=ns, replace=False)) for _ in range(R)]
    offs[1][:3] = [0, 1, 2]
    offs[1] = np.sort(offs[1])
    vert = np.array(cols, np.int32)
    slash = np.array(offs, np.int32)
    t = torch()
    nb = N // 64
    iv = t.empty((R, nb, ns, 2), dtype=t.int32, device="cuda:0")
    ivc = t.empty((R, nb), dtype=t.int32, device="cuda:0")
    col = t.empty((R, nb, nv), dtype=t.int32, device="cuda:0")
    colc = t.empty((R, nb), dtype=t.int32, device="cuda:0")
    cnt_v = np.full(R, nv, np.int32)
    cnt_v[2] = 17                                    # a short selection row
    sa.sa_vs_build(dev_i32(vert), dev_i32(cnt_v), dev_i32(slash), dev_i32(np.full(R, ns, np.int32)),
                   iv.view(R, -1), ivc, col.view(R, -1), colc, seq=N)
    t.cuda.synchronize()
    ivh, ivch, colh, colch = host(iv), host(ivc), host(col), host(colc)
    for rr in range(R):
        tables = oracle.vs_block_tables(cols[rr][:cnt_v[rr]], offs[rr], N, 64)
        for i, (ivs, vert_i) in enumerate(tables):
            assert ivch[rr, i] == len(ivs)
            assert [tuple(x) for x in ivh[rr, i, :len(ivs)]] == ivs
            assert np.array_equal(colh[rr, i, :colch[rr, i]], vert_i)


def run_vs_fwd(sa, inp, sel, N, out_bf16=False):
    """forward in tile-list mode on tables built by the library from sel."""
    t = torch()
    B, Hq = inp.q.shape[:2]
    nv = max(len(c) for c, _ in sel[0])
    ns = max(len(o) for _, o in sel[0])
    vert = np.zeros((Hq, nv), np.int32)
    slash = np.zeros((Hq, ns), np.int32)
    cv = np.zeros(Hq, np.int32)
    cs = np.zeros(Hq, np.int32)
    for h, (c, o) in enumerate(sel[0]):
        vert[h, :len(c)], cv[h] = c, len(c)
        slash[h, :len(o)], cs[h] = o, len(o)
    nb = N // 64
    iv = t.empty((B, Hq, nb, ns, 2), dtype=t.int32, device="cuda:0")
    ivc = t.empty((B, Hq, nb), dtype=t.int32, device="cuda:0")
    col = t.empty((B, Hq, nb, nv), dtype=t.int32, device="cuda:0")
    colc = t.empty((B, Hq, nb), dtype=t.int32, device="cuda:0")
    sa.sa_vs_build(dev_i32(vert), dev_i32(cv), dev_i32(slash), dev_i32(cs), iv.view(Hq, -1), ivc.view(Hq, -1),
                   col.view(Hq, -1), colc.view(Hq, -1), seq=N)
    out = t.empty(inp.q.shape, dtype=t.bfloat16 if out_bf16 else t.float32, device="cuda:0")
    lse = t.empty((B, Hq, N), dtype=t.float32, device="cuda:0")
    up = dev_bf16 if inp.dtype == "bf16" else dev_f32
    sa.sa_block_sparse_fwd(up(inp.q), up(inp.k), up(inp.v), out, iv=iv, iv_cnt=ivc, col=col, col_cnt=colc, lse=lse)
    t.cuda.synchronize()
    return host(out), host(lse)


def test_vs_forward_on_oracle_selection(sa):
    N, d = 2048, 128
    inp = W.prefill_bf16(53, 1, 4, 2, N, d)
    r = np.random.default_rng(53)
    sel = [[(np.sort(r.choice(N, size=150, replace=False)), np.sort(r.choice(N, size=12, replace=False)))
            for _ in range(4)]]
    # block-aligned slash tiles cover every causal key (1920 columns: the bf16 path's table capacity)
    sel[0][2] = (np.arange(1920), np.arange(0, N, 64))
    sel[0][3] = (np.sort(r.choice(N, size=5, replace=False)), np.array([1000, 1500]))   # many empty rows
    o, l = run_vs_fwd(sa, inp, sel, N)
    wo, wl = oracle.vs_attention(inp.f32("q"), inp.f32("k"), inp.f32("v"), sel, 64, 1 / math.sqrt(d))
    assert_attention_close(o, wo, bf16=True, what="vs forward")
    assert np.array_equal(np.isneginf(l), np.isneginf(wl))
    fin = np.isfinite(wl)
    assert np.max(np.abs(l[fin] - wl[fin])) < 1e-3


@pytest.mark.parametrize("d,dtype,out_bf16", [(128, "bf16", True), (64, "bf16", False), (64, "bf16", True),
                                             (64, "f32", False), (128, "f32", False)])
def test_vs_forward_head_dims_and_dtypes(sa, d, dtype, out_bf16):
    """The tile-list forward for each head size, input type and output type
    on random vertical and slash selections, against the oracle."""
    N, H = 1024, 2
    inp = W.prefill_bf16(54, 1, H, H, N, d) if dtype == "bf16" else W.prefill_fp32(54, 1, H, N, d)
    r = np.random.default_rng(54)
    sel = [[(np.sort(r.choice(N, size=90, replace=False)), np.sort(r.choice(N, size=9, replace=False)))
            for _ in range(H)]]
    o, l = run_vs_fwd(sa, inp, sel, N, out_bf16=out_bf16)
    wo, wl = oracle.vs_attention(inp.f32("q"), inp.f32("k"), inp.f32("v"), sel, 64, 1 / math.sqrt(d))
    assert_attention_close(o, wo, bf16=dtype == "bf16", what=f"vs forward d{d} {dtype} out_bf16={out_bf16}")
    assert np.array_equal(np.isneginf(l), np.isneginf(wl))
    fin = np.isfinite(wl)
    assert np.max(np.abs(l[fin] - wl[fin])) < (1e-3 if dtype == "bf16" else 1e-5)


def test_vs_end_to_end_planted_certified(sa):
    from dynamic_sparse_attention_pool_amd.pipelines import VerticalSlashLayer
    N, d, nv, ns = 4096, 128, 100, 16
    base = W.prefill_bf16(54, 1, 4, 2, N, d)
    scale = 1 / math.sqrt(d)
    for bv, bs in [(80, 3), (100, 3), (120, 4)]:    # fixed planting schedule
        inp, _, _ = W.plant_vertical_slash(base, 54, nv, ns, bv, bs)
        sc = [oracle_vs_scores(inp, h, scale) for h in range(4)]
        if all(oracle.certified_row(a, nv, NONE) and oracle.certified_row(s, ns, NONE) for a, s in sc):
            break
    else:
        pytest.fail("planting schedule did not certify")
    layer = VerticalSlashLayer(dev_bf16(inp.q), dev_bf16(inp.k), dev_bf16(inp.v), n_vert=nv, n_slash=ns,
                               out_dtype=torch().float32)
    layer.step()
    torch().cuda.synchronize()
    sel = [[oracle.vs_select(a, s, nv, ns) for a, s in sc]]
    vh, sh = host(layer.vert), host(layer.slash)
    for h in range(4):
        assert np.array_equal(vh[h], sel[0][h][0]) and np.array_equal(sh[h], sel[0][h][1])
    wo, _ = oracle.vs_attention(inp.f32("q"), inp.f32("k"), inp.f32("v"), sel, 64, scale)
    assert_attention_close(host(layer.out), wo, bf16=True, what="planted vs end to end")


def test_vs_full_size_sampled(sa):
    """The 131072-token vertical-slash layer as the benchmark runs it; sampled
    heads and query blocks against the oracle."""
    from dynamic_sparse_attention_pool_amd.pipelines import VerticalSlashLayer
    N, d = 131072, 128
    inp = W.prefill_bf16(W.CONFIG_SEEDS[3], 1, 32, 8, N, d)
    layer = VerticalSlashLayer(dev_bf16(inp.q), dev_bf16(inp.k), dev_bf16(inp.v), n_vert=1000, n_slash=64,
                               out_dtype=torch().float32)
    layer.out.fill_(float("nan"))   # every row of the launch must be written
    layer.step()
    torch().cuda.synchronize()
    assert bool(torch().isfinite(layer.out).all()), "some output rows were not written"
    scale = 1 / math.sqrt(d)
    vh, sh = host(layer.vert), host(layer.slash)
    av_all, as_all = host(layer.a_v), host(layer.a_s)
    for h in [0, 13, 31]:
        wv, ws = oracle_vs_scores(inp, h, scale)
        assert_scores_close(av_all[0, h][None], wv[None], f"vertical h{h}")
        assert_scores_close(as_all[0, h][None], ws[None], f"slash h{h}")
        same = True
        for got, sc, kk in [(vh[h], wv, 1000), (sh[h], ws, 64)]:
            if oracle.certified_row(sc, kk, NONE):
                assert np.array_equal(got, oracle.topk_row(sc, kk, NONE))
            else:
                assert tie_tolerant_valid(got, sc, kk, NONE)
            same = same and np.array_equal(got, oracle.topk_row(sc, kk, NONE))
        cols, offs = oracle.vs_select(wv, ws, 1000, 64)
        sel = [[None] * 32]
        sel[0][h] = (cols, offs)
        blocks = [0, 1, 1000, 2047]
        wo, _ = oracle.vs_attention(inp.f32("q"), inp.f32("k"), inp.f32("v"), sel, 64, scale, heads=[h], blocks=blocks)
        # the layer's own output where its selection is the oracle's; the forward on the oracle's tables always
        outs = [host(layer.out[0, h])] if same else []
        outs.append(fwd_on_oracle_vs(sa, layer.q, layer.k, layer.v, h, cols, offs, 64, 1000))
        for o in outs:
            for i in blocks:
                rows = slice(64 * i, 64 * i + 64)
                assert_attention_close(o[rows], wo[0, h, rows], bf16=True, what=f"h{h} block {i}")


def test_vs_out_of_range_entries(sa):
    """Out-of-range selections and tables never reach memory outside K and V.
    sa_vs_build drops negative offsets and columns outside [0, N) and clips
    counts to the capacities: its tables equal those built from the valid
    entries alone.  The forward clips intervals to the block's visible keys,
    ignores columns outside [0, N) and clips counts: on such tables it equals
    the oracle on the valid keys."""
    t = torch()
    N, d, Hq = 1024, 128, 2
    nb = N // 64
    inp = W.prefill_bf16(63, 1, Hq, 1, N, d)
    r = np.random.default_rng(63)
    valid = [(np.sort(r.choice(N, size=40, replace=False)), np.sort(r.choice(N, size=6, replace=False)))
             for _ in range(Hq)]
    nv, ns = 48, 10
    # the same selections with junk: negative offsets sort first, columns out of range at both ends
    vert = np.zeros((Hq, nv), np.int32)
    slash = np.zeros((Hq, ns), np.int32)
    vc = np.zeros(Hq, np.int32)
    sc = np.zeros(Hq, np.int32)
    for h, (c, o) in enumerate(valid):
        cj = np.concatenate([[-9, -1], c, [N, N + 7, 10 ** 9]])
        oj = np.concatenate([[-50, -3], o])
        vert[h, :cj.size], vc[h] = cj, cj.size + 20     # count above the capacity: clipped to nv
        slash[h, :oj.size], sc[h] = oj, oj.size
    vert[:, 45:] = N + 1
    tables = []
    for vsel in ((vert, vc, slash, sc), None):
        if vsel is None:
            v2 = np.zeros((Hq, nv), np.int32)
            s2 = np.zeros((Hq, ns), np.int32)
            for h, (c, o) in enumerate(valid):
                v2[h, :c.size], s2[h, :o.size] = c, o
            vsel = (v2, np.array([c.size for c, _ in valid], np.int32), s2,
                    np.array([o.size for _, o in valid], np.int32))
        iv = t.empty((1, Hq, nb, ns, 2), dtype=t.int32, device="cuda:0")
        ivc = t.empty((1, Hq, nb), dtype=t.int32, device="cuda:0")
        col = t.empty((1, Hq, nb, nv), dtype=t.int32, device="cuda:0")
        colc = t.empty((1, Hq, nb), dtype=t.int32, device="cuda:0")
        sa.sa_vs_build(dev_i32(vsel[0]), dev_i32(vsel[1]), dev_i32(vsel[2]), dev_i32(vsel[3]), iv.view(Hq, -1),
                       ivc.view(Hq, -1), col.view(Hq, -1), colc.view(Hq, -1), seq=N)
        t.cuda.synchronize()
        tables.append((host(iv), host(ivc), host(col), host(colc)))
    (iv_j, ivc_j, col_j, colc_j), (iv_v, ivc_v, col_v, colc_v) = tables
    assert np.array_equal(ivc_j, ivc_v) and np.array_equal(colc_j, colc_v)
    for h in range(Hq):
        for i in range(nb):
            assert np.array_equal(iv_j[0, h, i, :ivc_j[0, h, i]], iv_v[0, h, i, :ivc_v[0, h, i]])
            assert np.array_equal(col_j[0, h, i, :colc_j[0, h, i]], col_v[0, h, i, :colc_v[0, h, i]])
    # forward on hand-made tables with out-of-range entries
    iv = iv_v.copy()
    ivc = ivc_v.copy()
    col = np.full_like(col_v, -1)
    colc = np.zeros_like(colc_v)
    for h in range(Hq):
        for i in range(nb):
            n = ivc[0, h, i]
            if n < ns:
                iv[0, h, i, n] = (64 * i + 64, 64 * i + 5000)   # beyond the block: clipped to nothing
                ivc[0, h, i] = n + 1
            good = col_v[0, h, i, :colc_v[0, h, i]]
            cj = np.concatenate([[-4], good, [N + 3]])[:nv]
            col[0, h, i, :cj.size] = cj
            colc[0, h, i] = cj.size + (5 if i % 2 else 0)     # some counts above the capacity
    # a negative start is clipped to 0; the row's listed columns are kept
    # disjoint from the widened interval, as the tables' contract requires
    first_end = iv[0, 0, 3, 0, 1]
    iv[0, 0, 3, 0, 0] = -100
    rest = [c for c in col[0, 0, 3, :min(colc[0, 0, 3], nv)] if not (0 <= c < first_end)]
    col[0, 0, 3] = -1
    col[0, 0, 3, :len(rest)] = rest
    colc[0, 0, 3] = len(rest)
    out = t.empty(inp.q.shape, dtype=t.float32, device="cuda:0")
    sa.sa_block_sparse_fwd(dev_bf16(inp.q), dev_bf16(inp.k), dev_bf16(inp.v), out, iv=dev_i32(iv), iv_cnt=dev_i32(ivc),
                           col=dev_i32(col), col_cnt=dev_i32(colc))
    got = host(out)
    t.cuda.synchronize()
    q, k, v = inp.f32("q"), inp.f32("k"), inp.f32("v")
    scale = 1 / math.sqrt(d)
    want = np.zeros_like(got)
    for h in range(Hq):
        for i in range(nb):
            # the stated clipping, applied to the tables as passed
            lim = min(N, 64 * i + 64)
            keys = set()
            for a, b in iv[0, h, i, :min(ivc[0, h, i], ns)]:
                keys.update(range(max(int(a), 0), min(int(b), lim)))
            keys.update(int(c) for c in col[0, h, i, :min(colc[0, h, i], nv)] if 0 <= c < N)
            rows = np.arange(64 * i, 64 * i + 64)
            o, _ = oracle.attend_rows(q[0, h, rows], k[0, 0], v[0, 0], np.array(sorted(keys), np.int64), scale,
                                      row_pos=rows)
            want[0, h, rows] = o
    assert_attention_close(got, want, bf16=True, what="vs forward on out-of-range tables")
