"""GPU parity of the fused block estimate + top-k (sa_estimate_topk), which
never writes the score matrix, against the oracle's pooled scores followed by
its selection."""
import math

import numpy as np
import pytest

import oracle
import workloads as W
from gpu_helpers import dev_bf16, dev_f32, host, tie_tolerant_valid, torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sa():
    import dynamic_sparse_attention_pool_amd as m
    m.load()
    return m


def kmax_of(nb, n_sink, n_local, k=None, ratio=None):
    from dynamic_sparse_attention_pool_amd.pipelines import max_kept_blocks
    return max_kept_blocks(nb, n_sink, n_local, k, ratio)


def run_fused(sa, q, k, n_sink, n_local, k_fixed=None, ratio=None, scale=None, heads=None, extra=0):
    t = torch()
    B, Hq, N, d = q.shape
    nb = N // 64
    nh = Hq if heads is None else len(heads)
    kmax = kmax_of(nb, n_sink, n_local, k_fixed, ratio) + extra
    idx = t.full((B, nh, nb, kmax), 77, dtype=t.int32, device=q.device)
    cnt = t.full((B, nh, nb), -3, dtype=t.int32, device=q.device)
    err = t.zeros(1, dtype=t.int32, device=q.device)
    budget = dict(ratio=ratio) if ratio is not None else dict(k_fixed=k_fixed)
    sa.sa_estimate_topk(q, k, idx, cnt, n_sink=n_sink, n_local=n_local, scale=scale, heads=heads, err_flag=err,
                        **budget)
    t.cuda.synchronize()
    return host(idx), host(cnt), int(host(err)[0])


def check_exact(idx, cnt, kept):
    B, H, nb, kmax = idx.shape
    for b in range(B):
        for h in range(H):
            for i in range(nb):
                want = kept[b][h][i]
                assert cnt[b, h, i] == len(want), (b, h, i)
                assert np.array_equal(idx[b, h, i, :cnt[b, h, i]], want), (b, h, i)
                assert np.all(idx[b, h, i, cnt[b, h, i]:] == -1), (b, h, i)


EXACT_CASES = [
    # (B, Hq, Hkv, N, d, dtype, n_sink, n_local, k, ratio)
    (1, 2, 1, 1024, 128, "bf16", 1, 1, 2, None),
    (2, 4, 2, 64 * 37, 128, "bf16", 1, 4, None, (10, 100)),
    (1, 4, 4, 64 * 50, 64, "bf16", 2, 3, None, (30, 100)),
    (1, 2, 2, 64 * 23, 64, "f32", 0, 0, 5, None),
    (1, 2, 1, 64 * 40, 128, "f32", 3, 0, 1000, None),       # budget above the pool: everything kept
    (1, 2, 1, 64 * 19, 128, "bf16", 0, 2, 0, None),          # forced only
]


@pytest.mark.parametrize("case", range(len(EXACT_CASES)))
def test_fused_topk_bit_exact_integer_inputs(sa, case):
    """Integer-valued bf16 inputs in [-2, 2] with scale 1: pooled means and
    their products are exact in fp32, so the selection must equal the oracle's
    on every row, ties included (integer scores tie often)."""
    B, Hq, Hkv, N, d, dt, ns, nl, kf, ratio = EXACT_CASES[case]
    print(f"fused exact case {case}", flush=True)
    qb = W.integer_bf16(81 + case, (B, Hq, N, d), -2, 2, 0)
    kb = W.integer_bf16(81 + case, (B, Hkv, N, d), -2, 2, 1)
    qf, kf32 = W.bf16_to_f32(qb), W.bf16_to_f32(kb)
    q, k = (dev_bf16(qb), dev_bf16(kb)) if dt == "bf16" else (dev_f32(qf), dev_f32(kf32))
    idx, cnt, err = run_fused(sa, q, k, ns, nl, k_fixed=kf, ratio=ratio, scale=1.0, extra=3)
    assert err == 0
    S = oracle.block_scores(qf, kf32, 64, 1.0)
    kept = oracle.block_select(S, n_sink=ns, n_local=nl, k=kf, ratio=ratio)
    check_exact(idx, cnt, kept)


def test_fused_topk_head_list_and_nan_flag(sa):
    B, Hq, Hkv, N, d = 2, 8, 2, 64 * 33, 128
    qb = W.integer_bf16(90, (B, Hq, N, d), -2, 2, 0)
    kb = W.integer_bf16(90, (B, Hkv, N, d), -2, 2, 1)
    heads = [6, 1, 3]
    idx, cnt, err = run_fused(sa, dev_bf16(qb), dev_bf16(kb), 1, 4, ratio=(20, 100), scale=1.0, heads=heads)
    assert err == 0
    S = oracle.block_scores(W.bf16_to_f32(qb), W.bf16_to_f32(kb), 64, 1.0)
    kept = oracle.block_select(S, n_sink=1, n_local=4, ratio=(20, 100))
    check_exact(idx, cnt, [[kept[b][h] for h in heads] for b in range(B)])
    qn = W.bf16_to_f32(qb).copy()
    qn[1, 6, 64 * 20 + 3, 7] = np.nan
    _, _, err = run_fused(sa, dev_f32(qn), dev_f32(W.bf16_to_f32(kb)), 1, 4, ratio=(20, 100), scale=1.0)
    assert err == 1


@pytest.mark.parametrize("N,ratio,seed", [(32768, (10, 100), W.CONFIG_SEEDS[2]), (131072, (5, 100), W.CONFIG_SEEDS[3])])
def test_fused_topk_full_size_sampled(sa, N, ratio, seed):
    """The benchmark's layers (GQA 32/8, d128, 1% shifted keys): sampled heads
    and rows against the oracle's pooled scores; certified rows exactly,
    others tie-tolerant valid; the kept-block total is data independent."""
    print(f"fused full size N={N}", flush=True)
    inp = W.prefill_bf16(seed, 1, 32, 8, N, 128)
    q, k = dev_bf16(inp.q), dev_bf16(inp.k)
    idx, cnt, err = run_fused(sa, q, k, 1, 4, ratio=ratio)
    assert err == 0
    nb = N // 64
    per_row = []
    for i in range(nb):
        f = oracle.forced_set(i + 1, 1, 4)
        per_row.append(f.shape[0] + oracle.budget(i + 1, f.shape[0], None, ratio))
    assert int(cnt.sum()) == 32 * sum(per_row)
    scale = 1 / math.sqrt(128)
    rng = np.random.default_rng(5)
    certified = total = 0
    for h in [0, 9, 31]:
        g = h * 8 // 32
        qbar = oracle.mean_pool(inp.f32("q")[0, h], 64)
        kbar = oracle.mean_pool(inp.f32("k")[0, g], 64)
        for i in np.unique(np.concatenate([[0, 1, 5, nb - 1], rng.integers(0, nb, 20)])):
            s = (kbar[:i + 1] @ qbar[i]) * scale
            f = oracle.forced_set(i + 1, 1, 4)
            kr = oracle.budget(i + 1, f.shape[0], None, ratio)
            got = idx[0, h, i, :cnt[0, h, i]]
            total += 1
            if oracle.certified_row(s, kr, f):
                certified += 1
                assert np.array_equal(got, oracle.topk_row(s, kr, f)), (h, i)
            else:
                assert tie_tolerant_valid(got, s, kr, f), (h, i)
    print(f"certified {certified}/{total}", flush=True)
    assert certified >= total // 2
