#!/usr/bin/env python3
"""Benchmark of the dynamic sparse attention path on one MI355X.

Step (timed): one block-sparse prefill layer at 131072 tokens — pooled
estimate, top-k with sink + 4 local blocks + ceil(5%) per query-block row, and
the bf16 matrix-core forward — for batch 1, 32 query heads / 8 KV heads,
head_dim 128, synthetic seeded inputs resident in HBM.

value = kept-block FLOP (4*64*64*128 per kept 64x64 block, counted from the
selected tables) / whole-step time.  ms_per_step = ms per layer at 128K.
The same run also reports, as extras, the clustered decode (KV GB/s, us per
token; with a fixed top-64 and with the adaptive softmax-mass budget), the
token-indexer prefill with index reuse, the vertical-slash layer, a layer
mixing A-shape, vertical-slash and block-sparse heads, and the offline k-means
of the decode context; then the roofline of
the dominant kernel (the forward) and the CPU oracle timed on a bounded sample
of the same workload.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extras] [--no-cpu]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
FLOP_PER_BLOCK = 4 * 64 * 64 * 128
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_fwd_bf16_128k.json")
FWD_SOURCES = [os.path.join(ROOT, "dynamic_sparse_attention_pool_amd", "csrc", f) for f in ("k_fwd.hip", "common.h")]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def dev_bf16(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to("cuda:0")


def dev_t(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda:0")


class Timer:
    """HIP events on torch's current stream (the stream libsa launches on)."""

    def __init__(self):
        import torch
        self.torch = torch
        self.marks = {}

    def span(self, name, fn):
        t = self.torch
        a, b = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        self.marks.setdefault(name, []).append((a, b))

    def mean_ms(self, name):
        return float(np.mean([a.elapsed_time(b) for a, b in self.marks[name]]))


def source_hash(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_for(launch_flops_unused=None):
    """HBM bytes per forward launch from the committed rocprofv3 counter
    summary, if it was taken on the current kernel source; else None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        t = json.load(f)
    if t.get("kernel_source_sha256_16") != source_hash(FWD_SOURCES):
        return None
    return t.get("hbm_bytes_per_launch")


# ---------------------------------------------------------------- main workload
def prefill_layer(N, ratio, steps, warmup, seed):
    import torch
    import workloads as W
    from dynamic_sparse_attention_pool_amd.pipelines import BlockSparseLayer
    t0 = time.time()
    inp = W.prefill_bf16(seed, 1, 32, 8, N, 128)
    q, k, v = dev_bf16(inp.q), dev_bf16(inp.k), dev_bf16(inp.v)
    log(f"[bench] inputs N={N} generated+uploaded in {time.time() - t0:.1f}s")
    layer = BlockSparseLayer(q, k, v, n_sink=1, n_local=4, ratio=ratio, out_dtype=torch.bfloat16)
    for _ in range(warmup):
        layer.step()
    torch.cuda.synchronize()
    tm = Timer()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        tm.span("estimate", layer.estimate)
        tm.span("select", layer.select)
        tm.span("forward", layer.forward)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    kept = int(layer.cnt.sum().item())
    assert int(layer.err.item()) == 0, "non-finite block score"
    res = dict(N=N, ms_per_step=ms, kept_blocks=kept, flop=kept * FLOP_PER_BLOCK,
               ms_estimate=tm.mean_ms("estimate"), ms_select=tm.mean_ms("select"),
               ms_forward=tm.mean_ms("forward"), inputs=inp)
    del layer, q, k, v
    torch.cuda.empty_cache()
    return res


# ---------------------------------------------------------------- extras
def decode_extra(steps, warmup, mass=None):
    """Clustered decode step; with ``mass`` the adaptive budget (fewest
    clusters holding that share of the centroid-score softmax, 1..64)."""
    import torch
    import workloads as W
    from dynamic_sparse_attention_pool_amd.pipelines import ClusterDecode
    T, Hq, Hkv, N, d, C, ksel = 8, 32, 8, 65536, 128, 256, 64
    copies = []
    for c in range(4):  # rotate over 4 contexts so no step finds the last one in the 256 MB MALL
        inp = W.decode_clustered(W.CONFIG_SEEDS[4] + 100 * c, T, Hq, Hkv, N, d, C)
        copies.append(ClusterDecode(dev_bf16(inp.q), dev_bf16(inp.k), dev_bf16(inp.v), dev_t(inp.labels),
                                    dev_t(inp.centroids), n_sel=ksel, mass=mass, k_min=1, fused=True))
    torch.cuda.synchronize()
    for i in range(max(warmup, 4)):
        copies[i % 4].step()
    torch.cuda.synchronize()
    # a decode step is a handful of short launches: replay each as one HIP graph so
    # the host's launch overhead is not what gets timed
    # (the fused estimate also selects: there is no separate selection launch to time)
    graphs = []
    for dc in copies:
        parts = []
        for fn in (dc.estimate, dc.forward, dc.step):
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr):
                fn()
            parts.append(gr)
        graphs.append(parts)
    # the same scores and selection as two calls, for comparison (one context)
    two = copies[0]
    two.fused = False
    two_graphs = []
    for fn in (two.estimate, two.select):
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            fn()
        two_graphs.append(gr)
    two.fused = True
    torch.cuda.synchronize()
    tm = Timer()
    for i in range(steps):
        tm.span("estimate_two_call", two_graphs[0].replay)
        tm.span("select_two_call", two_graphs[1].replay)
    for i in range(steps):
        ge, gf, _ = graphs[i % 4]
        tm.span("estimate", ge.replay)
        tm.span("forward", gf.replay)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(steps):
        graphs[i % 4][2].replay()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    # algorithmic bytes: K+V rows of the union of selected clusters per KV head
    kv_bytes = 0
    for dc in copies:
        sel = dc.sel.cpu().numpy()
        ptr = dc.ptr.cpu().numpy().astype(np.int64)
        for g in range(Hkv):
            used = np.unique(sel[:, g * (Hq // Hkv):(g + 1) * (Hq // Hkv), :])
            used = used[used >= 0]  # -1 pads rows that keep fewer clusters
            kv_bytes += int((ptr[g, used + 1] - ptr[g, used]).sum()) * 2 * d * 2
    kv_bytes //= len(copies)
    small = T * Hq * d * 2 + Hkv * C * d * 4 + T * Hq * d * 4
    step_bytes = kv_bytes + small
    fwd_ms = tm.mean_ms("forward")
    mean_sel = float(np.mean([dc.sel_cnt.float().mean().item() for dc in copies]))
    rule = ("top 64 of 256 clusters" if mass is None else
            f"fewest clusters holding {mass:g} of the centroid-score softmax, 1..64 of 256") + \
        " (scores and selection in one call)"
    return {"workload": f"clustered decode: 8 queries x 32/8 heads, d128, 65536-key context, {rule}; "
                        "each step replayed as a HIP graph, rotating 4 contexts",
            "mean_clusters": mean_sel,
            "us_per_step": ms * 1e3, "us_per_token": ms * 1e3 / T,
            "kv_bytes_per_step": kv_bytes, "GB_per_s_step": step_bytes / (ms * 1e-3) / 1e9,
            "us_gather": fwd_ms * 1e3, "GB_per_s_gather": kv_bytes / (fwd_ms * 1e-3) / 1e9,
            "frac_hbm_gather": kv_bytes / (fwd_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "us_estimate_and_select": tm.mean_ms("estimate") * 1e3,
            "us_estimate_two_call": tm.mean_ms("estimate_two_call") * 1e3,
            "us_select_two_call": tm.mean_ms("select_two_call") * 1e3}


def indexer_extra(steps, warmup):
    import torch
    import workloads as W
    from dynamic_sparse_attention_pool_amd.pipelines import IndexerPrefill
    seed = W.CONFIG_SEEDS[5]
    T, N, Hi, di, k_sel = 4096, 131072, 64, 64, 2048
    ind = W.indexer_random(seed, T, Hi, di, N)
    layers = []
    for l in range(4):
        L = W.mqa_layer(seed, l, T, 16, 1, N, 128)
        layers.append((dev_bf16(L.q), dev_bf16(L.k), dev_bf16(L.v)))
    ip = IndexerPrefill(dev_bf16(ind.qi), dev_bf16(ind.ki), dev_t(ind.w), ind.pos0, layers, k_sel=k_sel,
                        out_dtype=torch.bfloat16)
    for _ in range(warmup):
        ip.step(reuse=True)
    torch.cuda.synchronize()
    tm = Timer()
    for _ in range(steps):
        tm.span("total_reuse", lambda: ip.step(reuse=True))
        tm.span("total_noreuse", lambda: ip.step(reuse=False))
        tm.span("indexer", lambda: __import__("dynamic_sparse_attention_pool_amd").sa_estimate(
            __import__("dynamic_sparse_attention_pool_amd").INDEXER, ip.qi, ip.ki, ip.scores, weights=ip.w,
            q_pos0=ip.pos0))
        tm.span("select", lambda: __import__("dynamic_sparse_attention_pool_amd").sa_select_topk(
            ip.scores, ip.idx, ip.cnt, k=k_sel, causal=True, causal_period=T, causal_offset=ip.pos0))
        tm.span("attend", lambda: ip.attend(1))
    fu = IndexerPrefill(ip.qi, ip.ki, ip.w, ind.pos0, layers, k_sel=k_sel, out_dtype=torch.bfloat16, fused=True)
    fu.index()
    torch.cuda.synchronize()
    for _ in range(steps):
        tm.span("index_fused", fu.index)
        tm.span("total_reuse_fused", lambda: fu.step(reuse=True))
    torch.cuda.synchronize()
    same = bool(torch.equal(fu.idx, ip.idx)) and int(fu.err.item()) == 0
    pairs = sum(ind.pos0 + t + 1 for t in range(T))
    idx_ms = tm.mean_ms("indexer")
    return {"workload": "token top-2048 prefill chunk: 4096 queries at the end of 131072, 64x64 indexer, "
                        "MQA 16/1 d128, 4 layers, layer 1 full / 2-4 shared",
            "ms_4layers_with_reuse": tm.mean_ms("total_reuse"), "ms_4layers_without_reuse": tm.mean_ms("total_noreuse"),
            "ms_indexer": idx_ms, "indexer_TFLOP_per_s": pairs * 8192 / (idx_ms * 1e-3) / 1e12,
            "ms_select": tm.mean_ms("select"), "ms_attend_layer": tm.mean_ms("attend"),
            "ms_index_fused": tm.mean_ms("index_fused"), "ms_4layers_with_reuse_fused": tm.mean_ms("total_reuse_fused"),
            "fused_index_equals_two_call": same}


def vs_extra(steps, warmup, inp):
    import torch
    from dynamic_sparse_attention_pool_amd.pipelines import VerticalSlashLayer
    q, k, v = dev_bf16(inp.q), dev_bf16(inp.k), dev_bf16(inp.v)
    layer = VerticalSlashLayer(q, k, v, n_vert=1000, n_slash=64, out_dtype=torch.bfloat16)
    for _ in range(warmup):
        layer.step()
    torch.cuda.synchronize()
    tm = Timer()
    for _ in range(steps):
        tm.span("estimate", layer.estimate)
        tm.span("select", layer.select)
        tm.span("forward", layer.forward)
    torch.cuda.synchronize()
    flop = vs_table_keys(layer) * 4 * 64 * 128
    fwd = tm.mean_ms("forward")
    return {"workload": "vertical-slash layer at 131072: last-64-query estimate, top 1000 columns + top 64 offsets",
            "ms_layer": tm.mean_ms("estimate") + tm.mean_ms("select") + fwd, "ms_estimate": tm.mean_ms("estimate"),
            "ms_select_build": tm.mean_ms("select"), "ms_forward": fwd, "kept_key_flop": flop,
            "forward_TFLOP_per_s": flop / (fwd * 1e-3) / 1e12}


def vs_table_keys(layer):
    """Kept keys over all query blocks of a vertical-slash layer, counted from
    its built tables (diagonal tiles whole)."""
    ivc = layer.iv.cpu().numpy()
    ivn = layer.iv_cnt.cpu().numpy()
    keys = int(layer.col_cnt.cpu().numpy().astype(np.int64).sum())
    B, H, nb = ivn.shape
    for b in range(B):
        for h in range(H):
            for i in range(nb):
                n = ivn[b, h, i]
                keys += int((ivc[b, h, i, :n, 1] - ivc[b, h, i, :n, 0]).sum())
    return keys


def mixed_extra(steps, warmup, inp):
    """The 128K layer with a per-head pattern assignment: in every group of 4
    query heads sharing a KV head, one A-shape head (sink + 4 local blocks),
    one vertical-slash head (1000 columns, 64 offsets) and two block-sparse
    heads (sink + 4 local + ceil(5%))."""
    import torch
    from dynamic_sparse_attention_pool_amd.pipelines import MixedPatternLayer
    q, k, v = dev_bf16(inp.q), dev_bf16(inp.k), dev_bf16(inp.v)
    Hq, N = q.shape[1], q.shape[2]
    pats = [("A", "VS", "BS", "BS")[h % 4] for h in range(Hq)]
    layer = MixedPatternLayer(q, k, v, pats, a_shape=(1, 4), block=dict(n_sink=1, n_local=4, ratio=(5, 100)),
                              vslash=(1000, 64), out_dtype=torch.bfloat16)
    for _ in range(warmup):
        layer.step()
    torch.cuda.synchronize()
    tm = Timer()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        tm.span("estimate", layer.estimate)
        tm.span("select", layer.select)
        tm.span("forward", layer.forward)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    parts = {type(p).__name__: p for p in layer.parts}
    nb = N // 64
    a_blocks = sum(len(set(range(min(1, i + 1))) | set(range(max(0, i - 3), i + 1))) for i in range(nb))
    flop = (int(parts["BlockSparseLayer"].cnt.sum().item()) + a_blocks * len(layer.groups["A"])) * FLOP_PER_BLOCK
    flop += vs_table_keys(parts["VerticalSlashLayer"]) * 4 * 64 * 128
    fwd = tm.mean_ms("forward")
    return {"workload": "mixed-pattern layer at 131072, GQA 32/8, d128: per KV head 1 A-shape (sink + 4 local), "
                        "1 vertical-slash (1000 cols, 64 offsets), 2 block-sparse (sink + 4 local + ceil(5%)) heads",
            "ms_layer": ms, "ms_estimate": tm.mean_ms("estimate"), "ms_select": tm.mean_ms("select"),
            "ms_forward": fwd, "kept_flop": flop, "TFLOP_per_s_layer": flop / (ms * 1e-3) / 1e12,
            "forward_TFLOP_per_s": flop / (fwd * 1e-3) / 1e12}


def fused_extra(steps, inp):
    """Block estimate + top-k at 131072 tokens: the fused call (no score
    matrix) against pooled scores followed by the separate selection."""
    import torch
    from dynamic_sparse_attention_pool_amd.pipelines import BlockSparseLayer
    q, k, v = dev_bf16(inp.q), dev_bf16(inp.k), dev_bf16(inp.v)
    res = {"workload": "block estimate + top-k at 131072, GQA 32/8, d128, sink + 4 local + ceil(5%)"}
    for name, fused in (("separate", False), ("fused", True)):
        layer = BlockSparseLayer(q, k, v, n_sink=1, n_local=4, ratio=(5, 100), fused=fused)
        layer.estimate()
        layer.select()
        torch.cuda.synchronize()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        for _ in range(steps):
            layer.estimate()
            layer.select()
        end.record()
        torch.cuda.synchronize()
        res[f"ms_{name}"] = start.elapsed_time(end) / steps
        if fused:
            # the two paths sum the pooled dot products in different orders, so a
            # row whose cut falls between nearly equal scores may keep another block
            same = (layer.cnt == ref_cnt) & (layer.idx == ref_idx).all(dim=-1)
            res["rows_identical_frac"] = float(same.float().mean().item())
        else:
            ref_idx, ref_cnt = layer.idx.clone(), layer.cnt.clone()
        del layer
        torch.cuda.empty_cache()
    return res


def kmeans_extra(steps, iters=10):
    """Offline clustering of the decode context: 8 KV heads x 65536 keys, d128,
    256 clusters, Lloyd iterations from sampled keys."""
    import torch
    import workloads as W
    from dynamic_sparse_attention_pool_amd import sa_kmeans
    Hkv, N, d, C = 8, 65536, 128, 256
    inp = W.decode_clustered(W.CONFIG_SEEDS[4], 1, Hkv, Hkv, N, d, C)
    k = dev_bf16(inp.k)
    init = dev_t(W.kmeans_init(W.CONFIG_SEEDS[4], inp.k, C))
    cent = init.clone()
    labels = torch.empty((Hkv, N), dtype=torch.int32, device=k.device)
    ptr = torch.empty((Hkv, C + 1), dtype=torch.int32, device=k.device)
    perm = torch.empty((Hkv, N), dtype=torch.int32, device=k.device)
    ws = sa_kmeans(k, cent, labels, iters=1, cluster_ptr=ptr, perm=perm)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    total = 0.0
    for _ in range(steps):
        cent.copy_(init)
        start.record()
        sa_kmeans(k, cent, labels, iters=iters, cluster_ptr=ptr, perm=perm, workspace=ws)
        end.record()
        torch.cuda.synchronize()
        total += start.elapsed_time(end)
    ms = total / steps
    flop = 2.0 * Hkv * N * C * d * iters   # distance dot products of the assignments
    # bf16 keys: each dot product runs as three bf16 products (centroid split
    # hi + lo + lo2) on the matrix cores
    tflops = flop / (ms * 1e-3) / 1e12
    return {"workload": f"k-means of the decode context: 8 KV heads x 65536 keys, d128, 256 clusters, {iters} "
                        "Lloyd iterations from sampled keys",
            "ms_total": ms, "ms_per_iteration": ms / iters,
            "distance_TFLOP_per_s_over_whole_iterations": tflops,
            "frac_bf16_peak_three_products_over_whole_iterations": 3 * tflops / PEAK_BF16_TFLOPS}


# ---------------------------------------------------------------- CPU oracle baseline
def cpu_baseline(inp, ratio, budget_s=20.0):
    """The fp64 oracle on head 0 of the same layer: pooled estimate of head 0
    and its KV head, selection of every query-block row, attention for a
    strided subset of query blocks (as many as fit the time budget)."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        cores = len(os.sched_getaffinity(0))
    _, Hq, N, d = inp.q.shape
    nb = N // 64
    scale = 1 / math.sqrt(d)
    import workloads as W
    q0 = W.bf16_to_f32(inp.q[0:1, 0:1])
    k0 = W.bf16_to_f32(inp.k[0:1, 0:1])
    v0 = W.bf16_to_f32(inp.v[0:1, 0:1])
    t0 = time.perf_counter()
    S = oracle.block_scores(q0, k0, 64, scale)
    kept = oracle.block_select(S, n_sink=1, n_local=4, ratio=ratio)
    t_sel = time.perf_counter() - t0
    blocks, flop = [], 0
    t1 = time.perf_counter()
    stride = 1
    # longest rows first, strided, until the budget is used
    order = list(range(nb - 1, -1, -1))
    done = []
    for i in order[::stride]:
        oracle.block_sparse_attention(q0, k0, v0, kept, 64, scale, heads=[0], blocks=[i])
        done.append(i)
        flop += len(kept[0][0][i]) * FLOP_PER_BLOCK
        if time.perf_counter() - t1 > budget_s:
            break
    t_att = time.perf_counter() - t1
    # scale the estimate/select share to the sampled rows
    frac_rows = len(done) / nb
    t_total = t_att + t_sel * frac_rows
    return {"value": flop / t_total / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"head 0 of the 128K layer: pooled estimate + selection (time pro-rated to the sampled rows) "
                      f"and fp64 attention for the {len(done)} longest query-block rows of {nb}; "
                      f"{flop / 1e9:.1f} GFLOP of kept blocks in {t_total:.1f}s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-extras", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--only", default="", help="comma list of extras to run: decode,decode_adaptive,indexer,vs,mixed,kmeans,fused")
    ap.add_argument("--pmc-copy", action="store_true",
                    help="first run a plain 1 GiB device copy, the known-size reference for HBM counters")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (each GPU would run "
              "the same kernels on its own share of heads); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    import dynamic_sparse_attention_pool_amd as sa
    sa.load()
    torch.cuda.init()

    if args.pmc_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log("[bench] reference copy: 1073741824 bytes read, 1073741824 bytes written")
        del src, dst
    main = prefill_layer(131072, (5, 100), args.steps, args.warmup, seed=3)
    ms = main["ms_per_step"]
    value = main["flop"] / (ms * 1e-3) / 1e12
    fwd_tflops = main["flop"] / (main["ms_forward"] * 1e-3) / 1e12
    traffic = traffic_for()
    line = {
        "metric": "sparse-attn prefill TFLOP/s (kept blocks) & ms at 128K; decode KV GB/s",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "block-sparse prefill layer, 131072 tokens, batch 1, GQA 32/8, head_dim 128, "
                               "1% keys +3u / queries +1u, sink + 4 local + ceil(5%) blocks of 64",
                   "seq_len": 131072, "heads_q": 32, "heads_kv": 8, "head_dim": 128, "block": 64,
                   "kept_blocks": main["kept_blocks"], "parallelism": "single GPU"},
        "breakdown_ms": {"estimate": round(main["ms_estimate"], 4), "select": round(main["ms_select"], 4),
                         "forward": round(main["ms_forward"], 4)},
        "roofline": {"bound": "mfma", "kernel": "k_fwd_bf16<128,block>", "achieved": round(fwd_tflops, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(fwd_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic},
    }
    if traffic is not None:
        # the same launch seen from DRAM: measured HBM-side bytes over its duration
        tbps = traffic / (main["ms_forward"] * 1e-3) / 1e12
        line["roofline"]["traffic_TB_per_s"] = round(tbps, 3)
        line["roofline"]["traffic_frac_hbm"] = round(tbps * 1e3 / PEAK_HBM_GBS, 4)
    extras = {}
    only = set(x for x in args.only.split(",") if x)
    if not args.no_extras:
        for name, fn in [("decode", lambda: decode_extra(max(args.steps, 20), args.warmup)),
                         ("decode_adaptive", lambda: decode_extra(max(args.steps, 20), args.warmup, mass=0.5)),
                         ("indexer", lambda: indexer_extra(max(2, args.steps // 3), 1)),
                         ("vs", lambda: vs_extra(max(2, args.steps // 3), 1, main["inputs"])),
                         ("mixed", lambda: mixed_extra(max(2, args.steps // 3), 1, main["inputs"])),
                         ("kmeans", lambda: kmeans_extra(3)),
                         ("fused", lambda: fused_extra(max(5, args.steps), main["inputs"]))]:
            if only and name not in only:
                continue
            try:
                log(f"[bench] extra {name}")
                extras[name] = fn()
            except Exception as e:  # noqa: BLE001  (an extra that is not available is reported, not fatal)
                extras[name] = {"error": f"{type(e).__name__}: {e}"}
            torch.cuda.empty_cache()
    if extras:
        line["extras"] = extras
    if not args.no_cpu:
        log("[bench] cpu oracle baseline")
        line["cpu_baseline"] = cpu_baseline(main["inputs"], (5, 100))
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
