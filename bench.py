#!/usr/bin/env python3
"""Benchmark of the dynamic sparse attention path on one MI355X.

Step (the headline, timed as the contract asks): one block-sparse prefill
layer at 131072 tokens — pooled estimate, top-k with sink + 4 local blocks +
ceil(5%) per query-block row, and the bf16 matrix-core forward — for batch 1,
32 query heads / 8 KV heads, head_dim 128, synthetic seeded inputs resident in
HBM.  value = kept-block FLOP (4*64*64*128 per kept 64x64 block, counted from
the selected tables) / whole-step time over exactly K back-to-back steps;
ms_per_step = ms per layer at 128K.

Beside it, every workload is measured with one method: HIP events per rep on
the stream the library launches on, a 512 MB write before each rep (outside
the timed span) so no rep starts from the previous one's caches, then the
median and minimum of at least 20 reps:
  1. block-sparse parity layer, 1024 tokens fp32, sink + diagonal + top-2 (us)
  2. 32K GQA layer, sink + 4 local + ceil(10%) (ms per layer, forward TFLOP/s)
  3. the 128K layer (headline) and its vertical-slash variant
  4. clustered decode over a 65536-key context (KV GB/s, us per token)
  5. the token-indexer prefill chunk with index reuse over 4 layers
Each kernel's rate is reported against the spec peak and against the peak the
chip sustains in the same run (a matrix-core loop and a streaming read from
libsa's probes), with the shader clock sampled (amdsmi) inside the timed reps.  The CPU oracle is
timed on a bounded sample of every workload.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--reps R] [--no-extras] [--no-cpu]
"""
from __future__ import annotations

import argparse
import ctypes as C
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak (spec)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E (spec)
FLOP_PER_BLOCK_128 = 4 * 64 * 64 * 128
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_fwd_bf16_128k.json")
FWD_SOURCES = [os.path.join(ROOT, "dynamic_sparse_attention_pool_amd", "csrc", f) for f in ("k_fwd.hip", "common.h")]
EVICT_BYTES = 512 << 20


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def dev_bf16(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to("cuda:0")


def dev_t(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda:0")


def stats(ms_list):
    a = np.asarray(ms_list, np.float64)
    return {"median": float(np.median(a)), "min": float(a.min()), "mean": float(a.mean()), "n": int(a.size)}


class Reps:
    """Per-rep HIP events on torch's current stream (the stream libsa launches
    on), with a 512 MB write before every rep outside the timed spans."""

    def __init__(self):
        import torch
        self.torch = torch
        self.evict = torch.empty(EVICT_BYTES, dtype=torch.uint8, device="cuda:0")
        self.marks = {}

    def flush(self):
        self.evict.fill_(1)

    def span(self, name, fn):
        t = self.torch
        a, b = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        self.marks.setdefault(name, []).append((a, b))

    def run(self, reps, parts, clock=None):
        """parts: list of (name, fn); one rep = flush, then each part timed.
        clock: name of the window the shader clock is sampled in."""
        for _ in range(reps):
            self.flush()
            for name, fn in parts:
                self.span(name, fn)
            clock_sample(clock)
        self.torch.cuda.synchronize()

    def ms(self, name):
        return [a.elapsed_time(b) for a, b in self.marks[name]]

    def stat(self, name):
        return stats(self.ms(name))

    def total(self, names):
        """Per-rep sum of several spans."""
        per = np.sum([self.ms(n) for n in names], axis=0)
        return stats(per)


class ClockWindows:
    """Shader clock read in-process (amdsmi's GPU metrics table, median over
    the XCDs) from the launching thread right after each timed rep is
    enqueued, while the GPU is still running it."""

    def __init__(self):
        self.samples, self.handle, self.api, self.errors, self.raw = {}, None, None, [], None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            self.handle = amdsmi.amdsmi_get_processor_handles()[0]
            self.api = amdsmi
            m = amdsmi.amdsmi_get_gpu_metrics_info(self.handle)
            self.raw = {k: m.get(k) for k in ("current_gfxclk", "average_gfxclk_frequency", "current_gfxclks")}
            self._read()
        except Exception:  # noqa: BLE001  (the clock is context, not a result)
            self.handle = None

    def _read(self):
        m = self.api.amdsmi_get_gpu_metrics_info(self.handle)
        per = [x for x in (m.get("current_gfxclks") or []) if isinstance(x, (int, float)) and 0 < x < 10000]
        if per:
            return float(np.median(per))
        for key in ("current_gfxclk", "average_gfxclk_frequency"):
            x = m.get(key)
            if isinstance(x, (int, float)) and 0 < x < 10000:
                return float(x)
        raise RuntimeError("no gfx clock in the metrics table")

    def sample_now(self, name):
        if self.handle is not None:
            try:
                self.samples.setdefault(name, []).append(self._read())
            except Exception as e:  # noqa: BLE001
                if len(self.errors) < 4:
                    self.errors.append(f"{name}: {type(e).__name__}: {e}"[:200])

    def summary(self):
        if not self.samples and not self.errors:
            return None
        out = {"errors": self.errors} if self.errors else {}
        out["metrics_at_start"] = str(self.raw)[:300]
        out["source"] = ("amdsmi GPU metrics, current gfx clock (median over XCDs), one sample right after each "
                         "timed rep is enqueued")
        for k, v in self.samples.items():
            a = np.asarray(v)
            out[k] = {"mhz_median": float(np.median(a)), "mhz_min": float(a.min()), "mhz_max": float(a.max()),
                      "n": int(a.size)}
        return out


CLOCK = None


def clock_sample(name):
    if CLOCK is not None and name:
        CLOCK.sample_now(name)


def source_hash(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_for():
    """L2-miss bytes per forward launch from the committed rocprofv3 counter
    summary, if it was taken on the current kernel source; else None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        t = json.load(f)
    if t.get("kernel_source_sha256_16") != source_hash(FWD_SOURCES):
        return None
    return t.get("hbm_bytes_per_launch")


# ---------------------------------------------------------------- achievable peaks
def measured_peaks():
    """The bf16 matrix-core loop and a 2 GiB streaming read (well beyond the
    256 MB Infinity Cache), each timed with HIP events (best of 3)."""
    import torch
    import dynamic_sparse_attention_pool_amd as sa
    lib = sa.load()
    st = torch.cuda.current_stream().cuda_stream
    sink = torch.zeros(1 << 16, dtype=torch.float32, device="cuda:0")
    res = {}
    best = 0.0
    for _ in range(3):
        fl = C.c_double(0)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        assert lib.sa_peak_mfma_bf16(C.c_void_p(sink.data_ptr()), 2000, 8, C.byref(fl), st) == 0
        b.record()
        torch.cuda.synchronize()
        best = max(best, fl.value / (a.elapsed_time(b) * 1e-3) / 1e12)
    res["mfma_bf16_TFLOP_per_s"] = best
    buf = torch.ones(2 << 30, dtype=torch.uint8, device="cuda:0")
    best = 0.0
    for _ in range(3):
        nb = C.c_double(0)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        assert lib.sa_peak_read(C.c_void_p(buf.data_ptr()), buf.numel(), 2, C.c_void_p(sink.data_ptr()),
                                C.byref(nb), st) == 0
        b.record()
        torch.cuda.synchronize()
        best = max(best, nb.value / (a.elapsed_time(b) * 1e-3) / 1e9)
    res["hbm_read_GB_per_s"] = best
    del buf
    torch.cuda.empty_cache()
    return res


def frac_pair(rate, spec, measured):
    return {"frac_spec": rate / spec, "frac_measured": (rate / measured) if measured else None}


# ---------------------------------------------------------------- headline: the 128K layer
def prefill_headline(steps, warmup, reps, seed):
    import torch
    import workloads as W
    from dynamic_sparse_attention_pool_amd.pipelines import BlockSparseLayer
    N = 131072
    t0 = time.time()
    inp = W.prefill_bf16(seed, 1, 32, 8, N, 128)
    q, k, v = dev_bf16(inp.q), dev_bf16(inp.k), dev_bf16(inp.v)
    log(f"[bench] 128K inputs generated+uploaded in {time.time() - t0:.1f}s")
    layer = BlockSparseLayer(q, k, v, n_sink=1, n_local=4, ratio=(5, 100), out_dtype=torch.bfloat16)
    for _ in range(warmup):
        layer.step()
    torch.cuda.synchronize()
    # the contract's loop: exactly `steps` back-to-back steps between two synchronizations
    R = Reps()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(steps):
        R.span("c_estimate", layer.estimate)
        R.span("c_select", layer.select)
        R.span("c_forward", layer.forward)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    # the measurement method: reps with a cache flush before each
    R.run(reps, [("estimate", layer.estimate), ("select", layer.select), ("forward", layer.forward)], clock="prefill_128k")
    kept = int(layer.cnt.sum().item())
    assert int(layer.err.item()) == 0, "non-finite block score"
    res = dict(N=N, ms_per_step=ms, kept_blocks=kept, flop=kept * FLOP_PER_BLOCK_128,
               contract_ms={n: float(np.mean(R.ms("c_" + n))) for n in ("estimate", "select", "forward")},
               layer=R.total(["estimate", "select", "forward"]),
               parts={n: R.stat(n) for n in ("estimate", "select", "forward")}, inputs=inp)
    del layer, q, k, v, R
    torch.cuda.empty_cache()
    return res


# ---------------------------------------------------------------- configs 1 and 2
def config1(reps):
    """1024 tokens, 1 head, d64 fp32, sink + diagonal + top-2 other blocks."""
    import torch
    import workloads as W
    from dynamic_sparse_attention_pool_amd.pipelines import BlockSparseLayer
    inp = W.prefill_fp32(W.CONFIG_SEEDS[1], 1, 1, 1024, 64)
    layer = BlockSparseLayer(dev_t(inp.q), dev_t(inp.k), dev_t(inp.v), n_sink=1, n_local=1, k_fixed=2)
    layer.step()
    torch.cuda.synchronize()
    R = Reps()
    R.run(max(reps, 50), [("estimate", layer.estimate), ("select", layer.select), ("forward", layer.forward)], clock="c1_1k_fp32")
    kept = int(layer.cnt.sum().item())
    lay = R.total(["estimate", "select", "forward"])
    return {"workload": "block-sparse parity layer: 1024 tokens, 1 head, d64, fp32, blocks of 64 (16x16 grid), "
                        "sink + diagonal + top-2 other causal blocks",
            "kept_blocks": kept, "flop": kept * 4 * 64 * 64 * 64,
            "us_layer_median": lay["median"] * 1e3, "us_layer_min": lay["min"] * 1e3,
            "us_forward_median": R.stat("forward")["median"] * 1e3, "reps": lay["n"],
            "bound": "16 workgroups, one per query block: the serial work per tile (parity configuration; no roofline claim)", "inputs": inp}


def config2(reps, peaks):
    """32K GQA 32/8 d128 bf16 layer, sink + 4 local + ceil(10%)."""
    import torch
    import workloads as W
    from dynamic_sparse_attention_pool_amd.pipelines import BlockSparseLayer
    inp = W.prefill_bf16(W.CONFIG_SEEDS[2], 1, 32, 8, 32768, 128)
    layer = BlockSparseLayer(dev_bf16(inp.q), dev_bf16(inp.k), dev_bf16(inp.v), n_sink=1, n_local=4,
                             ratio=(10, 100), out_dtype=torch.bfloat16)
    for _ in range(3):
        layer.step()
    torch.cuda.synchronize()
    R = Reps()
    R.run(reps, [("estimate", layer.estimate), ("select", layer.select), ("forward", layer.forward)], clock="c2_32k")
    kept = int(layer.cnt.sum().item())
    flop = kept * FLOP_PER_BLOCK_128
    fwd = R.stat("forward")
    tf = flop / (fwd["median"] * 1e-3) / 1e12
    lay = R.total(["estimate", "select", "forward"])
    out = {"workload": "block-sparse layer: 32768 tokens, GQA 32/8, d128, bf16, 1% keys +3u / queries +1u, "
                       "sink + 4 local + ceil(10%) blocks of 64",
           "kept_blocks": kept, "flop": flop, "ms_layer_median": lay["median"], "ms_layer_min": lay["min"],
           "ms_estimate_median": R.stat("estimate")["median"], "ms_select_median": R.stat("select")["median"],
           "ms_forward_median": fwd["median"], "ms_forward_min": fwd["min"], "forward_TFLOP_per_s": tf,
           "target_forward_ms": 0.85, "reps": lay["n"], "inputs": inp}
    out.update(frac_pair(tf, PEAK_BF16_TFLOPS, peaks.get("mfma_bf16_TFLOP_per_s")))
    del layer
    torch.cuda.empty_cache()
    return out


# ---------------------------------------------------------------- config 3, vertical-slash
def vs_table_keys(layer):
    """Kept keys over all query blocks of a vertical-slash layer, counted from
    its built tables."""
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


def vs_config(reps, inp, peaks):
    import torch
    from dynamic_sparse_attention_pool_amd.pipelines import VerticalSlashLayer
    q, k, v = dev_bf16(inp.q), dev_bf16(inp.k), dev_bf16(inp.v)
    layer = VerticalSlashLayer(q, k, v, n_vert=1000, n_slash=64, out_dtype=torch.bfloat16)
    layer.step()
    torch.cuda.synchronize()
    R = Reps()
    R.run(reps, [("estimate", layer.estimate), ("select", layer.select), ("forward", layer.forward)], clock="vslash_128k")
    flop = vs_table_keys(layer) * 4 * 64 * 128
    fwd = R.stat("forward")
    tf = flop / (fwd["median"] * 1e-3) / 1e12
    lay = R.total(["estimate", "select", "forward"])
    out = {"workload": "vertical-slash layer at 131072 (the 128K data): last-64-query estimate, top 1000 columns "
                       "+ top 64 offsets",
           "ms_layer_median": lay["median"], "ms_layer_min": lay["min"],
           "ms_estimate_median": R.stat("estimate")["median"], "ms_select_build_median": R.stat("select")["median"],
           "ms_forward_median": fwd["median"], "ms_forward_min": fwd["min"], "kept_key_flop": flop,
           "forward_TFLOP_per_s": tf, "reps": lay["n"],
           "sel": (layer.vert.cpu().numpy(), layer.vert_cnt.cpu().numpy(), layer.slash.cpu().numpy(),
                   layer.slash_cnt.cpu().numpy())}
    out.update(frac_pair(tf, PEAK_BF16_TFLOPS, peaks.get("mfma_bf16_TFLOP_per_s")))
    del layer
    torch.cuda.empty_cache()
    return out


# ---------------------------------------------------------------- config 4, clustered decode
def decode_config(steps, peaks, mass=None):
    """Clustered decode step; with ``mass`` the adaptive budget (fewest
    clusters holding that share of the centroid-score softmax, 1..64).  A
    decode step is a handful of short launches: each part is captured as a HIP
    graph and `steps` replays run back to back between two events (the host's
    launch cost is not what gets timed), rotating 4 contexts so no step finds
    the previous one's context in the 256 MB Infinity Cache."""
    import torch
    import workloads as W
    from dynamic_sparse_attention_pool_amd.pipelines import ClusterDecode
    T, Hq, Hkv, N, d, C, ksel = 8, 32, 8, 65536, 128, 256, 64
    copies, inps = [], []
    for c in range(4):
        inp = W.decode_clustered(W.CONFIG_SEEDS[4] + 100 * c, T, Hq, Hkv, N, d, C)
        inps.append(inp)
        copies.append(ClusterDecode(dev_bf16(inp.q), dev_bf16(inp.k), dev_bf16(inp.v), dev_t(inp.labels),
                                    dev_t(inp.centroids), n_sel=ksel, mass=mass, k_min=1, fused=True))
    torch.cuda.synchronize()
    for i in range(8):
        copies[i % 4].step()
    torch.cuda.synchronize()
    # one graph per part holding `reps` rounds over the 4 contexts, so a replay
    # runs 4*reps launches back to back on the GPU (no host launch in between)
    reps_g = max(1, steps // 4)
    graphs = []
    for which in ("estimate", "forward", "step"):
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            for _ in range(reps_g):
                for dc in copies:
                    getattr(dc, which)()
        graphs.append(gr)
    torch.cuda.synchronize()

    def timed(which):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        graphs[which].replay()
        torch.cuda.synchronize()
        ev[0].record()
        graphs[which].replay()
        ev[1].record()
        if which == 2:
            clock_sample("decode" if mass is None else "decode_adaptive")
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) / (4 * reps_g)

    ms_step = [timed(2) for _ in range(5)]
    ms_est = [timed(0) for _ in range(3)]
    ms_fwd = [timed(1) for _ in range(3)]
    kv_bytes = 0
    for dc in copies:
        sel = dc.sel.cpu().numpy()
        ptr = dc.ptr.cpu().numpy().astype(np.int64)
        for g in range(Hkv):
            used = np.unique(sel[:, g * (Hq // Hkv):(g + 1) * (Hq // Hkv), :])
            used = used[used >= 0]
            kv_bytes += int((ptr[g, used + 1] - ptr[g, used]).sum()) * 2 * d * 2
    kv_bytes //= len(copies)
    small = T * Hq * d * 2 + Hkv * C * d * 4 + T * Hq * d * 4
    ms = float(np.median(ms_step))
    fwd = float(np.median(ms_fwd))
    hbm = peaks.get("hbm_read_GB_per_s")
    rule = ("top 64 of 256 clusters" if mass is None else
            f"fewest clusters holding {mass:g} of the centroid-score softmax, 1..64 of 256")
    out = {"workload": f"clustered decode: 8 queries x 32/8 heads, d128, 65536-key context, {rule} (scores and "
                       "selection in one call, then the gathered attention); each part captured as one HIP graph "
                       "of 4 x reps steps rotating 4 contexts, replayed whole",
           "mean_clusters": float(np.mean([dc.sel_cnt.float().mean().item() for dc in copies])),
           "us_per_step_median": ms * 1e3, "us_per_step_min": float(np.min(ms_step)) * 1e3,
           "us_per_token": ms * 1e3 / T, "kv_bytes_per_step": kv_bytes,
           "KV_GB_per_s_step": (kv_bytes + small) / (ms * 1e-3) / 1e9,
           "us_estimate_select": float(np.median(ms_est)) * 1e3, "us_gather": fwd * 1e3,
           "KV_GB_per_s_gather": kv_bytes / (fwd * 1e-3) / 1e9,
           "frac_hbm_spec_step": (kv_bytes + small) / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
           "frac_hbm_measured_step": ((kv_bytes + small) / (ms * 1e-3) / 1e9 / hbm) if hbm else None,
           "target_us_per_step": 47.9, "steps_per_timing": 4 * reps_g}
    if mass is None:
        out["inputs"] = inps[0]
        out["sel0"] = copies[0].sel.cpu().numpy()
    del copies, graphs
    torch.cuda.empty_cache()
    return out


# ---------------------------------------------------------------- config 5, indexer + IndexCache
def indexer_config(reps, peaks):
    import torch
    import workloads as W
    import dynamic_sparse_attention_pool_amd as sa
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
    fu = IndexerPrefill(ip.qi, ip.ki, ip.w, ind.pos0, layers, k_sel=k_sel, out_dtype=torch.bfloat16, fused=True)
    ip.step(reuse=True)
    fu.step(reuse=True)
    torch.cuda.synchronize()
    R = Reps()
    r = max(5, reps // 4)
    R.run(r, [("indexer", lambda: sa.sa_estimate(sa.INDEXER, ip.qi, ip.ki, ip.scores, weights=ip.w,
                                                 q_pos0=ip.pos0)),
              ("select", lambda: sa.sa_select_topk(ip.scores, ip.idx, ip.cnt, k=k_sel, causal=True, causal_period=T,
                                                   causal_offset=ip.pos0)),
              ("attend", lambda: ip.attend(1)),
              ("index_fused", lambda: fu.index(check=False))], clock="indexer")
    R.run(max(3, r // 2), [("total_reuse", lambda: ip.step(reuse=True)),
                           ("total_noreuse", lambda: ip.step(reuse=False)),
                           ("total_reuse_fused", lambda: fu.step(reuse=True))])
    same = bool(torch.equal(fu.idx, ip.idx)) and int(fu.err.item()) == 0
    pairs = sum(ind.pos0 + t + 1 for t in range(T))
    idx_ms = R.stat("indexer")["median"]
    tf = pairs * 8192 / (idx_ms * 1e-3) / 1e12
    out = {"workload": "token top-2048 prefill chunk: 4096 queries at the end of a 131072-token context, 64x64 "
                       "indexer, MQA 16/1 d128, 4 layers, layer 1 full / 2-4 reuse its index",
           "ms_indexer_median": idx_ms, "ms_indexer_min": R.stat("indexer")["min"], "indexer_TFLOP_per_s": tf,
           "target_indexer_ms": 3.44, "ms_select_median": R.stat("select")["median"],
           "ms_attend_layer_median": R.stat("attend")["median"],
           "ms_index_fused_median": R.stat("index_fused")["median"],
           "ms_4layers_with_reuse": R.stat("total_reuse")["median"],
           "ms_4layers_without_reuse": R.stat("total_noreuse")["median"],
           "ms_4layers_with_reuse_fused": R.stat("total_reuse_fused")["median"],
           "fused_index_equals_two_call": same, "reps": r, "inputs": ind}
    out.update(frac_pair(tf, PEAK_BF16_TFLOPS, peaks.get("mfma_bf16_TFLOP_per_s")))
    del ip, fu, layers
    torch.cuda.empty_cache()
    return out


# ---------------------------------------------------------------- further extras
def mixed_extra(reps, inp):
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
    layer.step()
    torch.cuda.synchronize()
    R = Reps()
    R.run(reps, [("estimate", layer.estimate), ("select", layer.select), ("forward", layer.forward)])
    parts = {type(p).__name__: p for p in layer.parts}
    nb = N // 64
    a_blocks = sum(len(set(range(min(1, i + 1))) | set(range(max(0, i - 3), i + 1))) for i in range(nb))
    flop = (int(parts["BlockSparseLayer"].cnt.sum().item()) + a_blocks * len(layer.groups["A"])) * FLOP_PER_BLOCK_128
    flop += vs_table_keys(parts["VerticalSlashLayer"]) * 4 * 64 * 128
    lay = R.total(["estimate", "select", "forward"])
    fwd = R.stat("forward")["median"]
    return {"workload": "mixed-pattern layer at 131072, GQA 32/8, d128: per KV head 1 A-shape (sink + 4 local), "
                        "1 vertical-slash (1000 cols, 64 offsets), 2 block-sparse (sink + 4 local + ceil(5%)) heads",
            "ms_layer_median": lay["median"], "ms_forward_median": fwd, "kept_flop": flop,
            "forward_TFLOP_per_s": flop / (fwd * 1e-3) / 1e12}


def fused_extra(reps, inp):
    """Block estimate + top-k at 131072 tokens: the fused call (no score
    matrix) against pooled scores followed by the separate selection."""
    import torch
    from dynamic_sparse_attention_pool_amd.pipelines import BlockSparseLayer
    q, k, v = dev_bf16(inp.q), dev_bf16(inp.k), dev_bf16(inp.v)
    res = {"workload": "block estimate + top-k at 131072, GQA 32/8, d128, sink + 4 local + ceil(5%)"}
    ref = None
    for name, fused in (("separate", False), ("fused", True)):
        layer = BlockSparseLayer(q, k, v, n_sink=1, n_local=4, ratio=(5, 100), fused=fused)
        layer.estimate()
        layer.select()
        torch.cuda.synchronize()
        R = Reps()
        R.run(reps, [("es", lambda: (layer.estimate(), layer.select()))])
        res[f"ms_{name}_median"] = R.stat("es")["median"]
        if fused:
            same = (layer.cnt == ref[1]) & (layer.idx == ref[0]).all(dim=-1)
            res["rows_identical_frac"] = float(same.float().mean().item())
        else:
            ref = (layer.idx.clone(), layer.cnt.clone())
        del layer
        torch.cuda.empty_cache()
    return res


def kmeans_extra(reps, iters=10):
    """Offline clustering of the decode context: 8 KV heads x 65536 keys, d128,
    256 clusters, Lloyd iterations from sampled keys."""
    import torch
    import workloads as W
    from dynamic_sparse_attention_pool_amd import sa_kmeans
    Hkv, N, d, C_ = 8, 65536, 128, 256
    inp = W.decode_clustered(W.CONFIG_SEEDS[4], 1, Hkv, Hkv, N, d, C_)
    k = dev_bf16(inp.k)
    init = dev_t(W.kmeans_init(W.CONFIG_SEEDS[4], inp.k, C_))
    cent = init.clone()
    labels = torch.empty((Hkv, N), dtype=torch.int32, device=k.device)
    ptr = torch.empty((Hkv, C_ + 1), dtype=torch.int32, device=k.device)
    perm = torch.empty((Hkv, N), dtype=torch.int32, device=k.device)
    ws = sa_kmeans(k, cent, labels, iters=1, cluster_ptr=ptr, perm=perm)
    torch.cuda.synchronize()
    R = Reps()
    for _ in range(reps):
        cent.copy_(init)
        R.flush()
        R.span("km", lambda: sa_kmeans(k, cent, labels, iters=iters, cluster_ptr=ptr, perm=perm, workspace=ws))
    torch.cuda.synchronize()
    ms = R.stat("km")["median"]
    tflops = 2.0 * Hkv * N * C_ * d * iters / (ms * 1e-3) / 1e12
    return {"workload": f"k-means of the decode context: 8 KV heads x 65536 keys, d128, 256 clusters, {iters} Lloyd "
                        "iterations from sampled keys",
            "ms_per_iteration": ms / iters, "distance_TFLOP_per_s_over_whole_iterations": tflops,
            "frac_bf16_spec_three_products": 3 * tflops / PEAK_BF16_TFLOPS}


# ---------------------------------------------------------------- CPU oracle
def cpu_info():
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        cores = len(os.sched_getaffinity(0))
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return int(cores), model


def _bf(x):
    import workloads as W
    return W.bf16_to_f32(x)


def oracle_blocksparse(inp, ratio, n_local, k_fixed, budget_s, d=128):
    """Heads 0, 1, ...: each head's pooled estimate and selection of every row,
    then fp64 attention for its longest query-block rows, 16 at a time, until
    the budget is used.  Returns (TFLOP/s on kept blocks, description)."""
    import oracle
    Hq, Hkv, N = inp.q.shape[1], inp.k.shape[1], inp.q.shape[2]
    nb = N // 64
    scale = 1 / math.sqrt(d)
    t_total, flop, rows_done, heads = 0.0, 0, 0, 0
    for h in range(Hq):
        g = h * Hkv // Hq
        q0 = _bf(inp.q[0:1, h:h + 1])   # widen only the sampled head
        k0 = _bf(inp.k[0:1, g:g + 1])
        v0 = _bf(inp.v[0:1, g:g + 1])
        t0 = time.perf_counter()
        S = oracle.block_scores(q0, k0, 64, scale)
        kept = oracle.block_select(S, n_sink=1, n_local=n_local, k=k_fixed, ratio=ratio)
        t_sel = time.perf_counter() - t0
        done = 0
        t1 = time.perf_counter()
        order = list(range(nb - 1, -1, -1))
        for c in range(0, nb, 16):
            rows = order[c:c + 16]
            oracle.block_sparse_attention(q0, k0, v0, kept, 64, scale, heads=[0], blocks=rows)
            done += len(rows)
            flop += sum(len(kept[0][0][i]) for i in rows) * 4 * 64 * 64 * d
            if t_total + time.perf_counter() - t1 + t_sel > budget_s:
                break
        t_total += time.perf_counter() - t1 + t_sel * done / nb
        rows_done += done
        heads += 1
        if t_total > budget_s:
            break
    return flop / t_total / 1e12, (f"heads 0..{heads - 1}: each head's pooled estimate + selection (time pro-rated to "
                                   f"its sampled rows) and fp64 attention for its longest query-block rows, "
                                   f"{rows_done} query-block rows in all ({nb} per head); {flop / 1e9:.2f} GFLOP of kept blocks "
                                   f"in {t_total:.2f}s")


def oracle_all(res, headline_inp, budget):
    import oracle
    import workloads as W
    cores, model = cpu_info()
    out = {"cores": cores, "cpu_model": model, "kind": "oracle (fp64 NumPy, as committed)"}
    # config 1: the whole layer
    c1 = res["c1"]["inputs"]
    t0 = time.perf_counter()
    S = oracle.block_scores(c1.q, c1.k, 64, 1 / 8.0)
    kept = oracle.block_select(S, n_sink=1, n_local=1, k=2)
    oracle.block_sparse_attention(c1.q, c1.k, c1.v, kept, 64, 1 / 8.0)
    out["c1"] = {"ms": (time.perf_counter() - t0) * 1e3, "sample": "the whole layer"}
    # config 2: head 0 sample
    tf, desc = oracle_blocksparse(res["c2"]["inputs"], (10, 100), 4, None, budget["c2"])
    out["c2"] = {"TFLOP_per_s": tf, "sample": desc}
    # config 3 block-sparse: the headline's cpu_baseline
    tf, desc = oracle_blocksparse(headline_inp, (5, 100), 4, None, budget["c3"])
    out["c3_blocksparse"] = {"TFLOP_per_s": tf, "sample": desc}
    # config 3 vertical-slash: head 0's estimate, selection and a few query blocks
    if "c3_vs" in res and "sel" in res["c3_vs"]:
        N = headline_inp.q.shape[2]
        q0, k0, v0 = _bf(headline_inp.q[0, 0]), _bf(headline_inp.k[0, 0]), _bf(headline_inp.v[0, 0])
        scale = 1 / math.sqrt(128)
        t0 = time.perf_counter()
        av, as_ = oracle.vs_estimate(q0[N - 64:], k0, np.arange(N - 64, N), scale)
        cols, offs = oracle.vs_select(av, as_, 1000, 64)
        t_est = time.perf_counter() - t0
        nb = N // 64
        blocks = list(range(nb - 1, nb - 1 - 64, -8))
        t1 = time.perf_counter()
        sel = [[(cols, offs)]]
        oracle.vs_attention(q0[None, None], k0[None, None], v0[None, None], sel, 64, scale, heads=[0], blocks=blocks)
        t_att = time.perf_counter() - t1
        out["c3_vslash"] = {"s_estimate_select_head": t_est, "s_attention_per_block": t_att / len(blocks),
                            "sample": f"head 0: last-64 estimate + selection, then attention for {len(blocks)} "
                                      "query blocks near the end"}
    # config 4: the whole decode step of one context
    dec = res["c4"]["inputs"]
    t0 = time.perf_counter()
    scale = 1 / math.sqrt(128)
    s = oracle.centroid_scores(W.bf16_to_f32(dec.q), dec.centroids, scale)
    sel = oracle.cluster_select(s, 64)
    oracle.cluster_decode(W.bf16_to_f32(dec.q), W.bf16_to_f32(dec.k), W.bf16_to_f32(dec.v), dec.labels, sel, scale)
    out["c4"] = {"ms_step": (time.perf_counter() - t0) * 1e3, "sample": "one whole decode step (8 tokens x 32 heads)"}
    # config 5: a few query rows of the indexer, their selection and layer-1 attention
    ind = res["c5"]["inputs"]
    rows = np.array([0, 1365, 2730, 4095])
    t0 = time.perf_counter()
    I = oracle.indexer_scores(W.bf16_to_f32(ind.qi), W.bf16_to_f32(ind.ki), ind.w, ind.pos0, rows)
    oracle.indexer_select(I, rows, ind.pos0, 2048)
    dt = time.perf_counter() - t0
    out["c5"] = {"ms_indexer_select_per_query": dt * 1e3 / rows.size,
                 "indexer_TFLOP_per_s": float(sum(ind.pos0 + int(t) + 1 for t in rows)) * 8192 / dt / 1e12,
                 "sample": f"indexer scores + top-2048 of {rows.size} query rows"}
    return out


# ---------------------------------------------------------------- main
def strip(d):
    return {k: v for k, v in d.items() if k not in ("inputs", "sel", "sel0")}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--reps", type=int, default=20, help="reps per workload for the median/min (at least 20)")
    ap.add_argument("--no-extras", action="store_true", help="only the 128K layer (profiling runs)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--only", default="", help="comma list of parts: c1,c2,vs,decode,decode_adaptive,indexer,mixed,"
                                               "kmeans,fused,peaks")
    ap.add_argument("--pmc-copy", action="store_true",
                    help="first run a plain 1 GiB device copy, the known-size reference for HBM counters")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (each GPU would run "
              "the same kernels on its own share of heads); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    reps = max(20, args.reps)
    import torch
    import dynamic_sparse_attention_pool_amd as sa
    sa.load()
    torch.cuda.init()
    global CLOCK
    CLOCK = ClockWindows()

    if args.pmc_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log("[bench] reference copy: 1073741824 bytes read, 1073741824 bytes written")
        del src, dst
    only = set(x for x in args.only.split(",") if x)

    def want(name):
        return not args.no_extras and (not only or name in only)

    peaks = {}
    if want("peaks"):
        log("[bench] achievable peaks")
        peaks = measured_peaks()
    log("[bench] 128K block-sparse layer")
    main_res = prefill_headline(args.steps, args.warmup, reps, seed=3)
    ms = main_res["ms_per_step"]
    value = main_res["flop"] / (ms * 1e-3) / 1e12
    fwd_ms = main_res["contract_ms"]["forward"]
    fwd_tflops = main_res["flop"] / (fwd_ms * 1e-3) / 1e12
    traffic = traffic_for()
    line = {
        "metric": "sparse-attn prefill TFLOP/s (kept blocks) & ms at 128K; decode KV GB/s",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "block-sparse prefill layer, 131072 tokens, batch 1, GQA 32/8, head_dim 128, "
                               "1% keys +3u / queries +1u, sink + 4 local + ceil(5%) blocks of 64",
                   "seq_len": 131072, "heads_q": 32, "heads_kv": 8, "head_dim": 128, "block": 64,
                   "kept_blocks": main_res["kept_blocks"], "parallelism": "single GPU"},
        "breakdown_ms": {k: round(v, 4) for k, v in main_res["contract_ms"].items()},
        "timing": {"method": f"{reps} reps, each after a 512 MB write, HIP events on the launch stream",
                   "ms_layer_median": main_res["layer"]["median"], "ms_layer_min": main_res["layer"]["min"],
                   "ms_forward_median": main_res["parts"]["forward"]["median"],
                   "ms_forward_min": main_res["parts"]["forward"]["min"],
                   "ms_estimate_median": main_res["parts"]["estimate"]["median"],
                   "ms_select_median": main_res["parts"]["select"]["median"],
                   "TFLOP_per_s_layer_median": main_res["flop"] / (main_res["layer"]["median"] * 1e-3) / 1e12},
        "clock": CLOCK.summary() if CLOCK is not None else None,
        "peaks": {"mfma_bf16_spec_TFLOP_per_s": PEAK_BF16_TFLOPS, "hbm_spec_GB_per_s": PEAK_HBM_GBS, **peaks},
        "roofline": {"bound": "mfma", "kernel": "k_fwd_bf16<128,block>", "achieved": round(fwd_tflops, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(fwd_tflops / PEAK_BF16_TFLOPS, 4),
                     "frac_measured_peak": (round(fwd_tflops / peaks["mfma_bf16_TFLOP_per_s"], 4)
                                            if peaks.get("mfma_bf16_TFLOP_per_s") else None),
                     "traffic": traffic},
    }
    if traffic is not None:
        # FETCH_SIZE + WRITE_SIZE count L2 misses, served by HBM or by the Infinity Cache: fabric bytes
        tbps = traffic / (fwd_ms * 1e-3) / 1e12
        line["roofline"]["traffic_note"] = "L2-miss bytes per launch (HBM or Infinity Cache), rocprofv3 counters"
        line["roofline"]["l2_miss_TB_per_s"] = round(tbps, 3)
    res = {}
    steps_dec = max(args.steps, 20)
    for name, fn in [("c1", lambda: config1(reps)), ("c2", lambda: config2(reps, peaks)),
                     ("c3_vs", lambda: vs_config(reps, main_res["inputs"], peaks)),
                     ("c4", lambda: decode_config(steps_dec, peaks)),
                     ("c4_adaptive", lambda: decode_config(steps_dec, peaks, mass=0.5)),
                     ("c5", lambda: indexer_config(reps, peaks)),
                     ("mixed", lambda: mixed_extra(max(3, reps // 4), main_res["inputs"])),
                     ("kmeans", lambda: kmeans_extra(3)),
                     ("fused", lambda: fused_extra(reps, main_res["inputs"]))]:
        key = {"c3_vs": "vs", "c4": "decode", "c4_adaptive": "decode_adaptive", "c5": "indexer"}.get(name, name)
        if not want(key):
            continue
        try:
            log(f"[bench] {name}")
            res[name] = fn()
        except Exception as e:  # noqa: BLE001  (a part that fails is reported, not fatal)
            res[name] = {"error": f"{type(e).__name__}: {e}"}
        torch.cuda.empty_cache()
    if res:
        line["configs"] = {k: strip(v) for k, v in res.items()}
    if not args.no_cpu:
        log("[bench] cpu oracle")
        cores, model = cpu_info()
        if all(k in res and "error" not in res[k] for k in ("c1", "c2", "c4", "c5")):
            orc = oracle_all(res, main_res["inputs"], {"c2": 10.0, "c3": 15.0})
            line["oracle_per_config"] = orc
            tf, desc = orc["c3_blocksparse"]["TFLOP_per_s"], orc["c3_blocksparse"]["sample"]
        else:
            tf, desc = oracle_blocksparse(main_res["inputs"], (5, 100), 4, None, 15.0)
        line["cpu_baseline"] = {"value": tf, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
                                "cpu_model": model, "sample": desc}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
