"""The C-ABI library loads, exports every entry point include/sa.h declares,
agrees with the binding on struct layouts, and rejects bad arguments on the
host before any launch.  CPU only: no call here reaches a kernel."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sa.h")
HEADERS = sorted(os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include")) if f.endswith(".h"))


def declared_functions():
    """Every function any include/*.h declares."""
    text = "".join(open(h).read() for h in HEADERS)
    return sorted(set(re.findall(r"^(?:int|const char\*|size_t)\s+(sa_\w+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def lib():
    import torch  # noqa: F401  (load the HIP runtime the way the product does)
    from dynamic_sparse_attention_pool_amd import _ffi
    return _ffi.load()


def test_header_declares_the_four_entry_points_and_helpers():
    names = declared_functions()
    for n in ["sa_estimate", "sa_select_topk", "sa_block_sparse_fwd", "sa_gather_decode", "sa_gather_decode_static",
              "sa_vs_build",
              "sa_cluster_pack", "sa_select_mass", "sa_kmeans", "sa_estimate_topk", "sa_indexer_topk", "sa_last_error",
              "sa_version",
              "sa_args_size", "sa_peak_mfma_bf16", "sa_peak_read"]:
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    from dynamic_sparse_attention_pool_amd import _ffi
    for n in declared_functions():
        assert hasattr(lib, n), n
        assert n in _ffi.SYMBOLS, f"binding lacks {n}"


def test_struct_layouts_and_version(lib):
    from dynamic_sparse_attention_pool_amd import _ffi
    assert lib.sa_version() == _ffi.ABI_VERSION
    for i, st in enumerate(_ffi.STRUCTS):
        assert lib.sa_args_size(i) == C.sizeof(st)
    assert lib.sa_args_size(99) == 0


def _err(lib):
    return lib.sa_last_error().decode()


def test_fwd_argument_errors(lib):
    from dynamic_sparse_attention_pool_amd import _ffi as F
    a = F.FwdArgs()
    assert lib.sa_block_sparse_fwd(None, None, 0, None) == 1
    assert lib.sa_block_sparse_fwd(C.byref(a), None, 0, None) == 1   # q/k/v/out NULL
    a.q = a.k = a.v = a.out = 256
    a.dtype, a.out_dtype, a.block_size, a.head_dim = F.SA_BF16, F.SA_F32, 64, 128
    a.batch, a.heads_q, a.heads_kv, a.seq, a.scale = 1, 4, 3, 128, 0.1
    assert lib.sa_block_sparse_fwd(C.byref(a), None, 0, None) == 2   # 4 % 3
    assert "multiple" in _err(lib)
    a.heads_kv = 2
    a.seq = 100
    assert lib.sa_block_sparse_fwd(C.byref(a), None, 0, None) == 2
    a.seq = 128
    a.head_dim = 96
    assert lib.sa_block_sparse_fwd(C.byref(a), None, 0, None) == 6
    a.head_dim = 128
    a.q = 264   # misaligned
    assert lib.sa_block_sparse_fwd(C.byref(a), None, 0, None) == 4
    a.q = 256
    a.dtype = F.SA_I32
    assert lib.sa_block_sparse_fwd(C.byref(a), None, 0, None) == 3
    a.dtype = F.SA_BF16
    a.scale = -1.0
    assert lib.sa_block_sparse_fwd(C.byref(a), None, 0, None) == 8
    a.scale = 0.1
    assert lib.sa_block_sparse_fwd(C.byref(a), None, 0, None) == 1   # block tables missing
    a.mode = 7
    assert lib.sa_block_sparse_fwd(C.byref(a), None, 0, None) == 8


def test_select_argument_errors(lib):
    from dynamic_sparse_attention_pool_amd import _ffi as F
    a = F.SelectArgs()
    a.scores = a.idx = a.cnt = 256
    a.rows, a.ncand, a.ld, a.k, a.kmax = 4, 10, 8, 2, 4
    assert lib.sa_select_topk(C.byref(a), None, 0, None) == 2       # ld < ncand
    a.ld = 10
    a.n_sink, a.n_local, a.k, a.kmax = 1, 1, 3, 4
    assert lib.sa_select_topk(C.byref(a), None, 0, None) == 2       # 1+1+3 > 4
    assert "kmax" in _err(lib)
    a.kmax = 5
    n = C.c_size_t(7)
    assert lib.sa_select_topk_workspace_bytes(C.byref(a), C.byref(n)) == 0 and n.value == 0
    a.causal, a.causal_period = 1, 0
    assert lib.sa_select_topk(C.byref(a), None, 0, None) == 8
    a.causal, a.causal_period, a.causal_offset = 1, 16, 0
    a.ratio_num, a.ratio_den, a.n_sink, a.n_local, a.ncand, a.ld, a.rows = 10, 100, 1, 4, 16, 16, 16
    a.kmax = 6   # row 15: 5 forced + ceil(1.6)=2 -> 7
    assert lib.sa_select_topk(C.byref(a), None, 0, None) == 2
    a.kmax = 7
    assert lib.sa_select_topk_workspace_bytes(C.byref(a), C.byref(n)) == 0


def test_select_mass_argument_errors(lib):
    from dynamic_sparse_attention_pool_amd import _ffi as F
    a = F.SelectMassArgs()
    assert lib.sa_select_mass(None, None) == 1
    a.rows = 4
    assert lib.sa_select_mass(C.byref(a), None) == 1                 # pointers missing
    a.scores = a.idx = a.cnt = 256
    a.rows, a.ncand, a.ld, a.mass, a.k_min, a.k_max, a.kmax = 4, 5000, 5000, 0.5, 1, 64, 64
    assert lib.sa_select_mass(C.byref(a), None) == 2                 # above 4096 candidates
    a.ncand = a.ld = 256
    for bad in (0.0, -0.1, 1.5, float("nan")):
        a.mass = bad
        assert lib.sa_select_mass(C.byref(a), None) == 8
    a.mass = 1.0
    a.k_min = 65
    assert lib.sa_select_mass(C.byref(a), None) == 8                 # k_min > k_max
    a.k_min, a.kmax = 1, 63
    assert lib.sa_select_mass(C.byref(a), None) == 2                 # kmax < min(k_max, ncand)
    assert "kmax" in _err(lib)
    a.ncand = a.ld = 40
    a.rows = 0                                                       # min(64, 40) = 40 fits; nothing to launch
    assert lib.sa_select_mass(C.byref(a), None) == 0
    a.scores = a.idx = a.cnt = None                                  # empty tensors carry NULL pointers
    assert lib.sa_select_mass(C.byref(a), None) == 0
    a.rows = 1
    assert lib.sa_select_mass(C.byref(a), None) == 1
    t = F.SelectArgs()
    t.rows, t.ncand, t.ld, t.k, t.kmax = 0, 10, 10, 2, 2
    assert lib.sa_select_topk(C.byref(t), None, 0, None) == 0
    t.rows = 3
    assert lib.sa_select_topk(C.byref(t), None, 0, None) == 1


def test_head_list_and_ashape_argument_errors(lib):
    from dynamic_sparse_attention_pool_amd import _ffi as F
    a = F.FwdArgs()
    a.q = a.k = a.v = a.out = 256
    a.dtype, a.out_dtype, a.block_size, a.head_dim = F.SA_BF16, F.SA_F32, 64, 128
    a.batch, a.heads_q, a.heads_kv, a.seq, a.scale = 1, 8, 2, 128, 0.1
    a.mode = F.SA_FWD_ASHAPE
    a.n_sink, a.n_local = -1, 4
    assert lib.sa_block_sparse_fwd_workspace_bytes(C.byref(a), C.byref(C.c_size_t())) == 8
    a.n_sink, a.n_local = 1000, 1049
    assert lib.sa_block_sparse_fwd_workspace_bytes(C.byref(a), C.byref(C.c_size_t())) == 6
    a.n_sink, a.n_local = 1, 4
    assert lib.sa_block_sparse_fwd_workspace_bytes(C.byref(a), C.byref(C.c_size_t())) == 0
    for heads, code in [([3, 3], 8), ([8], 8), ([-1], 8), ([], 8), (list(range(8)), 0), ([7, 0, 2], 0)]:
        arr = (C.c_int32 * max(1, len(heads)))(*heads)
        a.head_list, a.n_heads_list = C.cast(arr, C.c_void_p), len(heads)
        assert lib.sa_block_sparse_fwd_workspace_bytes(C.byref(a), C.byref(C.c_size_t())) == code, heads
    e = F.EstimateArgs()
    e.q = e.k = e.scores = e.centroids = 256
    e.kind, e.dtype, e.batch, e.heads_q, e.heads_kv, e.seq_q, e.seq_k, e.head_dim = 0, F.SA_BF16, 1, 4, 2, 128, 128, 128
    e.block_size, e.scale, e.n_centroids = 64, 0.1, 16
    n = C.c_size_t(0)
    assert lib.sa_estimate_workspace_bytes(C.byref(e), C.byref(n)) == 0
    full = n.value
    arr = (C.c_int32 * 1)(2)
    e.head_list, e.n_heads_list = C.cast(arr, C.c_void_p), 1
    assert lib.sa_estimate_workspace_bytes(C.byref(e), C.byref(n)) == 0 and n.value < full   # one pooled head
    e.n_heads_list = 5
    assert lib.sa_estimate_workspace_bytes(C.byref(e), C.byref(n)) == 8
    e.kind, e.n_heads_list = F.SA_EST_CENTROID, 1
    assert lib.sa_estimate_workspace_bytes(C.byref(e), C.byref(n)) == 6


def test_kmeans_argument_errors(lib):
    from dynamic_sparse_attention_pool_amd import _ffi as F
    a = F.KmeansArgs()
    n = C.c_size_t(0)
    assert lib.sa_kmeans_workspace_bytes(C.byref(a), C.byref(n)) == 1
    a.k = a.centroids = a.labels = 256
    a.heads_kv, a.n_ctx, a.head_dim, a.n_clusters, a.iters, a.dtype = 8, 65536, 128, 256, 3, F.SA_BF16
    assert lib.sa_kmeans_workspace_bytes(C.byref(a), C.byref(n)) == 0 and n.value > 8 * 65536 * 4
    with_ws = n.value
    a.cluster_ptr = 512
    assert lib.sa_kmeans_workspace_bytes(C.byref(a), C.byref(n)) == 1        # ptr without perm
    a.perm = 1024
    assert lib.sa_kmeans_workspace_bytes(C.byref(a), C.byref(n)) == 0 and n.value < with_ws
    for field, bad, code in [("n_clusters", 0, 2), ("n_clusters", 5000, 2), ("iters", 0, 8), ("head_dim", 96, 6),
                             ("dtype", F.SA_I32, 3)]:
        good = getattr(a, field)
        setattr(a, field, bad)
        assert lib.sa_kmeans_workspace_bytes(C.byref(a), C.byref(n)) == code, field
        setattr(a, field, good)
    a.k = 264
    assert lib.sa_kmeans_workspace_bytes(C.byref(a), C.byref(n)) == 4
    a.k = 256
    assert lib.sa_kmeans(C.byref(a), None, 0, None) == 5                      # workspace missing


def test_estimate_topk_argument_errors(lib):
    from dynamic_sparse_attention_pool_amd import _ffi as F
    a = F.EstimateTopkArgs()
    n = C.c_size_t(0)
    assert lib.sa_estimate_topk_workspace_bytes(C.byref(a), C.byref(n)) == 1
    a.q = a.k_ptr = a.idx = a.cnt = 256
    a.kind, a.dtype, a.block_size, a.scale = F.SA_EST_BLOCK_MEANPOOL, F.SA_BF16, 64, 0.1
    a.batch, a.heads_q, a.heads_kv, a.seq, a.head_dim = 1, 32, 8, 131072, 128
    a.n_sink, a.n_local, a.ratio_num, a.ratio_den, a.kmax = 1, 4, 5, 100, 107
    assert lib.sa_estimate_topk_workspace_bytes(C.byref(a), C.byref(n)) == 2      # largest row keeps 5 + 103
    a.kmax = 108
    assert lib.sa_estimate_topk_workspace_bytes(C.byref(a), C.byref(n)) == 0 and n.value > 0
    a.pooled_q = a.pooled_k = 4096
    assert lib.sa_estimate_topk_workspace_bytes(C.byref(a), C.byref(n)) == 0 and n.value == 0
    a.seq = 131072 * 2
    assert lib.sa_estimate_topk_workspace_bytes(C.byref(a), C.byref(n)) == 6      # above 2048 blocks
    a.seq = 131072
    a.kind = F.SA_EST_INDEXER
    assert lib.sa_estimate_topk_workspace_bytes(C.byref(a), C.byref(n)) == 6
    c = F.EstimateTopkArgs()                                                     # centroid kind
    c.q = c.k_ptr = c.idx = c.cnt = 256
    c.kind, c.dtype, c.scale, c.k, c.kmax = F.SA_EST_CENTROID, F.SA_BF16, 0.1, 64, 64
    c.heads_q, c.heads_kv, c.seq, c.head_dim, c.n_centroids = 32, 8, 8, 128, 256
    assert lib.sa_estimate_topk_workspace_bytes(C.byref(c), C.byref(n)) == 0 and n.value == 0
    c.kmax = 63
    assert lib.sa_estimate_topk_workspace_bytes(C.byref(c), C.byref(n)) == 2
    c.kmax, c.n_centroids = 64, 2000
    assert lib.sa_estimate_topk_workspace_bytes(C.byref(c), C.byref(n)) == 2
    c.n_centroids = 1025                                                         # one past the cap
    assert lib.sa_estimate_topk_workspace_bytes(C.byref(c), C.byref(n)) == 2
    c.n_centroids = 1024                                                         # the cap itself
    assert lib.sa_estimate_topk_workspace_bytes(C.byref(c), C.byref(n)) == 0
    c.n_centroids, c.heads_q = 256, 80                                           # 10 query heads per KV head
    assert lib.sa_estimate_topk_workspace_bytes(C.byref(c), C.byref(n)) == 6
    c.heads_q, c.n_sink = 32, 1
    assert lib.sa_estimate_topk_workspace_bytes(C.byref(c), C.byref(n)) == 6
    c.n_sink, c.mass, c.k_min = 0, 0.5, 1                                        # adaptive budget
    assert lib.sa_estimate_topk_workspace_bytes(C.byref(c), C.byref(n)) == 0 and n.value == 0
    c.mass = 1.5
    assert lib.sa_estimate_topk_workspace_bytes(C.byref(c), C.byref(n)) == 8
    c.mass, c.k_min = 0.5, 65                                                   # above k
    assert lib.sa_estimate_topk_workspace_bytes(C.byref(c), C.byref(n)) == 8
    c.mass, c.k_min = 0.0, 0
    a.kind = F.SA_EST_BLOCK_MEANPOOL
    a.n_local = -1
    assert lib.sa_estimate_topk_workspace_bytes(C.byref(a), C.byref(n)) == 8


def test_indexer_topk_argument_errors(lib):
    from dynamic_sparse_attention_pool_amd import _ffi as F
    a = F.IndexerTopkArgs()
    n = C.c_size_t(0)
    assert lib.sa_indexer_topk_workspace_bytes(None, C.byref(n)) == 1
    a.seq_k = 131072
    assert lib.sa_indexer_topk_workspace_bytes(C.byref(a), C.byref(n)) == 0 and n.value == 0   # no queries
    assert lib.sa_indexer_topk(C.byref(a), None, 0, None) == 0
    a.seq_q, a.q_pos0, a.heads, a.head_dim, a.k, a.kmax = 4096, 126976, 64, 64, 2048, 2048
    assert lib.sa_indexer_topk_workspace_bytes(C.byref(a), C.byref(n)) == 1                    # NULL pointers
    a.q = a.k_ptr = a.weights = a.idx = a.cnt = 256
    assert lib.sa_indexer_topk_workspace_bytes(C.byref(a), C.byref(n)) == 0
    # sampled scores [T, N/16], thresholds, run counts, and runs of 2k + 128 per chunk
    assert n.value >= 4096 * (8192 + 1 + 16 + 2 * 10240) * 4
    assert lib.sa_indexer_topk(C.byref(a), None, 0, None) == 5                                 # no workspace
    assert lib.sa_indexer_topk(C.byref(a), C.c_void_p(4096), n.value - 1, None) == 5
    a.heads = 16
    assert lib.sa_indexer_topk_workspace_bytes(C.byref(a), C.byref(n)) == 6
    a.heads, a.head_dim = 32, 128
    assert lib.sa_indexer_topk_workspace_bytes(C.byref(a), C.byref(n)) == 6
    a.head_dim, a.k = 64, 4096
    assert lib.sa_indexer_topk_workspace_bytes(C.byref(a), C.byref(n)) == 8
    a.k = 0
    assert lib.sa_indexer_topk_workspace_bytes(C.byref(a), C.byref(n)) == 8
    a.k, a.kmax = 2048, 2047
    assert lib.sa_indexer_topk_workspace_bytes(C.byref(a), C.byref(n)) == 2
    a.seq_k, a.q_pos0, a.seq_q = 1000, 0, 1000                                                 # rows of 1..1000 keys
    assert lib.sa_indexer_topk_workspace_bytes(C.byref(a), C.byref(n)) == 0
    # no sampled scores (every row keeps all its keys): thresholds, run counts, runs of 8192 + 128 pairs
    assert n.value == 4096 + 4096 + 1000 * (8192 + 128) * 8
    a.kmax = 999
    assert lib.sa_indexer_topk_workspace_bytes(C.byref(a), C.byref(n)) == 2
    a.kmax, a.q_pos0 = 1000, -1
    assert lib.sa_indexer_topk_workspace_bytes(C.byref(a), C.byref(n)) == 8
    a.q_pos0, a.q = 0, 258
    assert lib.sa_indexer_topk_workspace_bytes(C.byref(a), C.byref(n)) == 4


def test_estimate_and_gather_argument_errors(lib):
    from dynamic_sparse_attention_pool_amd import _ffi as F
    e = F.EstimateArgs()
    e.q = e.k = e.scores = 256
    e.kind, e.dtype, e.batch, e.heads_q, e.heads_kv, e.seq_q, e.seq_k, e.head_dim = 0, F.SA_BF16, 1, 4, 2, 128, 128, 128
    e.block_size, e.scale = 32, 0.1
    assert lib.sa_estimate(C.byref(e), None, 0, None) == 6
    e.block_size = 64
    n = C.c_size_t(0)
    assert lib.sa_estimate_workspace_bytes(C.byref(e), C.byref(n)) == 0
    assert n.value == 2 * 1 * 4 * 128 * 4 + 2 * 1 * 2 * 128 * 4 or n.value >= (4 + 2) * 2 * 128 * 4
    assert lib.sa_estimate(C.byref(e), None, 0, None) == 5           # workspace missing
    e.kind = 3
    e.head_dim = 32
    e.weights = 256
    assert lib.sa_estimate(C.byref(e), None, 0, None) == 6
    e.head_dim, e.heads_kv, e.heads_q = 64, 1, 72                     # more than 64 indexer heads
    assert lib.sa_estimate(C.byref(e), None, 0, None) == 6
    e.heads_q = 20                                                    # not a multiple of 8
    assert lib.sa_estimate(C.byref(e), None, 0, None) == 6
    e.kind = 9
    assert lib.sa_estimate(C.byref(e), None, 0, None) == 8
    g = F.GatherArgs()
    g.q = g.k = g.v = g.out = 256
    g.dtype, g.out_dtype, g.head_dim, g.n_q, g.heads_q, g.heads_kv, g.n_ctx, g.scale = F.SA_BF16, F.SA_F32, 128, 8, 32, 8, 1024, 0.1
    g.mode = F.SA_GATHER_CLUSTER
    assert lib.sa_gather_decode(C.byref(g), None, 0, None) == 1      # cluster tables missing
    g.cluster_ptr = g.sel = 256
    g.n_clusters, g.n_sel = 16, 4
    g.n_q = 32                                                        # 32*4 queries per KV head > 64
    assert lib.sa_gather_decode(C.byref(g), None, 0, None) == 6
    g.n_q = 8
    g.q_pos = 256                                                     # a causal bound needs the pack's perm
    assert lib.sa_gather_decode(C.byref(g), None, 0, None) == 1
    g.mode = F.SA_GATHER_TOKEN
    g.tok_idx, g.n_tok, g.heads_kv = 256, 64, 4
    g.tok_per_head = 2                                                # neither shared (0) nor per head (1)
    assert lib.sa_gather_decode(C.byref(g), None, 0, None) == 8


def test_peak_probes_reject_bad_arguments(lib):
    d = C.c_double(0)
    assert lib.sa_peak_mfma_bf16(None, 10, 4, C.byref(d), None) == 1
    assert lib.sa_peak_mfma_bf16(256, 10, 6, C.byref(d), None) == 1   # waves per CU not a multiple of 4
    assert lib.sa_peak_read(None, 1 << 20, 1, 256, C.byref(d), None) == 1
    assert lib.sa_peak_read(264, 1 << 20, 1, 256, C.byref(d), None) == 1   # not 16-byte aligned


def test_static_decode_rejects_oversized_scratch(lib):
    """sa_gather_decode_static checks, before any launch, that the cluster
    partials fit its static scratch (64 KV heads x 2^20 keys need ~1.1 GB)."""
    from dynamic_sparse_attention_pool_amd import _ffi as F
    g = F.GatherArgs()
    g.q = g.k = g.v = g.out = g.cluster_ptr = g.sel = 256
    g.mode, g.dtype, g.out_dtype, g.head_dim, g.scale = F.SA_GATHER_CLUSTER, F.SA_BF16, F.SA_F32, 128, 0.1
    g.n_q, g.heads_q, g.heads_kv, g.n_ctx, g.n_clusters, g.n_sel = 1, 64, 64, 1 << 20, 256, 8
    n = C.c_size_t(0)
    assert lib.sa_gather_decode_workspace_bytes(C.byref(g), C.byref(n)) == 0
    assert n.value > F.STATIC_SCRATCH_BYTES
    assert lib.sa_gather_decode_static(C.byref(g), None) == 6
    assert "static buffer holds" in _err(lib)
    g.n_q = 0
    assert lib.sa_gather_decode_static(C.byref(g), None) == 2   # argument errors as in sa_gather_decode


def test_binding_rejects_inconsistent_tensors(lib):
    """Every wrapper checks dtype, shape and device of each tensor against
    the sizes it passes to the library, before any launch (CPU tensors here,
    so a consistent call would stop at the device check instead)."""
    import torch as tt

    import dynamic_sparse_attention_pool_amd as sa
    bf, f32, i32 = tt.bfloat16, tt.float32, tt.int32
    q = tt.zeros((1, 4, 256, 128), dtype=bf)
    k = tt.zeros((1, 2, 256, 128), dtype=bf)
    out = tt.zeros((1, 4, 256, 128), dtype=f32)
    idx, cnt = tt.zeros((1, 4, 4, 3), dtype=i32), tt.zeros((1, 4, 4), dtype=i32)
    cases = [
        (lambda: sa.sa_block_sparse_fwd(q, k.float(), k, out, block_idx=idx, block_cnt=cnt), "k"),
        (lambda: sa.sa_block_sparse_fwd(q, k[:, :, :128], k, out, block_idx=idx, block_cnt=cnt), "k"),
        (lambda: sa.sa_block_sparse_fwd(q, k, k[:, :1], out, block_idx=idx, block_cnt=cnt), "v"),
        (lambda: sa.sa_block_sparse_fwd(q, k, k, out[:, :2], block_idx=idx, block_cnt=cnt), "out"),
        (lambda: sa.sa_block_sparse_fwd(q, k, k, out, block_idx=idx.float(), block_cnt=cnt), "block_idx"),
        (lambda: sa.sa_block_sparse_fwd(q, k, k, out, block_idx=idx, block_cnt=cnt[:, :, :2]), "block_cnt"),
        (lambda: sa.sa_estimate(sa.BLOCK_MEANPOOL, q, k, tt.zeros((1, 4, 4, 3), dtype=f32)), "scores"),
        (lambda: sa.sa_estimate(sa.BLOCK_MEANPOOL, q, k, tt.zeros((1, 4, 4, 4), dtype=bf)), "scores"),
        (lambda: sa.sa_select_topk(tt.zeros((8, 16), dtype=f32), tt.zeros((7, 2), dtype=i32),
                                   tt.zeros(8, dtype=i32), k=2), "idx"),
        (lambda: sa.sa_select_topk(tt.zeros((8, 16), dtype=f32), tt.zeros((8, 2), dtype=i32),
                                   tt.zeros(8, dtype=f32), k=2), "cnt"),
        (lambda: sa.sa_gather_decode(tt.zeros((2, 32, 128), dtype=bf), tt.zeros((8, 64, 128), dtype=bf),
                                     tt.zeros((8, 64, 64), dtype=bf), tt.zeros((2, 32, 128), dtype=f32),
                                     tok_idx=tt.zeros((2, 16), dtype=i32)), "v"),
        (lambda: sa.sa_gather_decode(tt.zeros((2, 32, 128), dtype=bf), tt.zeros((8, 64, 128), dtype=bf),
                                     tt.zeros((8, 64, 128), dtype=bf), tt.zeros((2, 32, 128), dtype=f32),
                                     tok_idx=tt.zeros((2, 31, 16), dtype=i32)), "tok_idx"),
        (lambda: sa.sa_indexer_topk(tt.zeros((4, 32, 64), dtype=bf), tt.zeros((100, 64), dtype=bf),
                                    tt.zeros((4, 8), dtype=i32), tt.zeros(4, dtype=i32),
                                    weights=tt.zeros(16, dtype=f32), q_pos0=96, k=8), "weights"),
    ]
    for fn, name in cases:
        with pytest.raises(ValueError, match=name):
            fn()


def test_missing_library_fails_loudly(monkeypatch):
    """No CPU fallback: without libsa.so every entry point raises."""
    import numpy as np
    import torch as tt

    import dynamic_sparse_attention_pool_amd as sa
    from dynamic_sparse_attention_pool_amd import _ffi
    monkeypatch.setattr(_ffi, "LIB_PATH", "/nonexistent/libsa.so")
    monkeypatch.setattr(_ffi, "_lib", None)
    with pytest.raises(ImportError, match="no CPU fallback"):
        _ffi.load()
    s = tt.from_numpy(np.zeros((2, 8), np.float32))
    idx, cnt = tt.zeros((2, 2), dtype=tt.int32), tt.zeros(2, dtype=tt.int32)
    with pytest.raises(ImportError):
        sa.sa_select_topk(s, idx, cnt, k=2)
