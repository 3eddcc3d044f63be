"""The allocation-free clustered decode, sa_gather_decode_static (scratch in
the library's static device array), against sa_gather_decode with a
workspace: two calls in a row, the second with a smaller input, each
bit-identical in output and lse."""
import math

import numpy as np
import pytest

import oracle
import workloads as W
from gpu_helpers import dev_bf16, dev_i32, host, torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sa():
    import dynamic_sparse_attention_pool_amd as m
    m.load()
    return m


def decode_case(sa, seed, T, Hq, Hkv, N, C, ks):
    t = torch()
    d = 128
    print(f"static decode case T={T} Hq={Hq} Hkv={Hkv} N={N} C={C} k={ks}", flush=True)
    dec = W.decode_clustered(seed, T, Hq, Hkv, N, d, C)
    ptr = t.empty((Hkv, C + 1), dtype=t.int32, device="cuda:0")
    perm = t.empty((Hkv, N), dtype=t.int32, device="cuda:0")
    kp = t.empty((Hkv, N, d), dtype=t.bfloat16, device="cuda:0")
    vp = t.empty_like(kp)
    sa.sa_cluster_pack(dev_i32(dec.labels), ptr, perm, C, k=dev_bf16(dec.k), v=dev_bf16(dec.v), k_packed=kp,
                       v_packed=vp)
    scale = 1 / math.sqrt(d)
    sel = oracle.cluster_select(oracle.centroid_scores(W.bf16_to_f32(dec.q), dec.centroids, scale), ks)
    sel_d = dev_i32(np.array([[s for s in row] for row in sel], np.int32))
    q = dev_bf16(dec.q)
    outs = []
    for fn in (sa.sa_gather_decode, sa.sa_gather_decode_static):
        out = t.full((T, Hq, d), 7.0, dtype=t.float32, device="cuda:0")
        lse = t.full((T, Hq), 7.0, dtype=t.float32, device="cuda:0")
        fn(q, kp, vp, out, cluster_ptr=ptr, sel=sel_d, lse=lse)
        t.cuda.synchronize()
        outs.append((host(out), host(lse)))
    return outs


def test_static_decode_equals_workspace_decode_twice(sa):
    # the decode workload's full size, then a smaller call reusing the same scratch
    for case in [(81, 8, 32, 8, 65536, 256, 64), (82, 3, 8, 2, 8192, 64, 16)]:
        (o_ws, l_ws), (o_st, l_st) = decode_case(sa, *case)
        assert np.array_equal(o_ws, o_st) and np.array_equal(l_ws, l_st)
        assert np.all(np.isfinite(o_st))
