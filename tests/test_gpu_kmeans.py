"""GPU parity of the offline k-means (sa_kmeans) against the CPU oracle.

Labels are integers decided by floating point (fp32 |mu|^2 - 2 k.mu on the GPU,
fp64 distances in the oracle).  For fp32 keys the dot product is 128 fp32
FMAs; for bf16 keys it is 3 x 128 exact products (the centroid split into
three bf16 parts, which sum to it within about 2^-26) accumulated in fp32,
at most 384 * 2^-24 |k||mu| <= 1.2e-5 (|k|^2 + |mu|^2); the 128-term norm
adds at most 7.6e-6 |mu|^2.  So MARGIN_REL = 2e-5 of |k|^2 + |mu|^2 bounds
the GPU's distance error.  Keys whose oracle margin (second-nearest minus nearest squared
distance) exceeds it must get the oracle's label; any other key may take a
centroid whose oracle distance is within that tolerance of the nearest.
Several iterations are compared only on trajectories where every key of every
iteration clears the margin, so both sides visit the same tables.  Centroids
are compared where the cluster's members are the oracle's."""
import math

import numpy as np
import pytest

import oracle
import workloads as W
from gpu_helpers import dev_bf16, dev_f32, host, torch

pytestmark = pytest.mark.gpu

MARGIN_REL = 2e-5


@pytest.fixture(scope="module")
def sa():
    import dynamic_sparse_attention_pool_amd as m
    m.load()
    return m


def run_kmeans(sa, k_dev, init, iters, want_pack=True):
    t = torch()
    Hkv, N, _ = k_dev.shape
    C = init.shape[1]
    cent = dev_f32(init)
    labels = t.empty((Hkv, N), dtype=t.int32, device="cuda:0")
    ptr = t.empty((Hkv, C + 1), dtype=t.int32, device="cuda:0") if want_pack else None
    perm = t.empty((Hkv, N), dtype=t.int32, device="cuda:0") if want_pack else None
    sa.sa_kmeans(k_dev, cent, labels, iters=iters, cluster_ptr=ptr, perm=perm)
    t.cuda.synchronize()
    return host(cent), host(labels), (host(ptr) if want_pack else None), (host(perm) if want_pack else None)


def check_head(X, init, iters, cent, labels, exact_frac=0.99):
    """Compare one KV head with the oracle run of the same iterations."""
    mu, lab, margins = oracle.kmeans(X, init, iters)
    X64 = np.asarray(X, np.float64)
    table = np.asarray(init if iters == 1 else mu, np.float64)   # the table of the last assignment (or close to it)
    scale = (X64 ** 2).sum(axis=1) + (table[lab] ** 2).sum(axis=1)
    if iters > 1:   # the same tables at every step
        assert np.all(margins[:-1] > MARGIN_REL * scale), "trajectory not certified"
    sure = margins[-1] > MARGIN_REL * scale
    assert np.array_equal(labels[sure], lab[sure])
    assert sure.mean() >= exact_frac
    if iters == 1 and not sure.all():
        # the last assignment used the initial table: a GPU label is valid when its
        # distance is within the tolerance of the nearest
        _, d2 = oracle.kmeans_assign(X, init)
        rows = np.nonzero(~sure)[0]
        got = d2[rows, labels[rows]]
        assert np.all(got - d2[rows].min(axis=1) <= MARGIN_REL * scale[rows])
    same = [c for c in range(mu.shape[0]) if np.array_equal(np.nonzero(labels == c)[0], np.nonzero(lab == c)[0])]
    assert len(same) >= exact_frac * mu.shape[0]
    err = np.abs(cent[same] - mu[same])
    assert float(err.max()) <= 1e-5 * max(1.0, float(np.abs(mu[same]).max()))
    return mu, lab


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("f32", 128), ("f32", 64)])
def test_kmeans_separated_mixture(sa, dtype, d):
    """Keys drawn around C means; the table starts near the means: every key is
    far from any other centroid, so all labels and centroids must match."""
    Hkv, N, C, iters = 2, 5003, 20, 3
    inp = W.decode_clustered(71, 1, Hkv, Hkv, N, d, C)
    kf = W.bf16_to_f32(inp.k)
    init = (inp.centroids + 0.05 * W.normal(71, inp.centroids.shape, 99)).astype(np.float32)
    k_dev = dev_bf16(inp.k) if dtype == "bf16" else dev_f32(kf)
    cent, labels, ptr, perm = run_kmeans(sa, k_dev, init, iters)
    labs = []
    for g in range(Hkv):
        mu, lab = check_head(kf[g], init[g], iters, cent[g], labels[g], exact_frac=1.0)
        assert np.array_equal(lab, inp.labels[g])              # the generating clusters
        labs.append(lab)
    wptr, wperm = oracle.cluster_pack(np.stack(labs), C)       # the oracle's own labels
    assert np.array_equal(ptr, wptr) and np.array_equal(perm, wperm)


def test_kmeans_generic_keys_forgy_init(sa):
    """N(0,1) keys with no cluster structure, table started from sampled keys,
    one step (several steps are not certified on such data)."""
    Hkv, N, C, d = 2, 3000, 37, 128
    k = W.f32_to_bf16(W.normal(72, (Hkv, N, d), 0))
    init = W.kmeans_init(72, k, C)
    cent, labels, _, _ = run_kmeans(sa, dev_bf16(k), init, 1, want_pack=False)
    kf = W.bf16_to_f32(k)
    for g in range(Hkv):
        check_head(kf[g], init[g], 1, cent[g], labels[g])


def test_kmeans_empty_cluster_keeps_centroid_and_ties_go_low(sa):
    Hkv, N, d = 1, 700, 64
    k = W.f32_to_bf16(W.normal(73, (Hkv, N, d), 0))
    kf = W.bf16_to_f32(k)
    init = np.stack([kf[0, 0], kf[0, 0], kf[0, 5], np.full(d, 1e4, np.float32)])[None].astype(np.float32)
    cent, labels, ptr, _ = run_kmeans(sa, dev_bf16(k), init, 1)
    assert not np.any(labels == 1)                  # equal centroids: the lower index takes the keys
    assert not np.any(labels == 3)                  # far centroid: no member
    assert np.array_equal(cent[0, 1], init[0, 1]) and np.array_equal(cent[0, 3], init[0, 3])
    assert ptr[0, 2] - ptr[0, 1] == 0 and ptr[0, 4] - ptr[0, 3] == 0
    check_head(kf[0], init[0], 1, cent[0], labels[0], exact_frac=0.0)   # the tie is deliberate


def test_kmeans_full_context_and_decode_from_built_table(sa):
    """The 65536-key context of the clustered decode (8 KV heads, 256 clusters).
    One step from sampled keys, checked on two heads; three steps from the
    exact cluster means, which recover the generating clusters on every head;
    then the decode runs on that built table and its labels."""
    from dynamic_sparse_attention_pool_amd.pipelines import ClusterDecode
    seed = W.CONFIG_SEEDS[4]
    T, Hq, Hkv, N, d, C = 8, 32, 8, 65536, 128, 256
    inp = W.decode_clustered(seed, T, Hq, Hkv, N, d, C)
    kf = W.bf16_to_f32(inp.k)
    k_dev = dev_bf16(inp.k)
    init = W.kmeans_init(seed, inp.k, C)
    cent, labels, _, _ = run_kmeans(sa, k_dev, init, 1, want_pack=False)
    for g in (0, 5):
        check_head(kf[g], init[g], 1, cent[g], labels[g])
    cent, labels, ptr, perm = run_kmeans(sa, k_dev, inp.centroids, 3)
    assert np.array_equal(labels, inp.labels)
    built = {}
    for g in (0, 5):
        built[g] = check_head(kf[g], inp.centroids[g], 3, cent[g], labels[g], exact_frac=1.0)
        wptr, wperm = oracle.cluster_pack(built[g][1][None], C)
        assert np.array_equal(ptr[g], wptr[0]) and np.array_equal(perm[g], wperm[0])
    dc = ClusterDecode(dev_bf16(inp.q), k_dev, dev_bf16(inp.v), torch().from_numpy(labels).cuda(),
                       dev_f32(cent), n_sel=64)
    dc.step()
    torch().cuda.synchronize()
    scale = 1 / math.sqrt(d)
    none = np.zeros(0, np.int64)
    got_sel, got_out = host(dc.sel), host(dc.out)
    checked = 0
    for g, (mu, lab) in built.items():
        heads = [h for h in range(Hq) if h * Hkv // Hq == g]
        s = oracle.centroid_scores(W.bf16_to_f32(inp.q[:, heads]), mu[None], scale)
        for t in range(T):
            for j, h in enumerate(heads):
                if not oracle.certified_row(s[t, j], 64, none):
                    continue
                sel = oracle.topk_row(s[t, j], 64, none)
                assert np.array_equal(got_sel[t, h], sel), (t, h)
                keys = np.nonzero(np.isin(lab, sel))[0]
                o, _ = oracle.attend_rows(W.bf16_to_f32(inp.q[t, h])[None], kf[g], W.bf16_to_f32(inp.v[g]), keys,
                                          scale)
                assert np.max(np.abs(got_out[t, h] - o[0])) <= 2e-2, (t, h)
                checked += 1
    assert checked >= 32
