"""Seeded synthetic inputs for the dynamic sparse attention path.

This module holds only input recipes: random draws, bf16 rounding and the
planted structure that gives certified selections.  It contains none of the
method's arithmetic (no pooling, scoring, selection or attention), so the CPU
oracle and the HIP path can both be fed from it without sharing any code.

Every array comes from a counter-addressed substream:
``numpy.random.SeedSequence(seed, spawn_key=(stream, *coords))`` driving PCG64.
A head, a query block or a redraw attempt can therefore be regenerated alone.

bf16 tensors are returned as ``uint16`` bit patterns (round-to-nearest-even
from float32).  ``bf16_to_f32`` widens them exactly.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

# stream identifiers of the substreams; a new recipe appends, never renumbers
S_Q, S_K, S_V, S_SHIFT_POS, S_SHIFT_U = 0, 1, 2, 3, 4
S_LABELS, S_KMEANS, S_VMEANS, S_DECQ, S_IDXW = 5, 6, 7, 8, 9
S_IDXQ, S_IDXK, S_LAYER, S_REDRAW_QB, S_REDRAW_DECQ = 10, 11, 12, 13, 14
S_PLANT, S_TOPK, S_KMINIT = 15, 16, 17

CONFIG_SEEDS = {1: 1, 2: 2, 3: 3, 4: 4, 5: 5}


def rng(seed: int, *path: int) -> np.random.Generator:
    """Independent generator for the substream ``path`` of ``seed``."""
    return np.random.Generator(
        np.random.PCG64(np.random.SeedSequence(seed, spawn_key=tuple(int(p) for p in path))))


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit pattern (uint16), round to nearest, ties to even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit pattern (uint16) -> float32, exact."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal(seed: int, shape, *path: int) -> np.ndarray:
    return rng(seed, *path).standard_normal(shape, dtype=np.float32)


# ---------------------------------------------------------------- prefill
@dataclass
class PrefillInputs:
    """Q [B,Hq,N,d], K and V [B,Hkv,N,d]; bf16 bits (uint16) or float32."""
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    dtype: str                 # "f32" or "bf16"
    shift_pos: np.ndarray      # key positions carrying the +key_shift*u offset
    u: np.ndarray | None       # the shared unit vector (float32) or None

    def f32(self, name: str) -> np.ndarray:
        a = getattr(self, name)
        return a if self.dtype == "f32" else bf16_to_f32(a)


def prefill_fp32(seed: int, B: int, H: int, N: int, d: int) -> PrefillInputs:
    """i.i.d. N(0,1) fp32 Q/K/V, one substream per (tensor, batch, head)."""
    q = np.empty((B, H, N, d), np.float32)
    k = np.empty_like(q)
    v = np.empty_like(q)
    for b in range(B):
        for h in range(H):
            q[b, h] = normal(seed, (N, d), S_Q, b, h)
            k[b, h] = normal(seed, (N, d), S_K, b, h)
            v[b, h] = normal(seed, (N, d), S_V, b, h)
    return PrefillInputs(q, k, v, "f32", np.zeros(0, np.int64), None)


def shift_vector(seed: int, d: int) -> np.ndarray:
    u = rng(seed, S_SHIFT_U).standard_normal(d)
    return (u / np.linalg.norm(u)).astype(np.float32)


def shift_positions(seed: int, N: int, frac: float) -> np.ndarray:
    n = int(math.floor(frac * N))
    return np.sort(rng(seed, S_SHIFT_POS).choice(N, size=n, replace=False)).astype(np.int64)


def prefill_query_head(seed: int, b: int, h: int, N: int, d: int, u, q_shift: float) -> np.ndarray:
    q = normal(seed, (N, d), S_Q, b, h)
    if u is not None:
        q += np.float32(q_shift) * u
    return f32_to_bf16(q)


def prefill_kv_head(seed: int, b: int, g: int, N: int, d: int, u, pos, k_shift: float):
    k = normal(seed, (N, d), S_K, b, g)
    if u is not None and len(pos):
        k[pos] += np.float32(k_shift) * u
    v = normal(seed, (N, d), S_V, b, g)
    return f32_to_bf16(k), f32_to_bf16(v)


def prefill_bf16(seed: int, B: int, Hq: int, Hkv: int, N: int, d: int,
                 shift_frac: float = 0.01, k_shift: float = 3.0, q_shift: float = 1.0,
                 heads=None) -> PrefillInputs:
    """GQA prefill layer: N(0,1) Q/K/V; floor(shift_frac*N) seeded key positions
    get +k_shift*u (the same positions and u for every KV head); every query
    gets +q_shift*u.  Rounded to bf16.  ``heads`` restricts the query heads
    generated (others are left zero) to build a bounded sample cheaply."""
    u = shift_vector(seed, d) if shift_frac > 0 else None
    pos = shift_positions(seed, N, shift_frac) if shift_frac > 0 else np.zeros(0, np.int64)
    q = np.zeros((B, Hq, N, d), np.uint16)
    k = np.empty((B, Hkv, N, d), np.uint16)
    v = np.empty_like(k)
    hs = range(Hq) if heads is None else heads
    for b in range(B):
        for h in hs:
            q[b, h] = prefill_query_head(seed, b, h, N, d, u, q_shift)
        for g in range(Hkv):
            k[b, g], v[b, g] = prefill_kv_head(seed, b, g, N, d, u, pos, k_shift)
    return PrefillInputs(q, k, v, "bf16", pos, u)


def redraw_query_block(seed: int, b: int, h: int, i: int, attempt: int, bs: int, d: int,
                       u, q_shift: float, dtype: str) -> np.ndarray:
    """Fresh rows for query block i of head h (same law as the original rows);
    used to redraw a block whose selection is not certified."""
    x = normal(seed, (bs, d), S_REDRAW_QB, b, h, i, attempt)
    if u is not None:
        x += np.float32(q_shift) * u
    return x if dtype == "f32" else f32_to_bf16(x)


def integer_bf16(seed: int, shape, lo: int, hi: int, *path: int) -> np.ndarray:
    """bf16 bits of integers drawn uniformly from [lo, hi]: sums and products of
    such values stay exact in fp32 at the sizes used by the exact tests."""
    x = rng(seed, *path).integers(lo, hi + 1, size=shape).astype(np.float32)
    return f32_to_bf16(x)


# ---------------------------------------------------------------- vertical-slash planting
def plant_vertical_slash(inp: PrefillInputs, seed: int, n_cols: int, n_offs: int,
                         beta_v: float, beta_s: float, last_q: int = 64):
    """Planted vertical lines and slash lines on a bf16 prefill input.

    Per KV head g: n_cols seeded key columns get +beta_v*u (queries already
    carry +u), and n_offs seeded diagonal offsets o get key r-o pushed toward
    the normalised mean of the group's queries at row r, scaled by beta_s, for
    the last ``last_q`` rows r.  Returns (inputs, cols[Hkv], offs[Hkv])."""
    B, Hq, N, d = inp.q.shape
    Hkv = inp.k.shape[1]
    grp = Hq // Hkv
    k = bf16_to_f32(inp.k).copy()
    qf = bf16_to_f32(inp.q)
    cols_all, offs_all = [], []
    for b in range(B):
        for g in range(Hkv):
            r = rng(seed, S_PLANT, b, g)
            cols = np.sort(r.choice(N - last_q, size=n_cols, replace=False))
            offs = np.sort(r.choice(np.arange(1, N - last_q), size=n_offs, replace=False))
            k[b, g, cols] += np.float32(beta_v) * inp.u
            qg = qf[b, g * grp:(g + 1) * grp, N - last_q:].mean(axis=0)
            qg /= np.linalg.norm(qg, axis=1, keepdims=True)
            for o in offs:
                rows = np.arange(N - last_q, N)
                k[b, g, rows - o] += np.float32(beta_s) * qg
            cols_all.append(cols)
            offs_all.append(offs)
    out = PrefillInputs(inp.q, f32_to_bf16(k), inp.v, "bf16", inp.shift_pos, inp.u)
    return out, cols_all, offs_all


# ---------------------------------------------------------------- clustered decode
@dataclass
class DecodeInputs:
    q: np.ndarray          # [T,Hq,d] bf16 bits
    k: np.ndarray          # [Hkv,Nctx,d] bf16 bits (context order)
    v: np.ndarray          # [Hkv,Nctx,d] bf16 bits
    labels: np.ndarray     # [Hkv,Nctx] int32 mixture component of each key
    centroids: np.ndarray  # [Hkv,C,d] float32: the component means
    vmeans: np.ndarray     # [Hkv,C,d] float32: value means


def decode_clustered(seed: int, T: int, Hq: int, Hkv: int, Nctx: int, d: int, C: int,
                     sigma: float = 0.3) -> DecodeInputs:
    """Fixed context drawn from a C-component Gaussian mixture per KV head:
    key means and value means N(0,1), uniform labels, within-cluster sigma.
    Queries are N(0,I).  The centroid table is the exact float32 key means."""
    k = np.empty((Hkv, Nctx, d), np.uint16)
    v = np.empty_like(k)
    labels = np.empty((Hkv, Nctx), np.int32)
    mu = np.empty((Hkv, C, d), np.float32)
    nu = np.empty_like(mu)
    for g in range(Hkv):
        mu[g] = normal(seed, (C, d), S_KMEANS, g)
        nu[g] = normal(seed, (C, d), S_VMEANS, g)
        labels[g] = rng(seed, S_LABELS, g).integers(0, C, size=Nctx)
        zk = normal(seed, (Nctx, d), S_K, g)
        zv = normal(seed, (Nctx, d), S_V, g)
        k[g] = f32_to_bf16(mu[g][labels[g]] + np.float32(sigma) * zk)
        v[g] = f32_to_bf16(nu[g][labels[g]] + np.float32(sigma) * zv)
    q = np.empty((T, Hq, d), np.uint16)
    for t in range(T):
        q[t] = f32_to_bf16(normal(seed, (Hq, d), S_DECQ, t))
    return DecodeInputs(q, k, v, labels, mu, nu)


def kmeans_init(seed: int, k_bits: np.ndarray, C: int) -> np.ndarray:
    """Initial centroid table [Hkv, C, d] float32: C distinct keys per KV head,
    drawn without replacement from a seeded substream (the keys' own bf16
    values, widened exactly)."""
    Hkv, N, d = k_bits.shape
    out = np.empty((Hkv, C, d), np.float32)
    for g in range(Hkv):
        pick = rng(seed, S_KMINIT, g).choice(N, size=C, replace=False)
        out[g] = bf16_to_f32(k_bits[g][np.sort(pick)])
    return out


def redraw_decode_query(seed: int, t: int, h: int, attempt: int, d: int) -> np.ndarray:
    return f32_to_bf16(normal(seed, (d,), S_REDRAW_DECQ, t, h, attempt))


# ---------------------------------------------------------------- indexer + layers
@dataclass
class IndexerInputs:
    qi: np.ndarray      # [T,Hi,di] bf16 bits
    ki: np.ndarray      # [Nctx,di] bf16 bits
    w: np.ndarray       # [Hi] float32, U(0,1)
    pos0: int           # absolute position of query 0


def indexer_random(seed: int, T: int, Hi: int, di: int, Nctx: int) -> IndexerInputs:
    qi = np.empty((T, Hi, di), np.uint16)
    chunk = 512
    for c0 in range(0, T, chunk):
        c1 = min(T, c0 + chunk)
        qi[c0:c1] = f32_to_bf16(normal(seed, (c1 - c0, Hi, di), S_IDXQ, c0))
    ki = np.empty((Nctx, di), np.uint16)
    chunk = 16384
    for c0 in range(0, Nctx, chunk):
        c1 = min(Nctx, c0 + chunk)
        ki[c0:c1] = f32_to_bf16(normal(seed, (c1 - c0, di), S_IDXK, c0))
    w = rng(seed, S_IDXW).uniform(0.0, 1.0, size=Hi).astype(np.float32)
    return IndexerInputs(qi, ki, w, Nctx - T)


def indexer_planted(seed: int, T: int, Hi: int, di: int, Nctx: int, k_sel: int,
                    n_dir: int = 16, hot: float = 4.0, noise: float = 0.1) -> IndexerInputs:
    """Planted indexer input with a wide score gap at the k-th key: n_dir
    orthogonal directions e_g (basis vectors); query t points along
    e_{t mod n_dir}; each direction owns a disjoint hot set of k_sel keys
    below the first query position with key = hot*e_g; all else is noise."""
    pos0 = Nctx - T
    assert n_dir * k_sel <= pos0 and n_dir <= di
    r = rng(seed, S_PLANT)
    hot_keys = r.choice(pos0, size=n_dir * k_sel, replace=False).reshape(n_dir, k_sel)
    ki = np.float32(noise) * normal(seed, (Nctx, di), S_IDXK, 0)
    for g in range(n_dir):
        ki[hot_keys[g], g] += np.float32(hot)
    qi = np.float32(noise) * normal(seed, (T, Hi, di), S_IDXQ, 0)
    for t in range(T):
        qi[t, :, t % n_dir] += np.float32(1.0)
    w = rng(seed, S_IDXW).uniform(0.0, 1.0, size=Hi).astype(np.float32)
    return IndexerInputs(f32_to_bf16(qi), f32_to_bf16(ki), w, pos0)


@dataclass
class LayerInputs:
    q: np.ndarray   # [T,Hq,d] bf16 bits
    k: np.ndarray   # [Hkv,Nctx,d] bf16 bits
    v: np.ndarray


def mqa_layer(seed: int, layer: int, T: int, Hq: int, Hkv: int, Nctx: int, d: int) -> LayerInputs:
    q = f32_to_bf16(normal(seed, (T, Hq, d), S_LAYER, layer, 0))
    k = np.empty((Hkv, Nctx, d), np.uint16)
    v = np.empty_like(k)
    for g in range(Hkv):
        k[g] = f32_to_bf16(normal(seed, (Nctx, d), S_LAYER, layer, 1, g))
        v[g] = f32_to_bf16(normal(seed, (Nctx, d), S_LAYER, layer, 2, g))
    return LayerInputs(q, k, v)


# ---------------------------------------------------------------- raw score rows
def score_rows(seed: int, R: int, n: int, kind: str = "normal", *path: int) -> np.ndarray:
    """float32 score rows for selection tests: 'normal' (continuous),
    'ties' (few distinct values, many exact ties, signed zeros included),
    'coarse' (normal values rounded to multiples of 1/16)."""
    r = rng(seed, S_TOPK, *path)
    if kind == "normal":
        return r.standard_normal((R, n), dtype=np.float32)
    if kind == "ties":
        vals = np.array([-2.0, -1.0, -0.0, 0.0, 0.5, 1.0, 3.0], np.float32)
        return vals[r.integers(0, len(vals), size=(R, n))]
    if kind == "coarse":  # normal values on a 1/16 grid: runs of equal keys around any threshold
        return (np.round(r.standard_normal((R, n), dtype=np.float32) * 16) / 16).astype(np.float32)
    raise ValueError(kind)
