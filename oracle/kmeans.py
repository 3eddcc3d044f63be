"""Offline clustering of the fixed context's keys (oracle; test infrastructure only).

Squeezed Attention page, §技术方案, offline stage: the keys of the fixed
context are clustered, each cluster gets a representative centroid, and each
key an index to its cluster.  The page names k-means; the reading taken here
is plain Lloyd iterations on squared Euclidean distance, per KV head, from a
caller-given initial centroid table:
  1. assign every key to its nearest centroid (ties -> lower cluster index);
  2. move every centroid to the mean of its keys (a cluster with no key keeps
     its previous centroid);
repeated ``iters`` times.  The result is the centroid table after the last
update and the labels of the last assignment, so each non-empty cluster's
centroid is exactly the mean of the keys labelled with it.
"""
from __future__ import annotations

import numpy as np


def assign(X: np.ndarray, mu: np.ndarray):
    """Labels [N] (nearest centroid) and the squared distances [N, C] (fp64),
    written as the expansion |x|^2 - 2 x.mu + |mu|^2 of |x - mu|^2 so that a
    full context (65536 keys x 256 centroids) takes one matrix product."""
    X = np.asarray(X, np.float64)
    mu = np.asarray(mu, np.float64)
    d2 = (X * X).sum(axis=1)[:, None] - 2.0 * (X @ mu.T) + (mu * mu).sum(axis=1)[None, :]
    return np.argmin(d2, axis=1), d2


def update(X: np.ndarray, labels: np.ndarray, mu: np.ndarray) -> np.ndarray:
    """Mean of each cluster's keys; empty clusters keep their centroid."""
    X = np.asarray(X, np.float64)
    new = np.asarray(mu, np.float64).copy()
    for c in range(new.shape[0]):
        members = X[labels == c]
        if members.shape[0]:
            new[c] = members.mean(axis=0)
    return new


def kmeans(X: np.ndarray, mu0: np.ndarray, iters: int):
    """(centroids [C, d], labels [N], margins [iters, N]) for one KV head.
    margins[t, n] = second-nearest minus nearest squared distance at step t
    (how far key n was from changing cluster)."""
    mu = np.asarray(mu0, np.float64)
    labels = np.zeros(np.asarray(X).shape[0], np.int64)
    margins = []
    for _ in range(iters):
        labels, d2 = assign(X, mu)
        part = np.partition(d2, 1, axis=1) if d2.shape[1] > 1 else np.concatenate([d2, d2 + np.inf], axis=1)
        margins.append(part[:, 1] - part[:, 0])
        mu = update(X, labels, mu)
    return mu, labels, np.array(margins)


def objective(X: np.ndarray, mu: np.ndarray, labels: np.ndarray) -> float:
    """Sum of squared distances of the keys to their centroids."""
    X = np.asarray(X, np.float64)
    return float(((X - np.asarray(mu, np.float64)[labels]) ** 2).sum())
