"""Oracle: Lloyd K-means over one KV head's prefill keys, and the CSR pack.

Test infrastructure only (see the package header).

Source: LouisKV note (papernotes.org), "Key designs" item 2 -- at prefill the
keys of the input are grouped with K-means and each cluster's centroid is the
mean of its keys; the centroid is the cluster's retrieval index. The edgentiq
blog ("Decoupled Fine-Grained Management", prefill stage) says the same.

Readings (the pages give no algorithmic detail beyond the above):

* distance is squared Euclidean (the centroid is an arithmetic mean, which is
  the minimiser of squared Euclidean error);
* init: centroid k starts as key ``init_idx[k]`` (distinct indices given as
  an input);
* exactly ``iters`` rounds of (assign to nearest centroid, then replace each
  centroid by the mean of its members); no early exit; the returned
  assignment is the last one and the returned centroids are its means;
* ties in the assignment go to the lowest centroid index;
* an empty cluster keeps its previous centroid and has size 0;
* ``mode="parity"`` measures distances to the centroid as the matrix cores
  see it: fp64 -> fp32 -> storage dtype (bf16 RNE, or fp32). ``mode="exact"``
  uses the fp64 centroid. Both compute distances in fp64.
"""
from __future__ import annotations

import numpy as np

from .precision import to_storage


def centroid_for_distance(c, mode: str, dtype: str) -> np.ndarray:
    if mode == "exact":
        return np.asarray(c, dtype=np.float64)
    if mode == "parity":
        return to_storage(c, dtype)
    raise ValueError(mode)


def sq_distances(keys, centroids) -> np.ndarray:
    """D[i, k] = ||x_i - c_k||^2 in fp64 (expanded with one matrix product)."""
    x = np.asarray(keys, dtype=np.float64)
    c = np.asarray(centroids, dtype=np.float64)
    xx = np.einsum("nd,nd->n", x, x)[:, None]
    cc = np.einsum("kd,kd->k", c, c)[None, :]
    return xx - 2.0 * (x @ c.T) + cc


def assign(keys, centroids) -> np.ndarray:
    """Nearest centroid of every key; the first (lowest) index wins ties."""
    return np.argmin(sq_distances(keys, centroids), axis=1).astype(np.int64)


def update(keys, labels, prev_centroids):
    """Each centroid becomes the mean of its members; empty ones keep the old value.

    Returns (centroids [C, d] fp64, counts [C] int64).
    """
    x = np.asarray(keys, dtype=np.float64)
    prev = np.asarray(prev_centroids, dtype=np.float64)
    C, d = prev.shape
    counts = np.bincount(labels, minlength=C)
    sums = np.zeros((C, d), dtype=np.float64)
    np.add.at(sums, labels, x)
    new = prev.copy()
    nz = counts > 0
    new[nz] = sums[nz] / counts[nz, None]
    return new, counts


def objective(keys, labels, centroids) -> float:
    """J = sum_i ||x_i - c_{a(i)}||^2."""
    x = np.asarray(keys, dtype=np.float64)
    diff = x - np.asarray(centroids, dtype=np.float64)[labels]
    return float(np.einsum("nd,nd->", diff, diff))


def lloyd(keys, init_idx, iters: int, mode: str = "exact", dtype: str = "fp64",
          history: bool = False):
    """Lloyd's algorithm as the reading above states it.

    Returns a dict with ``labels`` (a^iters), ``centroids`` (c^iters),
    ``counts`` and, when ``history`` is set, the per-iteration
    ``(c_before, labels, c_after)`` triples.
    """
    if iters < 1:
        raise ValueError("iters must be >= 1")
    x = np.asarray(keys, dtype=np.float64)
    c = x[np.asarray(init_idx)].copy()
    hist = []
    labels = counts = None
    for _ in range(iters):
        c_before = c
        labels = assign(x, centroid_for_distance(c, mode, dtype))
        c, counts = update(x, labels, c)
        if history:
            hist.append((c_before, labels, c))
    out = {"labels": labels, "centroids": c, "counts": counts}
    if history:
        out["history"] = hist
    return out


def pack(keys, values, labels, centroids, dtype: str):
    """Rows regrouped cluster by cluster (stable in key order): the CSR unit table.

    Returns dict: ``order`` (pool row r holds key ``order[r]``), ``k``/``v``
    pool rows, ``unit_start``, ``unit_size``, ``unit_mean`` (fp64 centroid) and
    ``unit_index`` (the centroid as stored in ``dtype`` for scoring).
    """
    C = np.asarray(centroids).shape[0]
    order = np.argsort(np.asarray(labels), kind="stable")
    counts = np.bincount(labels, minlength=C)
    start = np.concatenate([[0], np.cumsum(counts)[:-1]]).astype(np.int64)
    return {
        "order": order,
        "k": np.asarray(keys, dtype=np.float64)[order],
        "v": np.asarray(values, dtype=np.float64)[order],
        "unit_start": start,
        "unit_size": counts.astype(np.int64),
        "unit_mean": np.asarray(centroids, dtype=np.float64),
        "unit_index": to_storage(centroids, dtype),
    }
