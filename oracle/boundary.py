"""Oracle: the semantic-boundary test.

Test infrastructure only (see the package header).

Source: LouisKV note (papernotes.org), "Key designs" item 1: at every layer
and step, r_t is the mean over the H attention heads of the cosine
similarity between the previous step's query q_{t-1}^h and the current one
q_t^h; a retrieval is triggered when r_t falls below the threshold tau
(0.7 for Qwen3-8B). The flowchart in "Overall framework" writes the test as
``cos(q_t, q_{t-1}) < tau``.

Readings: H is every query head of the layer, per sequence; the comparison
is strict; the first decode step (no previous query) always retrieves; a
zero-norm query gives cosine 0.
"""
from __future__ import annotations

import numpy as np


def cosine(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    na = float(np.dot(a, a))
    nb = float(np.dot(b, b))
    if na == 0.0 or nb == 0.0:
        return 0.0
    return float(np.dot(a, b)) / np.sqrt(na * nb)


def boundary(q_prev, q_cur, tau: float):
    """Per sequence: (flag, r).

    q_prev, q_cur: [B, Hq, d] (q_prev None on the first step).
    Returns flag [B] bool and r [B] fp64 (NaN when q_prev is None).
    """
    q_cur = np.asarray(q_cur, dtype=np.float64)
    B, H, _ = q_cur.shape
    if q_prev is None:
        return np.ones(B, dtype=bool), np.full(B, np.nan)
    q_prev = np.asarray(q_prev, dtype=np.float64)
    r = np.empty(B, dtype=np.float64)
    for b in range(B):
        r[b] = sum(cosine(q_prev[b, h], q_cur[b, h]) for h in range(H)) / H
    return r < tau, r
