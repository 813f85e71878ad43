"""Oracle: one decode loop of one sequence and one layer, in the flowchart's order.

Test infrastructure only (see the package header).

Source: LouisKV note (papernotes.org), "Overall framework" flowchart: compute
q_t; if cos(q_t, q_{t-1}) < tau, score q_t against every unit's centroid and
fetch the Top-B units, otherwise reuse the units fetched last time; then run
attention. Segments and the local buffer follow "Key designs" item 2; group
consistency follows item 3.

Readings: on non-boundary steps the unit set of the last retrieval is reused
with the new query (segments evicted since then wait for the next
retrieval); the attended rows are the selected pool units plus, when decode
segments are enabled, every row of the local buffer (including the current
token); the budget counts pool rows per KV head.
"""
from __future__ import annotations

import numpy as np

from .attend import attend_exact
from .boundary import boundary
from .segments import SegmentState
from .select import group_scores, select_prefix


class Pool:
    """Unified per-head row store: packed prefill rows, then decode rows."""

    def __init__(self, packs, seg: SegmentState | None):
        self.packs = packs  # per KV head: oracle.kmeans.pack(...) dicts
        self.seg = seg
        self.n_prefill = packs[0]["k"].shape[0]
        self.n_clusters = len(packs[0]["unit_size"])

    def n_candidates(self) -> int:
        return self.seg.n_units_pool if self.seg else self.n_clusters

    def unit_table(self, g: int):
        """(start, size, index) of every pool candidate of KV head g."""
        p = self.packs[g]
        start, size, index = [p["unit_start"]], [p["unit_size"]], [p["unit_index"]]
        if self.seg and self.seg.n_evicted:
            n = self.seg.n_evicted
            start.append(np.array(self.seg.seg_start[:n]))
            size.append(np.array(self.seg.seg_size[:n]))
            index.append(np.stack([self.seg.seg_index[j][g] for j in range(n)]))
        return np.concatenate(start), np.concatenate(size), np.concatenate(index)

    def rows(self, g: int, row_ids):
        """K, V of pool rows ``row_ids`` of head g."""
        row_ids = np.asarray(row_ids, dtype=np.int64)
        p = self.packs[g]
        pre = row_ids < self.n_prefill
        d = p["k"].shape[1]
        K = np.empty((row_ids.size, d))
        V = np.empty((row_ids.size, d))
        K[pre] = p["k"][row_ids[pre]]
        V[pre] = p["v"][row_ids[pre]]
        if (~pre).any():
            K[~pre], V[~pre] = self.seg.decode_rows(g, row_ids[~pre])
        return K, V


def unit_rows(start, size, units) -> np.ndarray:
    if len(units) == 0:
        return np.zeros(0, dtype=np.int64)
    return np.concatenate([np.arange(start[u], start[u] + size[u]) for u in units])


def run_decode(packs, queries, tau: float, budget: int, scale: float, dtype: str,
               buf_cap: int = 0, dec_k=None, dec_v=None, steps: int | None = None,
               keep_scores: bool = False, retrieve=None, attend_steps=None):
    """Decode loop for one (layer, sequence).

    packs: per KV head, ``oracle.kmeans.pack`` dicts (same cluster count).
    queries: [steps, Hq, d]; dec_k/dec_v: [steps, H, d] when buf_cap > 0.
    retrieve: optional [steps] bools that replace the boundary test's decision
    of when to retrieve (r is still computed and logged): all true is the
    per-token retrieval of the methods the note's "Motivation" section
    criticises, every S-th step the fixed-stride policy of its ablation
    table. Only without decode segments (buf_cap == 0), where the decision
    does nothing else.
    attend_steps: optional [steps] bools; attention is computed only on those
    steps (``out`` is None on the others). It changes nothing else: the
    attention output feeds no later step.
    Returns a list of per-step dicts: flag, r, sel (per head, ascending unit
    ids; the reused set on non-boundary steps), out [Hq, d], n_rows,
    buf_begin, n_cand and, if ``keep_scores``, the scores of boundary steps.
    """
    if retrieve is not None and buf_cap > 0:
        raise ValueError("a retrieval schedule replaces the boundary test only without segments")
    H = len(packs)
    steps = queries.shape[0] if steps is None else steps
    Hq, d = queries.shape[1], queries.shape[2]
    G = Hq // H
    seg = None
    if buf_cap > 0:
        seg = SegmentState(packs[0]["k"].shape[0], len(packs[0]["unit_size"]),
                           buf_cap, H, d, steps, dtype)
    pool = Pool(packs, seg)
    sel = [np.zeros(0, dtype=np.int64) for _ in range(H)]
    log = []
    for t in range(steps):
        q_prev = None if t == 0 else queries[t - 1][None]
        flag, r = boundary(q_prev, queries[t][None], tau)
        flag = bool(flag[0]) if retrieve is None else bool(retrieve[t])
        if seg is not None:
            seg.step(flag, dec_k[t], dec_v[t])
        scores = {}
        if flag:
            for g in range(H):
                start, size, index = pool.unit_table(g)
                s = group_scores(queries[t][g * G:(g + 1) * G], index)
                sel[g] = select_prefix(s, size, budget)
                if keep_scores:
                    scores[g] = s
        out = None
        if attend_steps is None or attend_steps[t]:
            out = np.zeros((Hq, d))
            for g in range(H):
                start, size, _ = pool.unit_table(g)
                rows = unit_rows(start, size, sel[g])
                if seg is not None:
                    rows = np.concatenate([rows, seg.buffer_rows()])
                K, V = pool.rows(g, rows)
                out[g * G:(g + 1) * G] = attend_exact(queries[t][g * G:(g + 1) * G], K, V,
                                                      scale)
        entry = {"flag": flag, "r": float(r[0]), "sel": [s.copy() for s in sel], "out": out,
                 "n_cand": pool.n_candidates()}
        if seg is not None:
            entry.update(n_rows=seg.n_rows, buf_begin=seg.buf_begin, seg_begin=seg.seg_begin)
        if keep_scores:
            entry["scores"] = scores
        log.append(entry)
    return log, pool
