"""Oracle: group-consistent centroid scoring and budgeted unit selection.

Test infrastructure only (see the package header).

Sources: LouisKV note (papernotes.org)
* "Overall framework" flowchart: on a boundary, q_t is compared with every
  unit's centroid and the Top-B units are fetched;
* "Key designs" item 2: attention scores are dominated by the q.k dot
  product, so keys (and their mean) close in that sense get similar
  attention -- the score of a unit is the dot product of q with its index;
* "Key designs" item 3: one common cluster/segment set is chosen for the
  whole GQA query group (group-consistent selection), and selection is done
  under a token budget over units holding variable numbers of KV rows.

Readings:
* score of unit u for KV head g: s_u = sum over the group's query heads h of
  q_h . idx_u (the group sum; ranks the same as the group mean);
* candidates are the non-empty pool units (empty clusters hold no KV);
* rank by (score descending, unit id ascending) and keep the longest prefix
  whose total size fits the budget; no partial unit, no skipping past a unit
  that does not fit ("Top-B" read as a token budget because units vary in
  size).
"""
from __future__ import annotations

import numpy as np


def group_scores(q_group, index) -> np.ndarray:
    """s_u = sum_h q_h . idx_u, fp64. q_group [G, d], index [U, d] -> [U]."""
    q = np.asarray(q_group, dtype=np.float64)
    idx = np.asarray(index, dtype=np.float64)
    s = np.zeros(idx.shape[0], dtype=np.float64)
    for h in range(q.shape[0]):
        s += idx @ q[h]
    return s


def rank_units(scores, sizes) -> np.ndarray:
    """Non-empty unit ids in rank order (score desc, id asc)."""
    scores = np.asarray(scores, dtype=np.float64)
    sizes = np.asarray(sizes)
    ids = np.nonzero(sizes > 0)[0]
    # np.lexsort sorts by the last key first; ascending, so negate scores.
    order = np.lexsort((ids, -scores[ids]))
    return ids[order]


def select_prefix(scores, sizes, budget: int) -> np.ndarray:
    """Longest rank-order prefix with total size <= budget; ids returned ascending."""
    sizes = np.asarray(sizes)
    chosen = []
    used = 0
    for u in rank_units(scores, sizes):
        if used + int(sizes[u]) > budget:
            break
        used += int(sizes[u])
        chosen.append(int(u))
    return np.array(sorted(chosen), dtype=np.int64)
