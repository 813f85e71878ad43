"""Oracle: decode-time temporal segments and the fixed-size local buffer.

Test infrastructure only (see the package header).

Sources: LouisKV note (papernotes.org), "Key designs" item 2 (decode half):
the generated KV is cut into temporal segments at the semantic boundaries of
item 1; each segment is indexed, like a cluster, by the mean of its keys; the
GPU keeps only a fixed-size local buffer of the most recent segments and,
when it is full, the oldest segment is moved to the unified pool, where it is
selected by the same centroid-similarity mechanism. The edgentiq blog
("Decoupled Fine-Grained Management", decode stage) says the same.

Readings:
* step order: close the open segment (if the step is a boundary and the
  segment is non-empty), append (k_t, v_t), then evict oldest closed
  segments while the buffer holds more than ``buf_cap`` rows;
* a boundary at step t closes the tokens since the previous boundary; token
  t opens the next segment; all KV heads of a sequence share the boundaries
  (r_t is per layer) while index vectors are per head;
* the buffer capacity counts the open segment too; an open segment that has
  reached ``buf_cap`` rows is closed before the next append, so eviction can
  always bring the buffer back within capacity;
* pool unit ids: clusters 0..C-1, segments C, C+1, ... in eviction order
  (which equals closing order, since the oldest is evicted first).
"""
from __future__ import annotations

import numpy as np

from .precision import to_storage


class SegmentState:
    """Bookkeeping of one sequence's decode rows, all KV heads together."""

    def __init__(self, n_prefill_rows: int, n_clusters: int, buf_cap: int,
                 n_kv_heads: int, head_dim: int, max_steps: int, dtype: str):
        if buf_cap < 1:
            raise ValueError("buf_cap must be >= 1")
        self.n_prefill = n_prefill_rows
        self.n_clusters = n_clusters
        self.buf_cap = buf_cap
        self.dtype = dtype
        self.n_rows = n_prefill_rows
        self.seg_begin = n_prefill_rows
        self.buf_begin = n_prefill_rows
        self.k = np.zeros((max_steps, n_kv_heads, head_dim), dtype=np.float64)
        self.v = np.zeros((max_steps, n_kv_heads, head_dim), dtype=np.float64)
        # closed segments, in closing order
        self.seg_start: list[int] = []
        self.seg_size: list[int] = []
        self.seg_mean: list[np.ndarray] = []   # [H, d] fp64
        self.seg_index: list[np.ndarray] = []  # [H, d] as stored
        self.n_evicted = 0

    # -- one decode step ---------------------------------------------------
    def step(self, flag: bool, k_t, v_t) -> None:
        open_len = self.n_rows - self.seg_begin
        if (flag and open_len > 0) or open_len >= self.buf_cap:
            self._close()
        i = self.n_rows - self.n_prefill
        self.k[i] = k_t
        self.v[i] = v_t
        self.n_rows += 1
        while (self.n_rows - self.buf_begin > self.buf_cap
               and self.n_evicted < len(self.seg_start)):
            j = self.n_evicted
            self.buf_begin = self.seg_start[j] + self.seg_size[j]
            self.n_evicted += 1

    def _close(self) -> None:
        lo = self.seg_begin - self.n_prefill
        hi = self.n_rows - self.n_prefill
        mean = self.k[lo:hi].mean(axis=0)  # [H, d]: the segment's key mean per head
        self.seg_start.append(self.seg_begin)
        self.seg_size.append(hi - lo)
        self.seg_mean.append(mean)
        self.seg_index.append(to_storage(mean, self.dtype))
        self.seg_begin = self.n_rows

    # -- views -------------------------------------------------------------
    @property
    def n_units_pool(self) -> int:
        """Pool candidates: clusters plus evicted segments."""
        return self.n_clusters + self.n_evicted

    def buffer_rows(self) -> np.ndarray:
        return np.arange(self.buf_begin, self.n_rows)

    def decode_rows(self, head: int, rows) -> tuple:
        idx = np.asarray(rows) - self.n_prefill
        return self.k[idx, head], self.v[idx, head]
