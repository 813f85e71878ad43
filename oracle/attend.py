"""Oracle: exact softmax attention of the group's queries over the retrieved rows.

Test infrastructure only (see the package header).

Source: LouisKV note (papernotes.org), "Overall framework" flowchart -- the
retrieved (or reused) critical KV feeds "Attention + FFN"; only the attention
half is on this path.

Readings: scale 1/sqrt(d); no mask (every attended row is in the past); no
positional transform (synthetic q and k stand in for post-rotary tensors);
an empty row set gives a zero output.
"""
from __future__ import annotations

import numpy as np


def attend_exact(q_heads, k_rows, v_rows, scale: float) -> np.ndarray:
    """o_h = softmax(scale * K q_h) V for each query head; fp64.

    q_heads [G, d]; k_rows, v_rows [R, d] -> [G, d].
    """
    q = np.asarray(q_heads, dtype=np.float64)
    K = np.asarray(k_rows, dtype=np.float64)
    V = np.asarray(v_rows, dtype=np.float64)
    if K.shape[0] == 0:
        return np.zeros_like(q)
    s = (K @ q.T) * scale  # [R, G]
    s = s - s.max(axis=0, keepdims=True)  # exp(s - m) / sum exp(s - m) == softmax(s)
    p = np.exp(s)
    return (p.T @ V) / p.sum(axis=0)[:, None]
