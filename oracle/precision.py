"""Oracle: storage precision of the scoring and distance copies.

Test infrastructure only (see the package header).

The pages fix no precision. The GPU path stores keys/values in the working
dtype and feeds centroids to the matrix cores as bf16 rounded from an fp32
master copy, accumulating in fp32 ("bf16 in, fp32 accumulate"). To compare
like with like, the oracle rounds its fp64 centroids the same way
(fp64 -> fp32 -> bf16, round to nearest even) before computing distances or
scores in fp64. This module is the oracle's own bf16 rounding, written from
the IEEE/bfloat16 definition: bf16 keeps the top 16 bits of the fp32
encoding, rounding the dropped 16 bits to nearest, ties to even.
"""
import numpy as np


def round_fp32(x) -> np.ndarray:
    """fp64 -> nearest fp32 (returned as float64)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def round_bf16(x) -> np.ndarray:
    """fp64 -> fp32 -> bf16 by round-to-nearest-even (returned as float64).

    Finite inputs only (the workloads never produce NaN/inf).
    """
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32))
    bits = f.view(np.uint32).astype(np.uint64)
    keep_lsb = (bits >> np.uint64(16)) & np.uint64(1)
    rounded = (bits + np.uint64(0x7FFF) + keep_lsb) & np.uint64(0xFFFF0000)
    return rounded.astype(np.uint32).view(np.float32).astype(np.float64)


def to_storage(x, dtype: str) -> np.ndarray:
    """Value after being stored in the working dtype (via fp32)."""
    if dtype == "bf16":
        return round_bf16(x)
    if dtype == "fp32":
        return round_fp32(x)
    if dtype == "fp64":
        return np.asarray(x, dtype=np.float64)
    raise ValueError(dtype)
