"""Centroid-indexed KV-cache retrieval (LouisKV's hot path) on MI355X.

Thin Python binding over ``libkvc.so`` (HIP, gfx950). Every function here
only marshals arguments -- device pointers of torch tensors, sizes and the
current HIP stream -- into the C ABI declared in ``include/kvc.h``; all
computation runs in the library's kernels. Torch supplies device memory and
streams only. If the library is missing, importing works but every call
raises ``KvcLibraryMissing``: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkvc.so")

KV_OK = 0
KV_ERR_INVALID_ARG = -1
KV_ERR_UNSUPPORTED = -2
KV_ERR_WORKSPACE = -3
KV_ERR_CAPACITY = -4
KV_ERR_HIP = -5

KV_F32 = 0
KV_BF16 = 1

EXPORTED = [
    "kv_status_string",
    "kv_cluster_build_workspace", "kv_cluster_build",
    "kv_kmeans_assign_workspace", "kv_kmeans_assign",
    "kv_kmeans_prepare", "kv_kmeans_assign_prepared",
    "kv_kmeans_update_workspace", "kv_kmeans_update",
    "kv_boundary",
    "kv_segment_append", "kv_boundary_segment_append",
    "kv_select_workspace", "kv_select", "kv_boundary_select",
    "kv_gather_attend_workspace", "kv_gather_attend", "kv_gather_attend_noalloc",
    "kv_fetch_selected", "kv_fetch_attend", "kv_host_device_pointer",
    "kv_decode_step_workspace", "kv_decode_step",
]


class KvcLibraryMissing(RuntimeError):
    pass


class KvError(RuntimeError):
    def __init__(self, fn: str, code: int):
        super().__init__(f"{fn} failed: {status_string(code)} ({code})")
        self.code = code


class KVPool(ctypes.Structure):
    """Mirror of ``struct kv_pool`` in kvc.h."""

    _fields_ = [
        ("batch", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("row_cap", ctypes.c_int32), ("unit_cap", ctypes.c_int32),
        ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("unit_start", ctypes.c_void_p), ("unit_size", ctypes.c_void_p),
        ("unit_mean", ctypes.c_void_p), ("unit_index", ctypes.c_void_p),
        ("n_rows", ctypes.c_void_p), ("n_units", ctypes.c_void_p), ("n_cand", ctypes.c_void_p),
        ("buf_cap", ctypes.c_int32),
        ("buf_begin", ctypes.c_void_p), ("seg_begin", ctypes.c_void_p),
        ("seg_sum", ctypes.c_void_p), ("status", ctypes.c_void_p),
        ("buf_k", ctypes.c_void_p), ("buf_v", ctypes.c_void_p), ("buf_ring", ctypes.c_int32),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libkvc.so; raises KvcLibraryMissing if it was never built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise KvcLibraryMissing(
            f"{LIB_PATH} not found: build it with `python -m long_context_kv_kmeans_amd._build`")
    L = ctypes.CDLL(LIB_PATH)
    c_int, c_size, vp = ctypes.c_int32, ctypes.c_size_t, ctypes.c_void_p
    pool_p = ctypes.POINTER(KVPool)
    sig = {
        "kv_status_string": (ctypes.c_char_p, [c_int]),
        "kv_cluster_build_workspace": (c_size, [c_int, c_int, c_int, c_int, c_int, c_int]),
        "kv_cluster_build": (c_int, [pool_p, vp, vp, c_int, c_int, c_int, vp, vp, vp, vp, vp,
                                     vp, c_size, vp]),
        "kv_kmeans_assign_workspace": (c_size, [c_int, c_int, c_int, c_int]),
        "kv_kmeans_assign": (c_int, [vp, vp, c_int, c_int, c_int, c_int, c_int, vp, vp, c_size, vp]),
        "kv_kmeans_prepare": (c_int, [vp, c_int, c_int, c_int, c_int, vp, c_size, vp]),
        "kv_kmeans_assign_prepared": (c_int, [vp, vp, c_int, c_int, c_int, c_int, c_int, vp, vp,
                                              c_size, vp]),
        "kv_kmeans_update_workspace": (c_size, [c_int, c_int, c_int]),
        "kv_kmeans_update": (c_int, [vp, vp, vp, vp, vp, c_int, c_int, c_int, c_int, c_int, vp,
                                     c_size, vp]),
        "kv_boundary": (c_int, [vp, vp, c_int, c_int, c_int, c_int, ctypes.c_float, vp, vp, vp]),
        "kv_segment_append": (c_int, [pool_p, vp, vp, vp, vp]),
        "kv_boundary_segment_append": (c_int, [pool_p, vp, vp, c_int, ctypes.c_float, vp, vp, vp,
                                               vp, vp]),
        "kv_select_workspace": (c_size, [pool_p, c_int]),
        "kv_select": (c_int, [pool_p, vp, c_int, c_int, vp, vp, c_int, vp, vp, vp, vp, vp, c_size,
                              vp]),
        "kv_boundary_select": (c_int, [pool_p, vp, vp, c_int, ctypes.c_float, c_int, vp, vp, vp,
                                       c_int, vp, vp, vp, vp, vp, c_size, vp]),
        "kv_gather_attend_workspace": (c_size, [pool_p, c_int, c_int]),
        "kv_gather_attend": (c_int, [pool_p, vp, c_int, ctypes.c_float, vp, vp, c_int, vp, c_int,
                                     vp, vp, c_size, vp]),
        "kv_gather_attend_noalloc": (c_int, [pool_p, vp, c_int, ctypes.c_float, vp, vp, c_int, vp,
                                             c_int, vp, vp]),
        "kv_fetch_selected": (c_int, [pool_p, vp, vp, vp, c_int, vp, pool_p, vp, vp, vp]),
        "kv_fetch_attend": (c_int, [pool_p, vp, c_int, ctypes.c_float, vp, vp, vp, c_int, vp,
                                    c_int, pool_p, vp, vp, vp, vp, c_size, vp]),
        "kv_host_device_pointer": (c_int, [vp, ctypes.POINTER(vp)]),
        "kv_decode_step_workspace": (c_size, [pool_p, c_int, c_int]),
        "kv_decode_step": (c_int, [pool_p, vp, vp, c_int, ctypes.c_float, ctypes.c_float, c_int,
                                   vp, vp, vp, vp, c_int, vp, vp, pool_p, vp, vp, vp, vp, c_size,
                                   vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def status_string(code: int) -> str:
    try:
        return lib().kv_status_string(code).decode()
    except KvcLibraryMissing:
        return str(code)


def _check(fn: str, code: int) -> None:
    if code != KV_OK:
        raise KvError(fn, code)


# ---------------------------------------------------------------- marshalling
def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _expect(name: str, t: Optional[torch.Tensor], shape=None, dtype=None,
            optional: bool = False) -> None:
    """Raise ValueError unless ``t`` has ``dtype`` and ``shape`` (None entries
    in ``shape`` match any extent). The C ABI takes bare device pointers, so a
    tensor of the wrong element type or extent would be read or written out of
    its bounds: every wrapper checks here first."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name}: element type {t.dtype}, expected {dtype}")
    if shape is not None:
        ok = t.dim() == len(shape) and all(e is None or int(a) == int(e)
                                            for a, e in zip(t.shape, shape))
        if not ok:
            want = "[" + ", ".join("*" if e is None else str(e) for e in shape) + "]"
            raise ValueError(f"{name}: shape {list(t.shape)}, expected {want}")


def _nbytes(t: torch.Tensor) -> int:
    return t.numel() * t.element_size()


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def dtype_code(t: torch.dtype) -> int:
    if t == torch.bfloat16:
        return KV_BF16
    if t == torch.float32:
        return KV_F32
    raise ValueError(f"unsupported element type {t}")


def torch_dtype(code: int) -> torch.dtype:
    return torch.bfloat16 if code == KV_BF16 else torch.float32


def workspace(nbytes: int, device="cuda") -> torch.Tensor:
    """Zero-filled device workspace of at least ``nbytes`` (256-byte aligned)."""
    return torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def _call_workspace(nbytes: int, stream=None) -> torch.Tensor:
    """A workspace for one call enqueued on ``stream``: allocated and zero-filled
    on that stream, so that the fill is ordered before the call's kernels and
    the caching allocator reuses the memory only after them."""
    if stream is None:
        return workspace(nbytes)
    with torch.cuda.stream(stream):
        return workspace(nbytes)


def host_device_pointer(t: torch.Tensor) -> int:
    """Device address of a pinned host tensor (hipHostMalloc memory)."""
    dev = ctypes.c_void_p()
    _check("kv_host_device_pointer",
           lib().kv_host_device_pointer(ctypes.c_void_p(t.data_ptr()), ctypes.byref(dev)))
    return int(dev.value)


@dataclass
class Pool:
    """Tensors behind one ``kv_pool`` (see kvc.h for the layout). With
    ``host_kv`` the K and V rows live in pinned host memory, which the kernels
    reach through its device address; every table stays on the GPU, and a
    pool with a local buffer also keeps an HBM copy of the buffer
    (``buf_k``, ``buf_v``, ``buf_cap`` slots per head)."""

    batch: int
    n_kv_heads: int
    head_dim: int
    dtype: torch.dtype
    row_cap: int
    unit_cap: int
    buf_cap: int = 0
    device: str = "cuda"
    host_kv: bool = False

    def __post_init__(self):
        B, H, D = self.batch, self.n_kv_heads, self.head_dim
        dev, i32 = self.device, torch.int32
        if self.host_kv:
            self.k = torch.zeros(B, H, self.row_cap, D, dtype=self.dtype, pin_memory=True)
            self.v = torch.zeros(B, H, self.row_cap, D, dtype=self.dtype, pin_memory=True)
        else:
            self.k = torch.zeros(B, H, self.row_cap, D, dtype=self.dtype, device=dev)
            self.v = torch.zeros_like(self.k)
        self.unit_start = torch.zeros(B, H, self.unit_cap, dtype=i32, device=dev)
        self.unit_size = torch.zeros(B, H, self.unit_cap, dtype=i32, device=dev)
        self.unit_mean = torch.zeros(B, H, self.unit_cap, D, dtype=torch.float32, device=dev)
        self.unit_index = torch.zeros(B, H, self.unit_cap, D, dtype=self.dtype, device=dev)
        self.n_rows = torch.zeros(B, dtype=i32, device=dev)
        self.n_units = torch.zeros(B, dtype=i32, device=dev)
        self.n_cand = torch.zeros(B, dtype=i32, device=dev)
        self.buf_begin = torch.zeros(B, dtype=i32, device=dev)
        self.seg_begin = torch.zeros(B, dtype=i32, device=dev)
        self.seg_sum = (torch.zeros(B, H, D, dtype=torch.float32, device=dev)
                        if self.buf_cap > 0 else None)
        self.status = torch.zeros(1, dtype=i32, device=dev)
        self.buf_k = self.buf_v = None
        if self.host_kv and self.buf_cap > 0:
            self.buf_k = torch.zeros(B, H, self.buf_cap, D, dtype=self.dtype, device=dev)
            self.buf_v = torch.zeros_like(self.buf_k)
        self._struct = None

    def struct(self) -> KVPool:
        if self._struct is None:
            p = lambda t: None if t is None else t.data_ptr()  # noqa: E731
            kv = p if not self.host_kv else host_device_pointer
            self._struct = KVPool(
                self.batch, self.n_kv_heads, self.head_dim, dtype_code(self.dtype),
                self.row_cap, self.unit_cap, kv(self.k), kv(self.v), p(self.unit_start),
                p(self.unit_size), p(self.unit_mean), p(self.unit_index), p(self.n_rows),
                p(self.n_units), p(self.n_cand), self.buf_cap, p(self.buf_begin),
                p(self.seg_begin), p(self.seg_sum), p(self.status), p(self.buf_k), p(self.buf_v),
                self.buf_cap if self.buf_k is not None else 0)
        return self._struct

    def ref(self):
        return ctypes.byref(self.struct())


# ---------------------------------------------------------------- K-means
def kv_cluster_build_workspace(batch, n_kv_heads, n_keys, head_dim, n_clusters, dtype) -> int:
    return lib().kv_cluster_build_workspace(batch, n_kv_heads, n_keys, head_dim, n_clusters,
                                            dtype_code(dtype))


def kv_cluster_build(pool: Pool, keys, values, n_clusters: int, iters: int, init_idx,
                     assign_in=None, assign_out=None, ws=None, stream=None,
                     rounds_out=None, sweeps_out=None) -> None:
    """rounds_out (optional) [B, H] int32 receives the rounds whose assignment
    ran for each head (a head at a fixed point of Lloyd's iteration skips the
    rest, with the same result); sweeps_out (optional) [B, H] float32 the
    assignment work in whole sweeps of keys x clusters (later rounds score
    only the centroids that moved, with the same result)."""
    B, H, D = pool.batch, pool.n_kv_heads, pool.head_dim
    _expect("keys", keys, (B, H, None, D), pool.dtype)
    N = keys.shape[2]
    _expect("values", values, (B, H, N, D), pool.dtype)
    _expect("init_idx", init_idx, (B, H, n_clusters), torch.int32)
    _expect("assign_in", assign_in, (B, H, N), torch.int32, optional=True)
    _expect("assign_out", assign_out, (B, H, N), torch.int32, optional=True)
    _expect("rounds_out", rounds_out, (B, H), torch.int32, optional=True)
    _expect("sweeps_out", sweeps_out, (B, H), torch.float32, optional=True)
    if ws is None:
        ws = _call_workspace(kv_cluster_build_workspace(B, H, N, D, n_clusters, keys.dtype), stream)
    _check("kv_cluster_build", lib().kv_cluster_build(
        pool.ref(), _ptr(keys), _ptr(values), N, n_clusters, iters, _ptr(init_idx),
        _ptr(assign_in), _ptr(assign_out), _ptr(rounds_out), _ptr(sweeps_out), _ptr(ws),
        _nbytes(ws),
        _stream(stream)))


def kv_kmeans_assign(keys, centroids, labels, ws=None, stream=None) -> None:
    """keys [BH, N, D]; centroids [BH, C, D] fp32; labels [BH, N] int32."""
    BH, N, D, C = _kmeans_shapes(keys, centroids, labels)
    dt = dtype_code(keys.dtype)
    if ws is None:
        ws = _call_workspace(lib().kv_kmeans_assign_workspace(BH, C, D, dt), stream)
    _check("kv_kmeans_assign", lib().kv_kmeans_assign(
        _ptr(keys), _ptr(centroids), BH, N, D, C, dt, _ptr(labels), _ptr(ws), _nbytes(ws),
        _stream(stream)))


def _kmeans_shapes(keys, centroids, labels):
    if keys.dim() != 3:
        raise ValueError(f"keys: shape {list(keys.shape)}, expected [BH, N, D]")
    dtype_code(keys.dtype)
    BH, N, D = keys.shape
    _expect("centroids", centroids, (BH, None, D), torch.float32)
    _expect("labels", labels, (BH, N), torch.int32)
    return BH, N, D, centroids.shape[1]


def kv_kmeans_prepare(centroids, dtype, ws, stream=None) -> None:
    """centroids [BH, C, D] fp32 -> their assignment form in ws (for keys of `dtype`)."""
    _expect("centroids", centroids, (None, None, None), torch.float32)
    BH, C, D = centroids.shape
    _check("kv_kmeans_prepare", lib().kv_kmeans_prepare(
        _ptr(centroids), BH, D, C, dtype_code(dtype), _ptr(ws), _nbytes(ws), _stream(stream)))


def kv_kmeans_assign_prepared(keys, centroids, labels, ws, stream=None) -> None:
    """Labels of keys [BH, N, D] against centroids already prepared in ws."""
    BH, N, D, C = _kmeans_shapes(keys, centroids, labels)
    _check("kv_kmeans_assign_prepared", lib().kv_kmeans_assign_prepared(
        _ptr(keys), _ptr(centroids), BH, N, D, C, dtype_code(keys.dtype), _ptr(labels), _ptr(ws),
        _nbytes(ws), _stream(stream)))


def kv_kmeans_update(keys, labels, centroids_in, centroids_out, counts=None, ws=None,
                     stream=None) -> None:
    BH, N, D, C = _kmeans_shapes(keys, centroids_in, labels)
    _expect("centroids_out", centroids_out, (BH, C, D), torch.float32)
    _expect("counts", counts, (BH, C), torch.int32, optional=True)
    if ws is None:
        ws = _call_workspace(lib().kv_kmeans_update_workspace(BH, N, C), stream)
    _check("kv_kmeans_update", lib().kv_kmeans_update(
        _ptr(keys), _ptr(labels), _ptr(centroids_in), _ptr(centroids_out), _ptr(counts), BH, N,
        D, C, dtype_code(keys.dtype), _ptr(ws), _nbytes(ws), _stream(stream)))


# ---------------------------------------------------------------- decode
def kv_boundary(q_prev, q_cur, tau: float, flag, r=None, stream=None) -> None:
    if q_cur.dim() != 3:
        raise ValueError(f"q_cur: shape {list(q_cur.shape)}, expected [B, Hq, D]")
    B, Hq, D = q_cur.shape
    _expect("q_prev", q_prev, (B, Hq, D), q_cur.dtype, optional=True)
    _expect("flag", flag, (B,), torch.uint8)
    _expect("r", r, (B,), torch.float32, optional=True)
    _check("kv_boundary", lib().kv_boundary(
        _ptr(q_prev), _ptr(q_cur), B, Hq, D, dtype_code(q_cur.dtype), float(tau), _ptr(flag),
        _ptr(r), _stream(stream)))


def _kv_step(pool: Pool, k_t, v_t, flag):
    shape = (pool.batch, pool.n_kv_heads, pool.head_dim)
    _expect("k_t", k_t, shape, pool.dtype)
    _expect("v_t", v_t, shape, pool.dtype)
    _expect("flag", flag, (pool.batch,), torch.uint8)


def _queries(pool: Pool, q, name="q"):
    """q [B, Hq, D] in the pool's element type; returns Hq."""
    if q.dim() != 3:
        raise ValueError(f"{name}: shape {list(q.shape)}, expected [B, Hq, D]")
    _expect(name, q, (pool.batch, None, pool.head_dim), pool.dtype)
    return q.shape[1]


def _selection(pool: Pool, sel_units, sel_spans, sel_n, cap_from=None):
    """Selection lists: sel_units [B, H, cap] and/or sel_spans [B, H, cap, 2]
    (int32, same cap), sel_n [B, H]; returns cap."""
    B, H = pool.batch, pool.n_kv_heads
    if sel_units is None and sel_spans is None:
        raise ValueError("sel_units or sel_spans is required")
    cap = sel_units.shape[-1] if sel_units is not None else sel_spans.shape[-2]
    _expect("sel_units", sel_units, (B, H, cap), torch.int32, optional=True)
    _expect("sel_spans", sel_spans, (B, H, cap, 2), torch.int32, optional=True)
    _expect("sel_n", sel_n, (B, H), torch.int32)
    return cap


def kv_segment_append(pool: Pool, k_t, v_t, flag, stream=None) -> None:
    _kv_step(pool, k_t, v_t, flag)
    _check("kv_segment_append", lib().kv_segment_append(
        pool.ref(), _ptr(k_t), _ptr(v_t), _ptr(flag), _stream(stream)))


def kv_boundary_segment_append(pool: Pool, q_prev, q_cur, tau: float, k_t, v_t, flag, r=None,
                               stream=None) -> None:
    """kv_boundary then kv_segment_append in one launch (q_prev None: first step)."""
    Hq = _queries(pool, q_cur, "q_cur")
    _expect("q_prev", q_prev, tuple(q_cur.shape), pool.dtype, optional=True)
    _kv_step(pool, k_t, v_t, flag)
    _expect("r", r, (pool.batch,), torch.float32, optional=True)
    _check("kv_boundary_segment_append", lib().kv_boundary_segment_append(
        pool.ref(), _ptr(q_prev), _ptr(q_cur), q_cur.shape[1], float(tau), _ptr(k_t), _ptr(v_t),
        _ptr(flag), _ptr(r), _stream(stream)))


def kv_select_workspace(pool: Pool, n_q_heads: int) -> int:
    return lib().kv_select_workspace(pool.ref(), n_q_heads)


def kv_select(pool: Pool, q, budget: int, flag, sel_units, sel_n, sel_rows, scores_out=None,
              ws=None, stream=None, sel_spans=None) -> None:
    """sel_spans (optional) [B, H, sel_cap, 2] int32 receives the selected units' row spans."""
    Hq = _queries(pool, q)
    _expect("flag", flag, (pool.batch,), torch.uint8, optional=True)  # None: every sequence
    _select_outputs(pool, sel_units, sel_n, sel_rows, sel_spans, scores_out)
    if ws is None:
        ws = _call_workspace(kv_select_workspace(pool, Hq), stream)
    _check("kv_select", lib().kv_select(
        pool.ref(), _ptr(q), Hq, int(budget), _ptr(flag), _ptr(sel_units), sel_units.shape[-1],
        _ptr(sel_n), _ptr(sel_rows), _ptr(sel_spans), _ptr(scores_out), _ptr(ws), _nbytes(ws),
        _stream(stream)))


def _select_outputs(pool: Pool, sel_units, sel_n, sel_rows, sel_spans, scores_out):
    B, H = pool.batch, pool.n_kv_heads
    _expect("sel_units", sel_units, (B, H, None), torch.int32)
    _selection(pool, sel_units, sel_spans, sel_n)
    _expect("sel_rows", sel_rows, (B, H), torch.int32)
    _expect("scores_out", scores_out, (B, H, pool.unit_cap), torch.float32, optional=True)


def kv_boundary_select(pool: Pool, q_prev, q_cur, tau: float, budget: int, flag, sel_units,
                       sel_n, sel_rows, r=None, scores_out=None, ws=None, stream=None,
                       sel_spans=None) -> None:
    """kv_boundary then kv_select in one launch (q_prev None: first decode step)."""
    Hq = _queries(pool, q_cur, "q_cur")
    _expect("q_prev", q_prev, tuple(q_cur.shape), pool.dtype, optional=True)
    _expect("flag", flag, (pool.batch,), torch.uint8)
    _expect("r", r, (pool.batch,), torch.float32, optional=True)
    _select_outputs(pool, sel_units, sel_n, sel_rows, sel_spans, scores_out)
    if ws is None:
        ws = _call_workspace(kv_select_workspace(pool, Hq), stream)
    _check("kv_boundary_select", lib().kv_boundary_select(
        pool.ref(), _ptr(q_prev), _ptr(q_cur), Hq, float(tau), int(budget), _ptr(flag), _ptr(r),
        _ptr(sel_units), sel_units.shape[-1], _ptr(sel_n), _ptr(sel_rows), _ptr(sel_spans),
        _ptr(scores_out), _ptr(ws), _nbytes(ws), _stream(stream)))


def kv_gather_attend_workspace(pool: Pool, n_q_heads: int, max_rows: int) -> int:
    return lib().kv_gather_attend_workspace(pool.ref(), n_q_heads, max_rows)


def kv_gather_attend(pool: Pool, q, scale: float, sel_units, sel_n, max_rows: int, out,
                     ws=None, stream=None, sel_spans=None) -> None:
    """sel_spans (optional, from kv_select) replaces the unit-table lookup of sel_units."""
    Hq = _queries(pool, q)
    cap = _selection(pool, sel_units, sel_spans, sel_n)
    _expect("out", out, (pool.batch, Hq, pool.head_dim), torch.float32)
    if ws is None:
        ws = _call_workspace(kv_gather_attend_workspace(pool, Hq, max_rows), stream)
    _check("kv_gather_attend", lib().kv_gather_attend(
        pool.ref(), _ptr(q), Hq, float(scale), _ptr(sel_units), _ptr(sel_spans), cap,
        _ptr(sel_n), int(max_rows), _ptr(out), _ptr(ws), _nbytes(ws), _stream(stream)))


def kv_gather_attend_noalloc(pool: Pool, q, scale: float, sel_units, sel_n, max_rows: int, out,
                             stream=None, sel_spans=None) -> None:
    """kv_gather_attend with the library's static device scratch in place of a
    workspace: allocates nothing (calls that overlap on one device race)."""
    Hq = _queries(pool, q)
    cap = _selection(pool, sel_units, sel_spans, sel_n)
    _expect("out", out, (pool.batch, Hq, pool.head_dim), torch.float32)
    _check("kv_gather_attend_noalloc", lib().kv_gather_attend_noalloc(
        pool.ref(), _ptr(q), Hq, float(scale), _ptr(sel_units), _ptr(sel_spans), cap,
        _ptr(sel_n), int(max_rows), _ptr(out), _stream(stream)))


# ---------------------------------------------------------------- working set
def kv_fetch_selected(pool: Pool, flag, sel_units, sel_n, dst: Pool, dst_spans, dst_n,
                      sel_spans=None, stream=None) -> None:
    """Selected rows of `pool` -> the HBM working set `dst` (sequences with flag 1).
    dst_spans [B, H, 1, 2] int32 and dst_n [B, H] int32 then describe it to
    kv_gather_attend(dst, ..., sel_spans=dst_spans, sel_n=dst_n)."""
    cap = _selection(pool, sel_units, sel_spans, sel_n)
    _working_set(pool, flag, dst, dst_spans, dst_n)
    _check("kv_fetch_selected", lib().kv_fetch_selected(
        pool.ref(), _ptr(flag), _ptr(sel_units), _ptr(sel_spans), cap, _ptr(sel_n), dst.ref(),
        _ptr(dst_spans), _ptr(dst_n), _stream(stream)))


def kv_fetch_attend(pool: Pool, q, scale: float, flag, sel_units, sel_n, max_rows: int,
                    dst: Pool, dst_spans, dst_n, out, ws=None, stream=None,
                    sel_spans=None) -> None:
    """kv_fetch_selected + kv_gather_attend over the working set (and the
    pool's local buffer), in one launch."""
    Hq = _queries(pool, q)
    cap = _selection(pool, sel_units, sel_spans, sel_n)
    _working_set(pool, flag, dst, dst_spans, dst_n)
    _expect("out", out, (pool.batch, Hq, pool.head_dim), torch.float32)
    if ws is None:
        ws = _call_workspace(kv_gather_attend_workspace(pool, Hq, max_rows), stream)
    _check("kv_fetch_attend", lib().kv_fetch_attend(
        pool.ref(), _ptr(q), Hq, float(scale), _ptr(flag), _ptr(sel_units), _ptr(sel_spans), cap,
        _ptr(sel_n), int(max_rows), dst.ref(), _ptr(dst_spans), _ptr(dst_n), _ptr(out), _ptr(ws),
        _nbytes(ws), _stream(stream)))


def _working_set(pool: Pool, flag, dst: Pool, dst_spans, dst_n):
    B, H = pool.batch, pool.n_kv_heads
    _expect("flag", flag, (B,), torch.uint8)
    _expect("dst_spans", dst_spans, None, torch.int32)
    if dst_spans.numel() != B * H * 2:  # one (start, rows) span per (sequence, KV head)
        raise ValueError(f"dst_spans: shape {list(dst_spans.shape)}, expected {B * H * 2} "
                         "int32 values (e.g. [B, H, 1, 2])")
    _expect("dst_n", dst_n, (B, H), torch.int32)


# ---------------------------------------------------------------- one launch per step
def kv_decode_step_workspace(pool: Pool, n_q_heads: int, budget: int) -> int:
    return lib().kv_decode_step_workspace(pool.ref(), n_q_heads, int(budget))


def kv_decode_step(pool: Pool, q_prev, q_cur, tau: float, scale: float, budget: int, flag,
                   sel_units, sel_spans, sel_n, sel_rows, dst: Pool, dst_spans, dst_n, out,
                   r=None, ws=None, stream=None) -> None:
    """kv_boundary_select + kv_fetch_attend (max_rows = budget) in one launch
    (q_prev None: first decode step)."""
    Hq = _queries(pool, q_cur, "q_cur")
    _expect("q_prev", q_prev, tuple(q_cur.shape), pool.dtype, optional=True)
    _expect("r", r, (pool.batch,), torch.float32, optional=True)
    _select_outputs(pool, sel_units, sel_n, sel_rows, sel_spans, None)
    _expect("sel_spans", sel_spans, (pool.batch, pool.n_kv_heads, sel_units.shape[-1], 2),
            torch.int32)
    _working_set(pool, flag, dst, dst_spans, dst_n)
    _expect("out", out, (pool.batch, Hq, pool.head_dim), torch.float32)
    if ws is None:
        ws = _call_workspace(kv_decode_step_workspace(pool, Hq, budget), stream)
    _check("kv_decode_step", lib().kv_decode_step(
        pool.ref(), _ptr(q_prev), _ptr(q_cur), Hq, float(tau), float(scale), int(budget),
        _ptr(flag), _ptr(r), _ptr(sel_units), _ptr(sel_spans), sel_units.shape[-1], _ptr(sel_n),
        _ptr(sel_rows), dst.ref(), _ptr(dst_spans), _ptr(dst_n), _ptr(out), _ptr(ws),
        _nbytes(ws), _stream(stream)))
