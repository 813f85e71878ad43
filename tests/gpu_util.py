"""Helpers for the GPU parity tests: device transfer, pool construction and a
decode-loop driver that calls the C ABI (through the Python binding) step by
step and records what each step produced."""
from __future__ import annotations

import numpy as np
import torch

import long_context_kv_kmeans_amd as kvc
from oracle import kmeans as okm


def tdtype(dtype: str) -> torch.dtype:
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def to_dev(a: np.ndarray, dtype: str) -> torch.Tensor:
    """float32 numpy array (values exact in `dtype`) -> device tensor of that dtype."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    t = t.to(tdtype(dtype))
    return t.cuda()


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def make_pool(batch, n_kv_heads, head_dim, dtype, n_keys, n_units, buf_cap=0, extra_rows=0,
              host_kv=False):
    return kvc.Pool(batch, n_kv_heads, head_dim, tdtype(dtype), row_cap=n_keys + extra_rows,
                    unit_cap=n_units, buf_cap=buf_cap, host_kv=host_kv)


def oracle_clustering(keys, init_idx, iters, dtype):
    """Oracle Lloyd (parity mode) for every (b, g). keys [B,H,N,d]."""
    B, H = keys.shape[:2]
    labels = np.empty(keys.shape[:3], np.int64)
    cents = np.empty((B, H, init_idx.shape[-1], keys.shape[-1]))
    for b in range(B):
        for g in range(H):
            out = okm.lloyd(keys[b, g], init_idx[b, g], iters, mode="parity", dtype=dtype)
            labels[b, g] = out["labels"]
            cents[b, g] = out["centroids"]
    return labels, cents


def oracle_packs(keys, values, labels, cents, dtype, b=0):
    H = keys.shape[1]
    return [okm.pack(keys[b, g], values[b, g], labels[b, g], cents[b, g], dtype) for g in range(H)]


def pool_from_labels(keys_np, values_np, labels, cents, dtype, n_units=None, buf_cap=0,
                     extra_rows=0, init_idx=None, host_kv=False):
    """GPU pool packed from the oracle's clustering, with the oracle's index vectors
    (host_kv: K/V rows in pinned host memory, packed there by the GPU)."""
    B, H, N, d = keys_np.shape
    C = cents.shape[2]
    pool = make_pool(B, H, d, dtype, N, n_units or C, buf_cap, extra_rows, host_kv=host_kv)
    keys = to_dev(keys_np, dtype)
    vals = to_dev(values_np, dtype)
    if init_idx is None:
        init_idx = np.tile(np.arange(C, dtype=np.int32), (B, H, 1))
    lab = torch.from_numpy(labels.astype(np.int32)).cuda()
    kvc.kv_cluster_build(pool, keys, vals, C, 1, torch.from_numpy(init_idx).cuda(), assign_in=lab)
    # hand the GPU the oracle's index vectors bit for bit
    from oracle.precision import to_storage
    idx = to_storage(cents, dtype).astype(np.float32)
    pool.unit_index[:, :, :C] = torch.from_numpy(idx).to(pool.unit_index.dtype).cuda()
    pool.unit_mean[:, :, :C] = torch.from_numpy(cents.astype(np.float32)).cuda()
    torch.cuda.synchronize()
    return pool, keys, vals


class DecodeRecord:
    pass


def working_set(pool, max_rows):
    """An HBM pool holding one span per (b, g): the target of kv_fetch_selected."""
    B, H = pool.batch, pool.n_kv_heads
    ws = kvc.Pool(B, H, pool.head_dim, pool.dtype, row_cap=max_rows, unit_cap=1)
    ws.spans = torch.zeros(B, H, 1, 2, dtype=torch.int32, device="cuda")
    ws.count = torch.zeros(B, H, dtype=torch.int32, device="cuda")
    return ws


def gpu_decode(pool, q, tau, budget, scale, sel_cap, dec_k=None, dec_v=None, steps=None,
               record_sel=True, fused=False, spans=False, fused_append=False, fetch=False,
               flags=None):
    """Run the decode loop through the C ABI. q: device [T, B, Hq, d].
    fused: boundary test and selection through kv_boundary_select (no segments).
    spans: selection also writes row spans and attention reads them.
    fused_append: boundary test and segment append through kv_boundary_segment_append.
    fetch: on retrieval steps kv_fetch_selected copies the selected rows into an
    HBM working set, and attention reads the working set; fetch="fused" does
    both through kv_fetch_attend; fetch="step" runs the whole step (boundary
    test, selection, fetch, attention) through kv_decode_step.
    flags: device [T, B] uint8 retrieval decisions to use instead of the boundary
    test's (kv_boundary still writes r; the selection follows the given flags)."""
    T = q.shape[0] if steps is None else steps
    B, Hq, d = q.shape[1:]
    H = pool.n_kv_heads
    dev = q.device
    rec = DecodeRecord()
    rec.wset = None
    rec.flag = torch.zeros(T, B, dtype=torch.uint8, device=dev)
    rec.r = torch.zeros(T, B, dtype=torch.float32, device=dev)
    rec.out = torch.zeros(T, B, Hq, d, dtype=torch.float32, device=dev)
    rec.sel_n = torch.zeros(T, B, H, dtype=torch.int32, device=dev)
    rec.sel = torch.zeros(T, B, H, sel_cap, dtype=torch.int32, device=dev) if record_sel else None
    rec.counters = torch.zeros(T, 5, B, dtype=torch.int32, device=dev)
    sel_units = torch.zeros(B, H, sel_cap, dtype=torch.int32, device=dev)
    sel_n = torch.zeros(B, H, dtype=torch.int32, device=dev)
    sel_rows = torch.zeros(B, H, dtype=torch.int32, device=dev)
    ws_sel = kvc.workspace(kvc.kv_select_workspace(pool, Hq))
    ws_att = kvc.workspace(kvc.kv_gather_attend_workspace(pool, Hq, budget))
    step = fetch == "step"
    sel_spans = (torch.zeros(B, H, sel_cap, 2, dtype=torch.int32, device=dev)
                 if spans or step else None)
    wset = working_set(pool, max(budget, 1)) if fetch else None
    ws_step = kvc.workspace(kvc.kv_decode_step_workspace(pool, Hq, budget)) if step else None
    for t in range(T):
        if step:
            assert flags is None and dec_k is None
            kvc.kv_decode_step(pool, q[t - 1] if t else None, q[t], tau, scale, budget,
                               rec.flag[t], sel_units, sel_spans, sel_n, sel_rows, wset,
                               wset.spans, wset.count, rec.out[t], r=rec.r[t], ws=ws_step)
        elif flags is not None:
            assert not fused and dec_k is None
            kvc.kv_boundary(q[t - 1] if t else None, q[t], tau, rec.flag[t], rec.r[t])
            rec.flag[t].copy_(flags[t])
            kvc.kv_select(pool, q[t], budget, rec.flag[t], sel_units, sel_n, sel_rows, ws=ws_sel,
                          sel_spans=sel_spans)
        elif fused:
            assert dec_k is None
            kvc.kv_boundary_select(pool, q[t - 1] if t else None, q[t], tau, budget, rec.flag[t],
                                   sel_units, sel_n, sel_rows, r=rec.r[t], ws=ws_sel,
                                   sel_spans=sel_spans)
        else:
            if fused_append:
                kvc.kv_boundary_segment_append(pool, q[t - 1] if t else None, q[t], tau,
                                               dec_k[t], dec_v[t], rec.flag[t], r=rec.r[t])
            else:
                kvc.kv_boundary(q[t - 1] if t else None, q[t], tau, rec.flag[t], rec.r[t])
                if dec_k is not None:
                    kvc.kv_segment_append(pool, dec_k[t], dec_v[t], rec.flag[t])
            kvc.kv_select(pool, q[t], budget, rec.flag[t], sel_units, sel_n, sel_rows, ws=ws_sel,
                          sel_spans=sel_spans)
        if step:
            pass
        elif fetch == "fused":
            kvc.kv_fetch_attend(pool, q[t], scale, rec.flag[t], None if spans else sel_units,
                                sel_n, budget, wset, wset.spans, wset.count, rec.out[t],
                                ws=ws_att, sel_spans=sel_spans)
        elif fetch:
            kvc.kv_fetch_selected(pool, rec.flag[t], None if spans else sel_units, sel_n, wset,
                                  wset.spans, wset.count, sel_spans=sel_spans)
            kvc.kv_gather_attend(wset, q[t], scale, None, wset.count, budget, rec.out[t],
                                 ws=ws_att, sel_spans=wset.spans)
        else:
            kvc.kv_gather_attend(pool, q[t], scale, None if spans else sel_units, sel_n, budget,
                                 rec.out[t], ws=ws_att, sel_spans=sel_spans)
        rec.sel_n[t].copy_(sel_n)
        if record_sel:
            rec.sel[t].copy_(sel_units)
        if dec_k is not None:
            for i, c in enumerate((pool.n_rows, pool.n_units, pool.n_cand, pool.buf_begin,
                                   pool.seg_begin)):
                rec.counters[t, i].copy_(c)
    torch.cuda.synchronize()
    rec.wset = wset
    return rec


def max_rel_err(out, ref):
    """max over vectors of ||o - o_ref||_inf / ||o_ref||_inf (last axis)."""
    out = np.asarray(out, np.float64)
    ref = np.asarray(ref, np.float64)
    num = np.abs(out - ref).max(axis=-1)
    den = np.abs(ref).max(axis=-1)
    den = np.where(den > 0, den, 1.0)
    return float((num / den).max())
