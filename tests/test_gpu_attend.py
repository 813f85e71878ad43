"""GPU parity: kv_gather_attend against exact softmax attention (oracle).

LouisKV note, flowchart: the retrieved units feed attention. Metric: per
(sequence, query head) ||o - o_ref||_inf / ||o_ref||_inf <= 2e-3 (bf16/fp32
inputs, fp32 accumulation).
"""
import numpy as np
import pytest
import torch

import long_context_kv_kmeans_amd as kvc
import workloads as wl
from oracle import attend as oat
from oracle.decode import unit_rows
from tests.gpu_util import make_pool, max_rel_err, oracle_clustering, oracle_packs, \
    pool_from_labels, to_dev

pytestmark = pytest.mark.gpu
TOL = 2e-3


def _attend(pool, q_d, sel_units, sel_n, max_rows, scale):
    B, Hq, d = q_d.shape
    out = torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device="cuda")
    kvc.kv_gather_attend(pool, q_d, scale, sel_units, sel_n, max_rows, out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _sel_tensors(sel_lists, B, H, cap):
    su = torch.zeros(B, H, cap, dtype=torch.int32)
    sn = torch.zeros(B, H, dtype=torch.int32)
    for b in range(B):
        for g in range(H):
            s = sel_lists[b][g]
            su[b, g, :len(s)] = torch.tensor(s, dtype=torch.int32)
            sn[b, g] = len(s)
    return su.cuda(), sn.cuda()


@pytest.mark.parametrize("cfg_idx,over,mode", [
    (0, {}, "budget"),
    (0, {}, "full"),
    (1, dict(n_keys=4096, n_clusters=256, n_components=64, iters=2), "budget"),
    (1, dict(n_keys=4096, n_clusters=256, n_components=64, iters=2), "full"),
    (4, dict(n_keys=2048, n_clusters=128, n_components=32, iters=2, batch=3), "budget"),
    (1, dict(n_keys=3001, n_clusters=100, n_components=30, iters=2, head_dim=64), "random"),
    # every GQA group size of the bf16 and fp32 kernels, single- and multi-share
    (1, dict(n_keys=4096, n_clusters=256, n_components=64, iters=2, n_q_heads=8), "budget"),
    (1, dict(n_keys=4096, n_clusters=256, n_components=64, iters=2, n_q_heads=8), "full"),
    (1, dict(n_keys=4096, n_clusters=256, n_components=64, iters=2, n_q_heads=16), "full"),
    (1, dict(n_keys=4096, n_clusters=256, n_components=64, iters=2, n_q_heads=64), "budget"),
    (1, dict(n_keys=4096, n_clusters=256, n_components=64, iters=2, n_q_heads=64), "full"),
    (1, dict(n_keys=3001, n_clusters=100, n_components=30, iters=2, head_dim=64,
             n_q_heads=64), "full"),
    (0, dict(n_q_heads=16), "full"),
    (0, dict(n_q_heads=2), "budget"),
])
def test_attend_parity(cfg_idx, over, mode):
    cfg = wl.get_config(cfg_idx, **over)
    inp = wl.layer_inputs(cfg, 0)
    B, H, N, d = inp["keys"].shape
    labels, cents = oracle_clustering(inp["keys"], inp["init_idx"], cfg.iters, cfg.dtype)
    pool, _, _ = pool_from_labels(inp["keys"], inp["values"], labels, cents, cfg.dtype)
    q, _ = wl.layer_queries(cfg, 0, steps=2)
    q = q[1]
    G = cfg.group
    rng = np.random.default_rng(7)
    sel, max_rows = [], cfg.budget
    from oracle import select as osel
    from oracle.precision import to_storage
    for b in range(B):
        row = []
        for g in range(H):
            sizes = np.bincount(labels[b, g], minlength=cfg.n_clusters)
            if mode == "full":
                s = np.nonzero(sizes)[0]
                max_rows = N
            elif mode == "random":
                s = np.sort(rng.choice(cfg.n_clusters, 37, replace=False))
                max_rows = int(sizes[s].sum())
            else:
                sc = osel.group_scores(q[b, g * G:(g + 1) * G], to_storage(cents[b, g], cfg.dtype))
                s = osel.select_prefix(sc, sizes, cfg.budget)
            row.append(list(s))
        sel.append(row)
    cap = max(len(s) for r in sel for s in r) + 3
    su, sn = _sel_tensors(sel, B, H, cap)
    out = _attend(pool, to_dev(q, cfg.dtype), su, sn, max_rows, cfg.scale)
    packs = [oracle_packs(inp["keys"], inp["values"], labels, cents, cfg.dtype, b) for b in range(B)]
    ref = np.zeros_like(out, dtype=np.float64)
    for b in range(B):
        for g in range(H):
            p = packs[b][g]
            rows = unit_rows(p["unit_start"], p["unit_size"], sel[b][g])
            ref[b, g * G:(g + 1) * G] = oat.attend_exact(q[b, g * G:(g + 1) * G], p["k"][rows],
                                                         p["v"][rows], cfg.scale)
            if mode == "full":  # full budget == dense attention over every key (any order)
                dense = oat.attend_exact(q[b, g * G:(g + 1) * G], inp["keys"][b, g],
                                         inp["values"][b, g], cfg.scale)
                np.testing.assert_allclose(ref[b, g * G:(g + 1) * G], dense, rtol=1e-9, atol=1e-12)
    assert max_rel_err(out, ref) <= TOL


def test_attend_golden_and_edge_cases(tiny):
    c = tiny["attend"]
    d = 64
    pool = make_pool(1, 1, d, "fp32", 4, 4)
    k = np.zeros((4, d), np.float32)
    v = np.zeros((4, d), np.float32)
    k[:2, :2] = c["k"]
    v[:2, :2] = c["v"]
    pool.k[0, 0] = torch.from_numpy(k).cuda()
    pool.v[0, 0] = torch.from_numpy(v).cuda()
    pool.unit_start[0, 0, :3] = torch.tensor([0, 1, 2], dtype=torch.int32).cuda()
    pool.unit_size[0, 0, :3] = torch.tensor([1, 1, 0], dtype=torch.int32).cuda()
    q = np.zeros((1, 1, d), np.float32)
    q[0, 0, :2] = c["q"][0]
    qd = to_dev(q, "fp32")
    su, sn = _sel_tensors([[[0, 1]]], 1, 1, 4)
    out = _attend(pool, qd, su, sn, 2, c["scale"])
    np.testing.assert_allclose(out[0, 0, :2], c["expect"][0], rtol=1e-5)
    assert (out[0, 0, 2:] == 0).all()
    # single row -> o = v; empty unit in the list is harmless
    su, sn = _sel_tensors([[[2, 1]]], 1, 1, 4)
    out = _attend(pool, qd, su, sn, 2, c["scale"])
    np.testing.assert_allclose(out[0, 0], v[1], rtol=1e-6)
    # empty selection -> zeros
    su, sn = _sel_tensors([[[]]], 1, 1, 4)
    out = _attend(pool, qd, su, sn, 0, c["scale"])
    assert (out == 0).all()


def test_attend_many_splits_and_buffer_rows():
    """Selected units plus local-buffer rows, row counts spanning many splits with a ragged tail."""
    rng = np.random.default_rng(9)
    B, H, G, d, N = 2, 2, 4, 128, 5000
    pool = make_pool(B, H, d, "bf16", N, 64, buf_cap=700)
    kk = wl.to_dtype(rng.standard_normal((B, H, N, d)), "bf16")
    vv = wl.to_dtype(rng.standard_normal((B, H, N, d)), "bf16")
    pool.k.copy_(to_dev(kk, "bf16"))
    pool.v.copy_(to_dev(vv, "bf16"))
    sizes = rng.integers(1, 60, 64)
    starts = np.concatenate([[0], np.cumsum(sizes)[:-1]])
    assert starts[-1] + sizes[-1] < 4000
    pool.unit_start[:] = torch.from_numpy(starts.astype(np.int32)).cuda()
    pool.unit_size[:] = torch.from_numpy(sizes.astype(np.int32)).cuda()
    pool.n_rows.copy_(torch.tensor([4700, 4321], dtype=torch.int32))
    pool.buf_begin.copy_(torch.tensor([4001, 4000], dtype=torch.int32))
    sel = [[sorted(rng.choice(64, k, replace=False).tolist()) for k in (20, 3)],
           [sorted(rng.choice(64, k, replace=False).tolist()) for k in (0, 40)]]
    su, sn = _sel_tensors(sel, B, H, 64)
    q = wl.to_dtype(rng.standard_normal((B, H * G, d)), "bf16")
    out = _attend(pool, to_dev(q, "bf16"), su, sn, 1024, d ** -0.5)
    # the same selection handed over as row spans (no unit ids) gives the same bits
    spans = torch.zeros(B, H, 64, 2, dtype=torch.int32)
    for b in range(B):
        for g in range(H):
            for i, u in enumerate(sel[b][g]):
                spans[b, g, i, 0], spans[b, g, i, 1] = int(starts[u]), int(sizes[u])
    out_s = torch.full((B, H * G, d), float("nan"), dtype=torch.float32, device="cuda")
    kvc.kv_gather_attend(pool, to_dev(q, "bf16"), d ** -0.5, None, sn, 1024, out_s,
                         sel_spans=spans.cuda())
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out_s.cpu().numpy().view(np.uint32), out.view(np.uint32))
    nr, bb = [4700, 4321], [4001, 4000]
    for b in range(B):
        for g in range(H):
            rows = unit_rows(starts, sizes, sel[b][g])
            rows = np.concatenate([rows, np.arange(bb[b], nr[b])])
            ref = oat.attend_exact(q[b, g * G:(g + 1) * G], kk[b, g][rows], vv[b, g][rows], d ** -0.5)
            assert max_rel_err(out[b, g * G:(g + 1) * G], ref) <= TOL


def test_attend_sel_n_out_of_range_is_clamped():
    # sel_n above sel_cap reads only sel_cap entries; a negative sel_n is an empty selection
    rng = np.random.default_rng(11)
    d, G = 64, 2
    pool = make_pool(1, 2, d, "fp32", 64, 8)
    kk = rng.standard_normal((1, 2, 64, d)).astype(np.float32)
    vv = rng.standard_normal((1, 2, 64, d)).astype(np.float32)
    pool.k.copy_(torch.from_numpy(kk).cuda())
    pool.v.copy_(torch.from_numpy(vv).cuda())
    pool.unit_start[0, :, :8] = torch.arange(0, 64, 8, dtype=torch.int32).cuda()
    pool.unit_size[0, :, :8] = 8
    su, _ = _sel_tensors([[[0, 3, 5], [1, 2, 6]]], 1, 2, 3)
    sn = torch.tensor([[7, -4]], dtype=torch.int32).cuda()
    q = rng.standard_normal((1, 2 * G, d)).astype(np.float32)
    out = _attend(pool, to_dev(q, "fp32"), su, sn, 24, 0.125)
    rows = unit_rows(np.arange(0, 64, 8), np.full(8, 8), [0, 3, 5])
    ref = oat.attend_exact(q[0, :G], kk[0, 0][rows], vv[0, 0][rows], 0.125)
    assert max_rel_err(out[0, :G], ref) <= TOL
    assert (out[0, G:] == 0).all()
