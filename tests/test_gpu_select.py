"""GPU parity: kv_select (group-consistent scoring + budgeted prefix selection).

LouisKV note: flowchart (score q_t against every unit's centroid, fetch the
Top-B units) and key design 3 (one unit set per GQA group; token budget over
units of variable size). Given the oracle's clustering and index vectors:
  1. the GPU's selection equals the oracle's rule applied to the GPU's own
     fp32 scores, bit for bit;
  2. GPU scores match the oracle's fp64 scores within the fp32 error bound;
  3. the GPU set equals the oracle's set, except where the units that differ
     sit within that bound of the cut (counted; expected 0).
"""
import numpy as np
import pytest
import torch

import long_context_kv_kmeans_amd as kvc
import workloads as wl
from oracle import select as osel
from tests.gpu_util import make_pool, oracle_clustering, pool_from_labels, to_dev

pytestmark = pytest.mark.gpu


def _run_select(pool, q_d, budget, sel_cap, flag=None, sel=None):
    B, H = pool.batch, pool.n_kv_heads
    if sel is None:
        sel = (torch.full((B, H, sel_cap), -7, dtype=torch.int32, device="cuda"),
               torch.full((B, H), -7, dtype=torch.int32, device="cuda"),
               torch.full((B, H), -7, dtype=torch.int32, device="cuda"))
    scores = torch.zeros(B, H, pool.unit_cap, dtype=torch.float32, device="cuda")
    spans = torch.full((B, H, sel_cap, 2), -9, dtype=torch.int32, device="cuda")
    kvc.kv_select(pool, q_d, budget, flag, sel[0], sel[1], sel[2], scores_out=scores,
                  sel_spans=spans)
    torch.cuda.synchronize()
    # row spans: (unit_start, unit_size) of each selected id, at the same positions
    su, sn, sp = sel[0].cpu().numpy(), sel[1].cpu().numpy(), spans.cpu().numpy()
    ust, usz = pool.unit_start.cpu().numpy(), pool.unit_size.cpu().numpy()
    fl = None if flag is None else flag.cpu().numpy()
    for b in range(B):
        for g in range(H):
            if fl is not None and fl[b] == 0:
                assert (sp[b, g] == -9).all()
                continue
            ids = su[b, g, :sn[b, g]]
            np.testing.assert_array_equal(sp[b, g, :sn[b, g], 0], ust[b, g, ids])
            np.testing.assert_array_equal(sp[b, g, :sn[b, g], 1], usz[b, g, ids])
    return sel, scores


def _score_bound(q_group, index):
    # |fp32 - exact| <= ~ (d + G) * 2^-24 * sum_e |qsum_e idx_e| + rounding of qsum
    qs = np.abs(np.asarray(q_group, np.float64)).sum(0)
    return 4e-6 * (np.abs(index) @ qs) + 1e-30


def _check_case(cfg, keys, values, labels, cents, queries, budget):
    B, H, N, d = keys.shape
    pool, _, _ = pool_from_labels(keys, values, labels, cents, cfg.dtype)
    sel_cap = max(1, min(budget, cfg.n_clusters))
    G = cfg.group
    from oracle.precision import to_storage
    near_ties = 0
    for qi in range(queries.shape[0]):
        q = queries[qi]  # [B, Hq, d]
        (su, sn, sr), scores = _run_select(pool, to_dev(q, cfg.dtype), budget, sel_cap)
        su, sn, sr, scores = (x.cpu().numpy() for x in (su, sn, sr, scores))
        for b in range(B):
            for g in range(H):
                sizes = np.bincount(labels[b, g], minlength=cfg.n_clusters)
                idx = to_storage(cents[b, g], cfg.dtype)
                gs = scores[b, g, :cfg.n_clusters].astype(np.float64)
                got = su[b, g, :sn[b, g]]
                # (1) the rule on the GPU's own scores, bit-exact
                rule = osel.select_prefix(gs, sizes, budget)
                np.testing.assert_array_equal(got, rule)
                assert sr[b, g] == sizes[got].sum() <= budget
                # (2) scores
                qg = q[b, g * G:(g + 1) * G]
                os_ = osel.group_scores(qg, idx)
                bound = _score_bound(qg, idx)
                assert (np.abs(gs - os_) <= bound).all()
                # (3) sets
                ref = osel.select_prefix(os_, sizes, budget)
                if not np.array_equal(got, ref):
                    diff = np.setxor1d(got, ref)
                    ranked = osel.rank_units(os_, sizes)
                    cut = os_[ranked[len(ref)]] if len(ref) < len(ranked) else -np.inf
                    assert (np.abs(os_[diff] - cut) <= 2 * bound[diff] + 2 * bound.max()).all()
                    near_ties += 1
    return near_ties


@pytest.mark.parametrize("cfg_idx,over,nq", [
    (0, {}, 6),
    (1, dict(n_keys=4096, n_clusters=256, n_components=64, iters=3), 4),
    (4, dict(n_keys=4096, n_clusters=256, n_components=64, iters=3, batch=3), 3),
])
def test_select_parity(cfg_idx, over, nq):
    cfg = wl.get_config(cfg_idx, **over)
    inp = wl.layer_inputs(cfg, 0)
    labels, cents = oracle_clustering(inp["keys"], inp["init_idx"], cfg.iters, cfg.dtype)
    q, _ = wl.layer_queries(cfg, 0, steps=nq)
    # make every query a "retrieval" query: use independent walk states
    near = _check_case(cfg, inp["keys"], inp["values"], labels, cents, q, cfg.budget)
    assert near == 0


def _hand_pool(scores, sizes, d=64, H=1):
    U = len(scores)
    rows = int(np.sum(sizes)) + 1
    pool = make_pool(1, H, d, "fp32", rows, U)
    idx = np.zeros((U, d), np.float32)
    idx[:, 0] = scores
    pool.unit_index[0, :, :U] = torch.from_numpy(idx).cuda()
    starts = np.concatenate([[0], np.cumsum(sizes)[:-1]]).astype(np.int32)
    pool.unit_start[0, :, :U] = torch.from_numpy(starts).cuda()
    pool.unit_size[0, :, :U] = torch.from_numpy(np.asarray(sizes, np.int32)).cuda()
    pool.n_cand.fill_(U)
    pool.n_units.fill_(U)
    pool.n_rows.fill_(rows - 1)
    q = np.zeros((1, H, d), np.float32)
    q[..., 0] = 1.0
    return pool, to_dev(q, "fp32")


def test_select_golden(tiny):
    case = tiny["select"]
    pool, q = _hand_pool(case["scores"], case["sizes"])
    for c in case["cases"]:
        (su, sn, sr), _ = _run_select(pool, q, c["budget"], 5)
        n = int(sn[0, 0])
        assert su[0, 0, :n].cpu().tolist() == c["expect"], c


def test_select_ties_large_and_empty_units():
    rng = np.random.default_rng(3)
    U = 3000
    scores = np.round(rng.standard_normal(U), 1).astype(np.float32)  # many exact ties
    sizes = rng.integers(0, 9, U)
    pool, q = _hand_pool(scores, sizes)
    for budget in [0, 1, 7, 100, 1000, 5000, int(sizes.sum())]:
        cap = max(1, min(budget, U))
        (su, sn, sr), sc = _run_select(pool, q, budget, cap)
        got = su[0, 0, :int(sn[0, 0])].cpu().numpy()
        ref = osel.select_prefix(scores.astype(np.float64), sizes, budget)
        np.testing.assert_array_equal(got, ref)
        assert int(sr[0, 0]) == int(sizes[ref].sum())
    # full budget takes every non-empty unit
    assert got.tolist() == np.nonzero(sizes)[0].tolist()


@pytest.mark.parametrize("case", ["outlier", "infinite", "all_equal", "two_values", "eps_range",
                                  "tiny_range"])
def test_select_score_distributions(case):
    """Score layouts for the selection's first pass (equal-width buckets between
    the lowest and highest score) and its fallbacks: a far outlier that puts
    hundreds of units in the crossing bucket, infinite scores (no value pass),
    all scores equal, two distinct values, and a range so narrow that the
    bucket width is not representable. Bit-exact against the oracle's rule."""
    rng = np.random.default_rng(17)
    U = 3000
    if case == "outlier":
        scores = rng.standard_normal(U).astype(np.float32)
        scores[5] = 1.0e6
    elif case == "infinite":
        scores = rng.standard_normal(U).astype(np.float32)
        scores[7], scores[11] = np.inf, -np.inf
    elif case == "all_equal":
        scores = np.full(U, 0.5, np.float32)
    elif case == "two_values":
        scores = np.where(rng.random(U) < 0.5, 1.0, 2.0).astype(np.float32)
    elif case == "eps_range":
        scores = (1.0 + rng.integers(0, 4, U) * np.finfo(np.float32).eps).astype(np.float32)
    else:  # normal floats whose range is too small for 256 / range to be finite
        scores = (1e-37 * (1.0 + 0.1 * rng.integers(0, 4, U))).astype(np.float32)
    sizes = rng.integers(1, 9, U)
    pool, q = _hand_pool(scores, sizes)
    for budget in [1, 9, 100, 1000, 7000, int(sizes.sum()) - 1]:
        cap = max(1, min(budget, U))
        (su, sn, sr), _ = _run_select(pool, q, budget, cap)
        got = su[0, 0, :int(sn[0, 0])].cpu().numpy()
        ref = osel.select_prefix(scores.astype(np.float64), sizes, budget)
        np.testing.assert_array_equal(got, ref, err_msg=f"{case} budget {budget}")
        assert int(sr[0, 0]) == int(sizes[ref].sum())


def test_select_negative_zero_and_negative_scores():
    scores = np.array([-0.0, 0.0, -1.5, -1.5, 2.0], np.float32)
    sizes = [1, 1, 1, 1, 1]
    pool, q = _hand_pool(scores, sizes)
    for budget in range(6):
        (su, sn, _), _ = _run_select(pool, q, budget, 5)
        ref = osel.select_prefix(scores.astype(np.float64), sizes, budget)
        assert su[0, 0, :int(sn[0, 0])].cpu().tolist() == ref.tolist()


def test_select_flag_zero_keeps_previous():
    pool, q = _hand_pool([1.0, 2.0, 3.0], [1, 1, 1])
    sel, _ = _run_select(pool, q, 2, 3)
    before = [x.clone() for x in sel]
    flag = torch.zeros(1, dtype=torch.uint8, device="cuda")
    q2 = -q
    sel, _ = _run_select(pool, q2.contiguous(), 2, 3, flag=flag, sel=sel)
    for a, b in zip(before, sel):
        assert torch.equal(a, b)
    flag.fill_(1)
    sel, _ = _run_select(pool, q2.contiguous(), 2, 3, flag=flag, sel=sel)
    assert sel[0][0, 0, :int(sel[1][0, 0])].cpu().tolist() == [0, 1]


def test_select_full_size_8192_unit_head():
    """The 36-layer 128K workload's cluster count on one head (8192 units, budget 2048), oracle scores."""
    cfg = wl.get_config(3)
    rng = np.random.default_rng(11)
    C, d = cfg.n_clusters, cfg.head_dim
    cents = rng.standard_normal((1, 1, C, d))
    sizes = np.maximum(1, rng.poisson(16, C))
    sizes[rng.choice(C, 50, replace=False)] = 0
    labels = np.repeat(np.arange(C), sizes)[None, None]
    N = labels.shape[-1]
    keys = wl.to_dtype(rng.standard_normal((1, 1, N, d)), "bf16")
    vals = wl.to_dtype(rng.standard_normal((1, 1, N, d)), "bf16")
    q = wl.to_dtype(rng.standard_normal((3, 1, cfg.group, d)), "bf16")
    sub = cfg.replace(n_kv_heads=1, n_q_heads=cfg.group, n_keys=N)
    assert _check_case(sub, keys, vals, labels, cents, q, cfg.budget) == 0


def test_select_budget_zero_selects_nothing():
    # no unit of positive size fits a zero budget
    pool, q = _hand_pool([1.0, 2.0, 3.0], [1, 2, 3])
    sel, _ = _run_select(pool, q, 0, 3)
    assert int(sel[1][0, 0]) == 0 and int(sel[2][0, 0]) == 0
