"""GPU parity: whole decode loops (boundary -> [segments] -> select -> attend).

LouisKV note, overall-framework flowchart and key designs 1-3. The GPU pool
is packed from the oracle's clustering with the oracle's index vectors, then
both sides run the same seeded query walk:
  * flags bit-exact at every step;
  * segment bookkeeping (long-output config) bit-exact: row/unit counters,
    buffer start, segment start/size;
  * selected unit sets equal the oracle's (near-ties within the fp32 score
    error are counted and must be 0 here);
  * attention output within 2e-3 of exact attention over the GPU's selection
    (which equals the oracle's when the sets agree).
"""
import numpy as np
import pytest
import torch

import workloads as wl
from oracle import attend as oat
from oracle import kmeans as okm
from oracle.decode import run_decode, unit_rows
from tests.gpu_util import gpu_decode, max_rel_err, oracle_clustering, oracle_packs, \
    pool_from_labels, to_dev

pytestmark = pytest.mark.gpu
TOL = 2e-3


def _fixed_clustering(keys, C):
    """Labels k mod C with the oracle's member means: a cheap, valid clustering for
    sequences that only fill the batch and are not checked."""
    B, H, N, d = keys.shape
    labels = np.tile(np.arange(N) % C, (B, H, 1))
    cents = np.empty((B, H, C, d))
    for b in range(B):
        for g in range(H):
            cents[b, g], _ = okm.update(keys[b, g], labels[b, g], np.zeros((C, d)))
    return labels, cents


def _page_units(keys, page):
    """Page-granularity units: key i in unit i // page, indexed by the page's key mean."""
    B, H, N, d = keys.shape
    labels = wl.page_labels(B, H, N, page).astype(np.int64)
    C = -(-N // page)
    cents = np.empty((B, H, C, d))
    for b in range(B):
        for g in range(H):
            cents[b, g], _ = okm.update(keys[b, g], labels[b, g], np.zeros((C, d)))
    return labels, cents


def _run(cfg, steps, seqs, compare_every=1, check=None, policy="boundary", page=None,
         pool_kw=None, clustering="oracle", **decode_kw):
    """check: positions in `seqs` compared with the oracle (default all); the other
    sequences get _fixed_clustering and only fill the launch. policy: when to
    retrieve ("boundary", "per-token", "stride:S"); page: page-granularity units of
    that many keys instead of K-means clusters; pool_kw: extra pool_from_labels
    arguments (host_kv); clustering="fixed": every sequence, checked ones too, gets
    _fixed_clustering (the decode comparison holds for any clustering both sides
    share)."""
    inp = wl.layer_inputs(cfg, 0, seqs=seqs)
    B, H, N, d = inp["keys"].shape
    check = list(range(B)) if check is None else list(check)
    if page is not None:
        labels, cents = _page_units(inp["keys"], page)
        cfg = cfg.replace(n_clusters=cents.shape[2])
    else:
        labels, cents = _fixed_clustering(inp["keys"], cfg.n_clusters)
        if clustering == "oracle":
            lc, cc = oracle_clustering(inp["keys"][check], inp["init_idx"][check], cfg.iters,
                                       cfg.dtype)
            labels[check], cents[check] = lc, cc
    q, _ = wl.layer_queries(cfg, 0, steps=steps, seqs=seqs)
    sched = wl.retrieval_schedule(policy, steps)
    if sched is not None:
        decode_kw["flags"] = torch.from_numpy(
            np.repeat(sched[:, None], B, axis=1).astype(np.uint8)).cuda()
    dk = dv = None
    extra_rows, n_units = 0, cfg.n_clusters
    if cfg.buf_cap > 0:
        dk, dv = wl.layer_decode_kv(cfg, 0, steps=steps, seqs=seqs)
        # unit table: the clusters, then one unit per segment closed (at most one per
        # step), within the selection's limit of 8192 units
        extra_rows, n_units = steps, cfg.n_clusters + min(steps, 8192 - cfg.n_clusters)
    pool, _, _ = pool_from_labels(inp["keys"], inp["values"], labels, cents, cfg.dtype,
                                  n_units=n_units, buf_cap=cfg.buf_cap, extra_rows=extra_rows,
                                  **(pool_kw or {}))
    sel_cap = min(cfg.budget, n_units)
    rec = gpu_decode(pool, to_dev(q, cfg.dtype), cfg.tau, cfg.budget, cfg.scale, sel_cap,
                     dec_k=None if dk is None else to_dev(dk, cfg.dtype),
                     dec_v=None if dv is None else to_dev(dv, cfg.dtype), **decode_kw)
    flags = rec.flag.cpu().numpy().astype(bool)
    out = rec.out.cpu().numpy()
    sel_n = rec.sel_n.cpu().numpy()
    sel = rec.sel.cpu().numpy()
    counters = rec.counters.cpu().numpy()
    G = cfg.group
    stats = {"retrievals": 0, "set_mismatch": 0, "max_err": 0.0}
    for bi in check:
        packs = oracle_packs(inp["keys"], inp["values"], labels, cents, cfg.dtype, bi)
        # the reference attention below is exact attention over the GPU's selection
        # (equal to the oracle's, which is checked), so the loop's own outputs are
        # not needed
        log, opool = run_decode(packs, q[:, bi], cfg.tau, cfg.budget, cfg.scale, cfg.dtype,
                                buf_cap=cfg.buf_cap,
                                dec_k=None if dk is None else dk[:, bi],
                                dec_v=None if dv is None else dv[:, bi], retrieve=sched,
                                attend_steps=np.zeros(steps, dtype=bool))
        for t, e in enumerate(log):
            assert flags[t, bi] == e["flag"], (t, bi)
            if cfg.buf_cap > 0:
                assert counters[t, :, bi].tolist() == [e["n_rows"], cfg.n_clusters + len(
                    [s for s in opool.seg.seg_start if s < e["seg_begin"]]), e["n_cand"],
                    e["buf_begin"], e["seg_begin"]], t
            stats["retrievals"] += int(e["flag"])
            if t % compare_every and not e["flag"]:
                continue
            for g in range(H):
                got = sel[t, bi, g, :sel_n[t, bi, g]]
                if not np.array_equal(got, e["sel"][g]):
                    stats["set_mismatch"] += 1
                start, size, _ = opool.unit_table(g)
                rows = unit_rows(start, size, got)
                if cfg.buf_cap > 0:
                    rows = np.concatenate([rows, np.arange(e["buf_begin"], e["n_rows"])])
                K, V = opool.rows(g, rows)
                ref = oat.attend_exact(q[t, bi, g * G:(g + 1) * G], K, V, cfg.scale)
                err = max_rel_err(out[t, bi, g * G:(g + 1) * G], ref)
                stats["max_err"] = max(stats["max_err"], err)
                assert err <= TOL, (t, bi, g, err)
        if cfg.buf_cap > 0:
            # segment tables: ids C.. in closing order, bit-exact rows
            st = opool.seg
            ns = len(st.seg_start)
            us = pool.unit_start[bi, 0, cfg.n_clusters:cfg.n_clusters + ns].cpu().numpy()
            uz = pool.unit_size[bi, 0, cfg.n_clusters:cfg.n_clusters + ns].cpu().numpy()
            assert us.tolist() == st.seg_start and uz.tolist() == st.seg_size
            um = pool.unit_mean[bi, :, cfg.n_clusters:cfg.n_clusters + ns].cpu().numpy()
            om = np.stack(st.seg_mean, axis=1)  # [H, ns, d]
            assert np.abs(um - om).max() <= 1e-5 * max(1.0, np.abs(om).max())
    print(stats)
    assert stats["set_mismatch"] == 0
    return stats


@pytest.mark.parametrize("cfg_idx,over,steps,seqs", [
    (0, {}, 64, [0]),
    (1, dict(n_keys=8192, n_clusters=512, n_components=128, iters=3), 96, [0]),
    (4, dict(n_keys=4096, n_clusters=256, n_components=64, iters=3), 48, [0, 5]),
])
def test_decode_loop_parity(cfg_idx, over, steps, seqs):
    cfg = wl.get_config(cfg_idx, **over)
    st = _run(cfg, steps, seqs)
    assert st["retrievals"] >= 1


@pytest.mark.parametrize("attend", ["step", "wset", "pool"])
def test_decode_full_size_qwen3_layer_32k_benchmark_path(attend):
    # the Qwen3-8B-shaped layer at full size (8 KV heads x 32768 keys, C = 2048, 256 steps)
    # through the calls the benchmark times: kv_boundary_select with row spans, then
    # kv_fetch_attend over an HBM working set (the default) or kv_gather_attend on the
    # spans (bench.py --attend pool). Two Lloyd rounds suffice: the clustering only sets
    # up the pool, and full-size K-means has its own sampled test.
    cfg = wl.get_config(1, iters=2)
    kw = (dict(fetch="fused", fused=True) if attend == "wset" else
          dict(fetch="step") if attend == "step" else dict(fused=True))
    st = _run(cfg, cfg.steps, [0], compare_every=8, spans=True, **kw)
    assert st["retrievals"] >= 2


@pytest.mark.parametrize("attend", ["step", "wset", "pool"])
def test_decode_full_size_batch16_32k_benchmark_path(attend):
    # batched decode at full size: 16 sequences x 8 KV heads x 32768 keys in one launch,
    # budget 1024; sequences 0 and 9 carry the oracle's clustering and are checked
    cfg = wl.get_config(4, iters=2)
    kw = (dict(fetch="fused", fused=True) if attend == "wset" else
          dict(fetch="step") if attend == "step" else dict(fused=True))
    st = _run(cfg, 128, list(range(16)), compare_every=8, check=[0, 9], spans=True, **kw)
    assert st["retrievals"] >= 2


@pytest.mark.parametrize("attend", ["step", "wset", "pool"])
def test_decode_full_size_128k_layer_shape(attend):
    # one layer of the long-input long-output workload at full size: 8 KV heads x 131072
    # keys, 8192 units, budget 2048, 1024 steps, through the benchmark's calls.
    # Both sides get the same fixed clustering (key i in unit i mod 8192, indexed by the
    # members' mean): the decode comparison does not depend on how the pool was
    # clustered, and Lloyd at this size in the fp64 oracle would take hours (full-size
    # K-means has its own sampled test).
    cfg = wl.get_config(3)
    kw = (dict(fetch="fused", fused=True) if attend == "wset" else
          dict(fetch="step") if attend == "step" else dict(fused=True))
    st = _run(cfg, cfg.steps, [0], compare_every=16, clustering="fixed", spans=True, **kw)
    assert st["retrievals"] >= 2


def test_decode_long_output_segments_small_buffer():
    # long-output config with a small buffer so eviction and forced closes occur often
    cfg = wl.get_config(2, buf_cap=64, steps=600, p_jump=0.05, budget=256, iters=3)
    _run(cfg, cfg.steps, [0])


def test_decode_long_output_segments():
    cfg = wl.get_config(2, iters=3)
    _run(cfg, 3000, [0], compare_every=7)


def test_decode_long_output_benchmark_path():
    # the long-output workload through the benchmark's calls (kv_boundary_segment_append,
    # kv_select with row spans, kv_gather_attend on the spans) for all of its 16384
    # steps: ~330 boundaries, the 1024-token buffer full and evicting segments from step
    # ~1024 on. Flags and segment counters are compared at every step, the selection
    # and the attention output at every retrieval step and every 64th step.
    cfg = wl.get_config(2, iters=3)
    st = _run(cfg, cfg.steps, [0], compare_every=64, fused_append=True, spans=True)
    assert st["retrievals"] >= 250


@pytest.mark.parametrize("cfg_idx,over,steps,seqs", [
    (0, {}, 64, [0]),
    (1, dict(n_keys=8192, n_clusters=512, n_components=128, iters=3), 96, [0]),
    (4, dict(n_keys=4096, n_clusters=256, n_components=64, iters=3), 48, [0, 5]),
])
def test_fused_boundary_select_matches_separate_calls(cfg_idx, over, steps, seqs):
    # kv_boundary_select == kv_boundary followed by kv_select, bit for bit
    cfg = wl.get_config(cfg_idx, **over)
    inp = wl.layer_inputs(cfg, 0, seqs=seqs)
    labels, cents = oracle_clustering(inp["keys"], inp["init_idx"], cfg.iters, cfg.dtype)
    q, _ = wl.layer_queries(cfg, 0, steps=steps, seqs=seqs)
    pool, _, _ = pool_from_labels(inp["keys"], inp["values"], labels, cents, cfg.dtype,
                                  n_units=cfg.n_clusters)
    sel_cap = min(cfg.budget, cfg.n_clusters)
    qd = to_dev(q, cfg.dtype)
    a = gpu_decode(pool, qd, cfg.tau, cfg.budget, cfg.scale, sel_cap)
    assert int(a.flag.sum()) >= 2
    # fused boundary+select, with and without row spans handed to the attention
    for kw in (dict(fused=True), dict(fused=True, spans=True)):
        b = gpu_decode(pool, qd, cfg.tau, cfg.budget, cfg.scale, sel_cap, **kw)
        for name in ("flag", "sel_n", "sel"):
            assert torch.equal(getattr(a, name), getattr(b, name)), (kw, name)
        ra, rb = a.r.cpu().numpy(), b.r.cpu().numpy()
        assert np.isnan(ra[0]).all() and np.isnan(rb[0]).all()
        np.testing.assert_array_equal(ra[1:].view(np.uint32), rb[1:].view(np.uint32))
        np.testing.assert_array_equal(a.out.cpu().numpy().view(np.uint32),
                                      b.out.cpu().numpy().view(np.uint32))


def test_decode_segments_spans_and_fused_append_match_separate_calls():
    # long-output config: spans written by kv_select (segments included) give the
    # same attention as the unit-table lookup, and kv_boundary_segment_append the
    # same flags, r, segment bookkeeping and outputs as kv_boundary +
    # kv_segment_append, bit for bit
    cfg = wl.get_config(2, buf_cap=64, steps=300, p_jump=0.05, budget=256, iters=3)
    inp = wl.layer_inputs(cfg, 0)
    labels, cents = oracle_clustering(inp["keys"], inp["init_idx"], cfg.iters, cfg.dtype)
    q, _ = wl.layer_queries(cfg, 0, steps=cfg.steps)
    dk, dv = wl.layer_decode_kv(cfg, 0, steps=cfg.steps)
    n_units = cfg.n_clusters + cfg.steps
    sel_cap = min(cfg.budget, n_units)
    outs = []
    # unit lookup; spans; spans + boundary test fused into the segment append
    for kw in (dict(), dict(spans=True), dict(spans=True, fused_append=True)):
        pool, _, _ = pool_from_labels(inp["keys"], inp["values"], labels, cents, cfg.dtype,
                                      n_units=n_units, buf_cap=cfg.buf_cap, extra_rows=cfg.steps)
        rec = gpu_decode(pool, to_dev(q, cfg.dtype), cfg.tau, cfg.budget, cfg.scale, sel_cap,
                         dec_k=to_dev(dk, cfg.dtype), dec_v=to_dev(dv, cfg.dtype), **kw)
        outs.append(rec)
    for o in outs[1:]:
        for name in ("flag", "sel_n", "sel", "counters"):
            assert torch.equal(outs[0].__dict__[name], o.__dict__[name]), name
        ra, rb = outs[0].r.cpu().numpy(), o.r.cpu().numpy()
        np.testing.assert_array_equal(ra[1:].view(np.uint32), rb[1:].view(np.uint32))
        assert np.isnan(rb[0]).all()
        np.testing.assert_array_equal(outs[0].out.cpu().numpy().view(np.uint32),
                                      o.out.cpu().numpy().view(np.uint32))


def test_segment_append_capacity_errors_are_reported():
    # out of rows: the status word says so, the sequence's step is skipped and
    # nothing is written past row_cap; out of units likewise when a close is due
    import long_context_kv_kmeans_amd as kvc
    from tests.gpu_util import make_pool
    d, H = 64, 2
    pool = make_pool(1, H, d, "fp32", 10, 4, buf_cap=4, extra_rows=2)  # row_cap 12
    pool.n_rows.fill_(10)
    pool.n_units.fill_(2)
    pool.n_cand.fill_(2)
    pool.buf_begin.fill_(10)
    pool.seg_begin.fill_(10)
    kt = torch.ones(1, H, d, device="cuda")
    flag = torch.zeros(1, dtype=torch.uint8, device="cuda")
    for _ in range(3):
        kvc.kv_segment_append(pool, kt, kt, flag)
    torch.cuda.synchronize()
    assert int(pool.status.item()) == kvc.KV_ERR_CAPACITY
    assert int(pool.n_rows.item()) == 12
    # units: a boundary with a full unit table
    pool2 = make_pool(1, H, d, "fp32", 10, 2, buf_cap=4, extra_rows=8)
    pool2.n_rows.fill_(12)
    pool2.n_units.fill_(2)
    pool2.n_cand.fill_(2)
    pool2.buf_begin.fill_(10)
    pool2.seg_begin.fill_(10)
    flag.fill_(1)
    kvc.kv_segment_append(pool2, kt, kt, flag)
    torch.cuda.synchronize()
    assert int(pool2.status.item()) == kvc.KV_ERR_CAPACITY
    assert int(pool2.n_rows.item()) == 12 and int(pool2.n_units.item()) == 2


def test_decode_128k_two_layers_through_captured_graphs():
    """Two layers of the 36-layer long-input long-output workload (131072 keys per KV
    head, 8192 units, budget 2048), each with its own keys, pool, working set and
    query walk, through the benchmark's launch configuration: every decode step
    runs kv_decode_step (boundary test, selection, working-set fetch and attention
    in one launch) for layer 0 then layer 1, captured into HIP graphs and replayed. Each layer is compared with its own oracle loop:
    flags and selected sets at every step, attention at every retrieval step and
    every 16th step. Both sides use the fixed clustering of the one-layer test."""
    import long_context_kv_kmeans_amd as kvc
    from tests.gpu_util import working_set
    cfg = wl.get_config(3)
    L, T, C = 2, cfg.steps, cfg.n_clusters
    sel_cap = min(cfg.budget, C)
    stream = torch.cuda.Stream()

    class Layer:
        pass

    layers = []
    for li in range(L):
        y = Layer()
        inp = wl.layer_inputs(cfg, li, threads=8)
        y.keys, y.vals = inp["keys"], inp["values"]
        y.labels, y.cents = _fixed_clustering(inp["keys"], C)
        y.q, _ = wl.layer_queries(cfg, li)
        y.pool, _, _ = pool_from_labels(y.keys, y.vals, y.labels, y.cents, cfg.dtype, n_units=C)
        y.qd = to_dev(y.q, cfg.dtype)
        B, H, Hq, d = 1, cfg.n_kv_heads, cfg.n_q_heads, cfg.head_dim
        z = lambda *s: torch.zeros(*s, dtype=torch.int32, device="cuda")  # noqa: E731
        y.sel, y.sel_n, y.sel_rows, y.spans = z(B, H, sel_cap), z(B, H), z(B, H), z(B, H, sel_cap, 2)
        y.flags = torch.zeros(T, B, dtype=torch.uint8, device="cuda")
        y.out = torch.zeros(B, Hq, d, dtype=torch.float32, device="cuda")
        y.wset = working_set(y.pool, cfg.budget)
        y.ws_step = kvc.workspace(kvc.kv_decode_step_workspace(y.pool, Hq, cfg.budget))
        y.rec_out = torch.zeros(T, B, Hq, d, dtype=torch.float32, device="cuda")
        y.rec_sel = z(T, B, H, sel_cap)
        y.rec_n = z(T, B, H)
        layers.append(y)

    def step(t):
        for y in layers:
            kvc.kv_decode_step(y.pool, y.qd[t - 1] if t else None, y.qd[t], cfg.tau,
                               cfg.scale, cfg.budget, y.flags[t], y.sel, y.spans, y.sel_n,
                               y.sel_rows, y.wset, y.wset.spans, y.wset.count, y.out,
                               ws=y.ws_step)
            y.rec_out[t].copy_(y.out)
            y.rec_sel[t].copy_(y.sel)
            y.rec_n[t].copy_(y.sel_n)

    with torch.cuda.stream(stream):
        step(0)  # loads the kernels; the replay starts again from step 0
    torch.cuda.synchronize()
    graphs = []
    for t0 in range(0, T, 128):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for t in range(t0, min(T, t0 + 128)):
                step(t)
        graphs.append(g)
    for g in graphs:
        g.replay()
    torch.cuda.synchronize()

    G = cfg.group
    for li, y in enumerate(layers):
        assert int(y.pool.status.item()) == 0
        flags = y.flags.cpu().numpy().astype(bool)[:, 0]
        sel, sel_n = y.rec_sel.cpu().numpy()[:, 0], y.rec_n.cpu().numpy()[:, 0]
        out = y.rec_out.cpu().numpy()[:, 0]
        packs = oracle_packs(y.keys, y.vals, y.labels, y.cents, cfg.dtype, 0)
        log, opool = run_decode(packs, y.q[:, 0], cfg.tau, cfg.budget, cfg.scale, cfg.dtype,
                                attend_steps=np.zeros(T, dtype=bool))
        assert flags.sum() >= 2, li
        for t, e in enumerate(log):
            assert flags[t] == e["flag"], (li, t)
            for g in range(H):
                got = sel[t, g, :sel_n[t, g]]
                assert np.array_equal(got, e["sel"][g]), (li, t, g)
            if t % 16 and not e["flag"]:
                continue
            for g in range(H):
                start, size, _ = opool.unit_table(g)
                K, V = opool.rows(g, unit_rows(start, size, e["sel"][g]))
                ref = oat.attend_exact(y.q[t, 0, g * G:(g + 1) * G], K, V, cfg.scale)
                err = max_rel_err(out[t, g * G:(g + 1) * G], ref)
                assert err <= TOL, (li, t, g, err)
        # the two layers are different workloads: their walks retrieve at different steps
        if li == 1:
            assert not np.array_equal(flags, layers[0].flags.cpu().numpy().astype(bool)[:, 0])


@pytest.mark.parametrize("cfg_idx,over,steps,seqs,host", [
    (1, dict(n_keys=8192, n_clusters=512, n_components=128, iters=3), 96, [0], False),
    (1, dict(n_keys=8192, n_clusters=512, n_components=128, iters=3, p_jump=0.3), 40, [0], True),
    (1, dict(n_keys=3000, n_clusters=100, n_components=20, head_dim=64, n_q_heads=16,
             iters=3, p_jump=0.2), 48, [0], False),
    (1, dict(n_keys=2500, n_clusters=300, n_components=40, n_q_heads=64, iters=3,
             p_jump=0.2), 48, [0], False),
    (4, dict(n_keys=4096, n_clusters=256, n_components=64, iters=3, p_jump=0.2), 48, [0, 5, 9],
     False),
    (3, dict(n_keys=20000, n_clusters=8192, n_components=1024, iters=1, p_jump=0.2), 48, [0],
     False),
])
def test_decode_step_one_launch_equals_two_launches(cfg_idx, over, steps, seqs, host):
    """kv_decode_step == kv_boundary_select followed by kv_fetch_attend (max_rows =
    budget), bit for bit: flags, r, selections, spans, working sets and outputs, for
    group sizes 2, 4, 8, head dims 64 and 128, batches, a pool in host memory, many
    retrievals, and 8192 units (the largest selection, 16 keys per thread)."""
    cfg = wl.get_config(cfg_idx, **over)
    inp = wl.layer_inputs(cfg, 0, seqs=seqs)
    labels, cents = _fixed_clustering(inp["keys"], cfg.n_clusters)
    q, _ = wl.layer_queries(cfg, 0, steps=steps, seqs=seqs)
    qd = to_dev(q, cfg.dtype)
    sel_cap = min(cfg.budget, cfg.n_clusters)
    recs = []
    for kw in (dict(fused=True, spans=True, fetch="fused"), dict(fetch="step")):
        pool, _, _ = pool_from_labels(inp["keys"], inp["values"], labels, cents, cfg.dtype,
                                      n_units=cfg.n_clusters, host_kv=host)
        recs.append(gpu_decode(pool, qd, cfg.tau, cfg.budget, cfg.scale, sel_cap, **kw))
        assert int(pool.status.item()) == 0
    a, b = recs
    assert int(a.flag.sum()) >= 3  # the first step and at least two jumps
    for name in ("flag", "sel_n", "sel"):
        assert torch.equal(getattr(a, name), getattr(b, name)), name
    ra, rb = a.r.cpu().numpy(), b.r.cpu().numpy()
    np.testing.assert_array_equal(ra[1:].view(np.uint32), rb[1:].view(np.uint32))
    assert np.isnan(rb[0]).all()
    np.testing.assert_array_equal(a.out.cpu().numpy().view(np.uint32),
                                  b.out.cpu().numpy().view(np.uint32))
    assert torch.equal(a.wset.k, b.wset.k) and torch.equal(a.wset.spans, b.wset.spans)
    assert torch.equal(a.wset.count, b.wset.count)
