"""Pins of the oracle's decode-time segments and of the composed decode loop.

Segments: LouisKV note, key design 2 (decode half). Decode loop: the
"Overall framework" flowchart. Checks: a hand-traced fixture, invariants
(partition, buffer bound, key-mean index), and the full-budget special case,
where budgeted retrieval must reproduce dense attention over every row.
"""
import numpy as np
import pytest

from oracle import attend, kmeans
from oracle.decode import run_decode
from oracle.segments import SegmentState


def test_segments_golden(tiny):
    c = tiny["segments"]
    st = SegmentState(c["n_prefill"], c["n_clusters"], c["buf_cap"], 1, 2, len(c["flags"]), "fp32")
    for t, f in enumerate(c["flags"]):
        st.step(bool(f), np.full((1, 2), float(t)), np.zeros((1, 2)))
    segs = [[s, z] for s, z in zip(st.seg_start, st.seg_size)]
    assert segs == c["expect_segments"]
    assert st.n_evicted == c["expect_n_evicted"]
    assert st.buf_begin == c["expect_buf_begin"]
    assert st.seg_begin == c["expect_seg_begin"]
    assert st.n_rows == c["expect_n_rows"]
    assert st.n_units_pool == c["n_clusters"] + c["expect_n_evicted"]
    # index of segment [10, 13) = mean of the keys appended at t = 0, 1, 2
    np.testing.assert_allclose(st.seg_mean[0][0], [1.0, 1.0])


@pytest.mark.parametrize("seed,cap,p", [(0, 16, 0.05), (1, 8, 0.3), (2, 64, 0.01), (3, 5, 0.0)])
def test_segment_invariants(seed, cap, p):
    rng = np.random.default_rng(seed)
    steps, H, d, n0 = 400, 3, 4, 50
    st = SegmentState(n0, 7, cap, H, d, steps, "bf16")
    keys = rng.standard_normal((steps, H, d))
    flags = rng.random(steps) < p
    flags[0] = True
    for t in range(steps):
        st.step(bool(flags[t]), keys[t], keys[t] * 0)
        assert st.n_rows - st.buf_begin <= cap
        # every decode row lies in exactly one place: an evicted segment or the buffer
        covered = []
        for j in range(st.n_evicted):
            covered.extend(range(st.seg_start[j], st.seg_start[j] + st.seg_size[j]))
        covered.extend(range(st.buf_begin, st.n_rows))
        assert covered == list(range(n0, st.n_rows))
    # segments partition a time-ordered prefix of the decode rows
    pos = n0
    for s, z, m in zip(st.seg_start, st.seg_size, st.seg_mean):
        assert s == pos and 1 <= z <= cap
        ref = [[sum(keys[i - n0, h, j] for i in range(s, s + z)) / z for j in range(d)] for h in range(H)]
        np.testing.assert_allclose(m, ref, rtol=1e-12)
        pos += z
    assert pos == st.seg_begin


def _tiny_pool(seed, H=2, N=96, d=8, C=6, dtype="fp32"):
    rng = np.random.default_rng(seed)
    packs = []
    for g in range(H):
        x = rng.standard_normal((N, d))
        v = rng.standard_normal((N, d))
        out = kmeans.lloyd(x, rng.choice(N, C, replace=False), 4)
        packs.append(kmeans.pack(x, v, out["labels"], out["centroids"], dtype))
    return packs


def test_full_budget_equals_dense_attention():
    packs = _tiny_pool(10)
    rng = np.random.default_rng(11)
    q = rng.standard_normal((12, 4, 8))  # G = 2
    log, _ = run_decode(packs, q, 0.7, budget=10 ** 6, scale=0.3, dtype="fp32")
    for t, e in enumerate(log):
        for g in range(2):
            dense = attend.attend_exact(q[t, 2 * g:2 * g + 2], packs[g]["k"], packs[g]["v"], 0.3)
            np.testing.assert_allclose(e["out"][2 * g:2 * g + 2], dense, rtol=1e-12, atol=1e-14)


def test_full_budget_with_segments_equals_dense():
    packs = _tiny_pool(12)
    rng = np.random.default_rng(13)
    T = 40
    q = rng.standard_normal((T, 4, 8))
    dk = rng.standard_normal((T, 2, 8))
    dv = rng.standard_normal((T, 2, 8))
    log, _ = run_decode(packs, q, 0.7, budget=10 ** 6, scale=0.3, dtype="fp32", buf_cap=5,
                        dec_k=dk, dec_v=dv)
    for t, e in enumerate(log):
        if not e["flag"]:
            continue  # reused sets may miss segments evicted since the last retrieval
        for g in range(2):
            K = np.concatenate([packs[g]["k"], dk[:t + 1, g]])
            V = np.concatenate([packs[g]["v"], dv[:t + 1, g]])
            dense = attend.attend_exact(q[t, 2 * g:2 * g + 2], K, V, 0.3)
            np.testing.assert_allclose(e["out"][2 * g:2 * g + 2], dense, rtol=1e-11, atol=1e-13)


def test_decode_reuses_selection_between_boundaries():
    packs = _tiny_pool(14)
    rng = np.random.default_rng(15)
    base = rng.standard_normal((4, 8))
    q = np.stack([base + 0.01 * rng.standard_normal((4, 8)) for _ in range(10)])
    q[6] = rng.standard_normal((4, 8))  # a jump
    log, _ = run_decode(packs, q, 0.7, budget=20, scale=0.3, dtype="fp32")
    flags = [e["flag"] for e in log]
    assert flags[0] and flags[6]
    for t in range(1, 10):
        if not flags[t]:
            for g in range(2):
                assert log[t]["sel"][g].tolist() == log[t - 1]["sel"][g].tolist()
    for e in log:
        for g in range(2):
            assert packs[g]["unit_size"][e["sel"][g]].sum() <= 20


def _walk(seed, T=30):
    rng = np.random.default_rng(seed)
    base = rng.standard_normal((4, 8))
    q = []
    for t in range(T):
        if t and rng.random() < 0.15:
            base = rng.standard_normal((4, 8))
        base = base + 0.05 * rng.standard_normal((4, 8))
        q.append(base.copy())
    return np.stack(q)


def test_retrieval_schedule_replaces_only_the_decision():
    packs = _tiny_pool(16)
    q = _walk(17)
    ref, _ = run_decode(packs, q, 0.7, budget=20, scale=0.3, dtype="fp32")
    flags = np.array([e["flag"] for e in ref])
    assert flags.sum() >= 2 and not flags.all()
    # the boundary test's own decisions as a schedule: the same loop
    same, _ = run_decode(packs, q, 0.7, budget=20, scale=0.3, dtype="fp32", retrieve=flags)
    for a, b in zip(ref, same):
        assert a["flag"] == b["flag"]
        np.testing.assert_array_equal(a["r"], b["r"])  # NaN at the first step on both
        assert all(np.array_equal(x, y) for x, y in zip(a["sel"], b["sel"]))
        np.testing.assert_array_equal(a["out"], b["out"])
    with pytest.raises(ValueError):
        run_decode(packs, q, 0.7, budget=20, scale=0.3, dtype="fp32", buf_cap=4,
                   dec_k=np.zeros((30, 2, 8)), dec_v=np.zeros((30, 2, 8)), retrieve=flags)


def test_per_token_and_fixed_stride_retrieval():
    # per-token: every step selects from its own query alone (a one-step loop,
    # whose first step always retrieves, gives the same set); fixed stride S:
    # steps between multiples of S reuse the set of the last multiple
    packs = _tiny_pool(18)
    q = _walk(19)
    T = q.shape[0]
    fresh = [run_decode(packs, q[t:t + 1], 0.7, budget=20, scale=0.3, dtype="fp32")[0][0]
             for t in range(T)]
    per_tok, _ = run_decode(packs, q, 0.7, budget=20, scale=0.3, dtype="fp32",
                            retrieve=np.ones(T, bool))
    boundary, _ = run_decode(packs, q, 0.7, budget=20, scale=0.3, dtype="fp32")
    differs = False
    for t in range(T):
        assert per_tok[t]["flag"]
        for g in range(2):
            assert per_tok[t]["sel"][g].tolist() == fresh[t]["sel"][g].tolist()
            differs |= per_tok[t]["sel"][g].tolist() != boundary[t]["sel"][g].tolist()
        np.testing.assert_array_equal(per_tok[t]["out"], fresh[t]["out"])
    assert differs  # reusing sets between boundaries is not per-token retrieval here
    S = 4
    stride, _ = run_decode(packs, q, 0.7, budget=20, scale=0.3, dtype="fp32",
                           retrieve=np.arange(T) % S == 0)
    for t in range(T):
        assert stride[t]["flag"] == (t % S == 0)
        src = fresh[t - t % S]
        for g in range(2):
            assert stride[t]["sel"][g].tolist() == src["sel"][g].tolist()


def test_page_units_keep_time_order():
    # pages of P consecutive keys: the CSR pack is the identity permutation,
    # unit u spans rows [u P, min((u + 1) P, N)), indexed by the page's key mean
    rng = np.random.default_rng(20)
    N, d, P = 50, 8, 8
    x = rng.standard_normal((N, d))
    v = rng.standard_normal((N, d))
    labels = np.arange(N) // P
    C = -(-N // P)
    cents, counts = kmeans.update(x, labels, np.zeros((C, d)))
    pk = kmeans.pack(x, v, labels, cents, "fp32")
    np.testing.assert_array_equal(pk["k"], x)
    np.testing.assert_array_equal(pk["v"], v)
    assert pk["unit_start"].tolist() == list(range(0, N, P))
    assert pk["unit_size"].tolist() == [P] * (C - 1) + [N - P * (C - 1)]
    np.testing.assert_allclose(cents[-1], x[P * (C - 1):].mean(0), rtol=1e-15, atol=0)


def test_attention_on_chosen_steps_only_changes_nothing_else():
    # skipping the attention output on some steps leaves every other logged
    # quantity (flags, selections, segment counters) and the computed outputs
    # exactly as in the full loop
    packs = _tiny_pool(20)
    rng = np.random.default_rng(21)
    T = 30
    q = _walk(22, T)
    dk = rng.standard_normal((T, 2, 8))
    dv = rng.standard_normal((T, 2, 8))
    kw = dict(budget=20, scale=0.3, dtype="fp32", buf_cap=5, dec_k=dk, dec_v=dv)
    full, _ = run_decode(packs, q, 0.7, **kw)
    at = np.arange(T) % 4 == 1
    part, _ = run_decode(packs, q, 0.7, attend_steps=at, **kw)
    for t, (a, b) in enumerate(zip(full, part)):
        for k in ("flag", "n_cand", "n_rows", "buf_begin", "seg_begin"):
            assert a[k] == b[k], (t, k)
        assert all(np.array_equal(x, y) for x, y in zip(a["sel"], b["sel"]))
        if at[t]:
            np.testing.assert_array_equal(a["out"], b["out"])
        else:
            assert b["out"] is None
