"""Pins of the oracle's K-means against what the definition fixes.

Lloyd's iteration with centroid = member mean (LouisKV note, key design 2).
Every check is independent of the oracle's own code path: brute force in
pure Python, closed forms, invariants, and hand-derived fixtures.
"""
import itertools
import math

import numpy as np
import pytest

from oracle import kmeans as km
from oracle.precision import round_bf16


def _mixture(seed, n, d, n_comp, sigma):
    rng = np.random.default_rng(seed)
    means = rng.standard_normal((n_comp, d))
    comp = rng.integers(0, n_comp, n)
    return means[comp] + sigma * rng.standard_normal((n, d)), comp, means


def _pure_sqdist(x, c):
    return sum((a - b) ** 2 for a, b in zip(x, c))


def test_golden_1d(tiny):
    case = tiny["kmeans_1d"]
    out = km.lloyd(np.array(case["keys"]), case["init_idx"], case["iters"])
    assert out["labels"].tolist() == case["expect_labels"]
    np.testing.assert_allclose(out["centroids"], case["expect_centroids"], rtol=1e-15)
    J = km.objective(np.array(case["keys"]), out["labels"], out["centroids"])
    assert J == pytest.approx(case["expect_objective"], rel=1e-14)


def test_golden_tie_lowest_index(tiny):
    case = tiny["kmeans_tie"]
    assert km.assign(np.array(case["keys"]), np.array(case["centroids"])).tolist() == [case["expect_label"]]


def test_golden_parity_flip(tiny):
    case = tiny["kmeans_parity_flip"]
    keys, cents = np.array(case["keys"]), np.array(case["centroids"])
    exact = km.assign(keys, km.centroid_for_distance(cents, "exact", "bf16"))
    parity = km.assign(keys, km.centroid_for_distance(cents, "parity", "bf16"))
    assert exact.tolist() == [case["expect_exact_label"]]
    assert parity.tolist() == [case["expect_parity_bf16_label"]]


def test_golden_empty_cluster_keeps_centroid(tiny):
    case = tiny["kmeans_empty"]
    keys = np.array(case["keys"])
    init = np.array(case["init_centroids"])
    labels = km.assign(keys, init)
    new, counts = km.update(keys, labels, init)
    np.testing.assert_array_equal(new, case["expect_centroids"])
    assert counts.tolist() == case["expect_counts"]


def test_objective_non_increasing():
    x, _, _ = _mixture(1, 600, 16, 12, 0.6)
    init = np.random.default_rng(2).choice(600, 20, replace=False)
    out = km.lloyd(x, init, 15, history=True)
    Js = []
    prev_c = x[init]
    for c_before, labels, c_after in out["history"]:
        # assignment step cannot raise J for fixed centroids ...
        J_assign = km.objective(x, labels, c_before)
        if Js:
            assert J_assign <= Js[-1] * (1 + 1e-12)
        # ... and the mean step cannot raise it for fixed labels
        J_update = km.objective(x, labels, c_after)
        assert J_update <= J_assign * (1 + 1e-12)
        Js.append(J_update)
        prev_c = c_after
    assert all(b <= a * (1 + 1e-12) for a, b in zip(Js, Js[1:]))
    assert prev_c.shape == (20, 16)


def test_centroids_are_member_means_pure_python():
    x, _, _ = _mixture(3, 120, 4, 5, 0.5)
    init = np.random.default_rng(4).choice(120, 7, replace=False)
    out = km.lloyd(x, init, 5)
    labels, cents = out["labels"], out["centroids"]
    for k in range(7):
        members = [x[i].tolist() for i in range(120) if labels[i] == k]
        if not members:
            continue
        mean = [sum(col) / len(members) for col in zip(*members)]
        assert np.allclose(mean, cents[k], rtol=1e-13, atol=1e-13)
    assert out["counts"].sum() == 120


def test_assignment_is_a_minimiser_pure_python():
    x, _, _ = _mixture(5, 40, 3, 4, 0.8)
    c = np.random.default_rng(6).standard_normal((6, 3))
    labels = km.assign(x, c)
    for i in range(40):
        d = [_pure_sqdist(x[i], c[k]) for k in range(6)]
        best = min(d)
        assert d[labels[i]] <= best + 1e-12
        # lowest index among exact minimisers
        assert labels[i] == min(k for k in range(6) if d[k] <= best + 1e-12)


def test_assignment_minimiser_numpy_brute_force():
    x, _, _ = _mixture(7, 2000, 32, 30, 0.3)
    c = x[np.random.default_rng(8).choice(2000, 64, replace=False)] + 0.01
    labels = km.assign(x, c)
    full = ((x[:, None, :] - c[None, :, :]) ** 2).sum(-1)
    np.testing.assert_array_equal(labels, np.argmin(full, axis=1))


def test_single_cluster_is_global_mean():
    x, _, _ = _mixture(9, 300, 8, 3, 1.0)
    out = km.lloyd(x, [17], 3)
    assert (out["labels"] == 0).all()
    np.testing.assert_allclose(out["centroids"][0], x.mean(axis=0), rtol=1e-13, atol=1e-14)


def test_c_equals_n_gives_zero_objective():
    x = np.random.default_rng(10).standard_normal((25, 5))
    out = km.lloyd(x, np.arange(25)[::-1].copy(), 2)
    assert km.objective(x, out["labels"], out["centroids"]) == 0.0
    assert sorted(out["labels"].tolist()) == list(range(25))


def test_separated_components_recovered():
    rng = np.random.default_rng(11)
    n_comp, d = 6, 16
    means = 20.0 * rng.standard_normal((n_comp, d))
    comp = rng.integers(0, n_comp, 500)
    x = means[comp] + 0.1 * rng.standard_normal((500, d))
    init = np.array([np.nonzero(comp == j)[0][0] for j in range(n_comp)])
    out = km.lloyd(x, init, 4)
    np.testing.assert_array_equal(out["labels"], comp)
    for j in range(n_comp):
        np.testing.assert_allclose(out["centroids"][j], x[comp == j].mean(axis=0), rtol=1e-12)


@pytest.mark.parametrize("seed", range(6))
def test_tiny_enumeration_lower_bound(seed):
    rng = np.random.default_rng(100 + seed)
    n, C = 7, 3
    x = rng.standard_normal((n, 2))
    init = rng.choice(n, C, replace=False)
    out = km.lloyd(x, init, 10)
    J_lloyd = km.objective(x, out["labels"], out["centroids"])
    best = math.inf
    for lab in itertools.product(range(C), repeat=n):
        J = 0.0
        for k in range(C):
            pts = [x[i] for i in range(n) if lab[i] == k]
            if pts:
                m = [sum(col) / len(pts) for col in zip(*pts)]
                J += sum(_pure_sqdist(p, m) for p in pts)
        best = min(best, J)
    assert J_lloyd >= best - 1e-12


def test_tiny_enumeration_separated_equality():
    x = np.array([[0.0, 0.0], [0.1, 0.0], [10.0, 0.0], [10.0, 0.2], [0.0, 9.0], [0.3, 9.0]])
    out = km.lloyd(x, [0, 2, 4], 5)
    J_lloyd = km.objective(x, out["labels"], out["centroids"])
    best = math.inf
    for lab in itertools.product(range(3), repeat=6):
        J = 0.0
        for k in range(3):
            pts = [x[i] for i in range(6) if lab[i] == k]
            if pts:
                m = [sum(col) / len(pts) for col in zip(*pts)]
                J += sum(_pure_sqdist(p, m) for p in pts)
        best = min(best, J)
    assert J_lloyd == pytest.approx(best, rel=1e-12)


def test_parity_mode_uses_rounded_centroids():
    x, _, _ = _mixture(12, 400, 16, 8, 0.4)
    c = x[np.random.default_rng(13).choice(400, 10, replace=False)] * 1.001
    chat = km.centroid_for_distance(c, "parity", "bf16")
    # every stored value is a bf16 value (low 16 bits of the fp32 encoding zero)
    bits = chat.astype(np.float32).view(np.uint32)
    assert (bits & 0xFFFF == 0).all()
    np.testing.assert_array_equal(chat, round_bf16(c))
    np.testing.assert_array_equal(km.assign(x, chat), km.assign(x, chat.astype(np.float32)))


def test_pack_is_stable_csr():
    labels = np.array([2, 0, 2, 1, 0, 2])
    keys = np.arange(6, dtype=np.float64)[:, None]
    cents = np.zeros((4, 1))
    p = km.pack(keys, keys * 10, labels, cents, "fp32")
    assert p["order"].tolist() == [1, 4, 3, 0, 2, 5]
    assert p["unit_start"].tolist() == [0, 2, 3, 6]
    assert p["unit_size"].tolist() == [2, 1, 3, 0]
    assert p["k"][:, 0].tolist() == [1, 4, 3, 0, 2, 5]
    assert p["v"][:, 0].tolist() == [10, 40, 30, 0, 20, 50]
