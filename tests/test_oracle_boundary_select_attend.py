"""Pins of the oracle's boundary test, selection and attention.

Boundary: LouisKV note, key design 1 (r_t); selection: flowchart Top-B and
key design 3; attention: flowchart "Attention". Each check uses a closed
form, an invariant, brute force or a hand-derived fixture.
"""
import math

import numpy as np
import pytest

from oracle import attend, boundary, select
from oracle.precision import round_bf16


# ---------------------------------------------------------------- precision
def test_bf16_rounding_golden(tiny):
    for case in tiny["bf16_rne"]["cases"]:
        assert round_bf16(np.array([case["x"]]))[0] == case["expect"], case


def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    base = (rng.standard_normal(20000) * 10.0 ** rng.integers(-6, 6, 20000)).astype(np.float32)
    # exact ties: keep the top 16 bits of finite fp32 values and set the dropped half to 0x8000
    ties = ((base[:4000].view(np.uint32) & np.uint32(0xFFFF0000)) | np.uint32(0x8000)).view(np.float32)
    x = np.concatenate([base, ties]).astype(np.float64)
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(round_bf16(x), ref)


# ---------------------------------------------------------------- boundary
def test_boundary_golden(tiny):
    case = tiny["boundary"]
    for c in case["cases"]:
        flag, r = boundary.boundary(np.array(case["q_prev"]), np.array(case["q_cur"]), c["tau"])
        assert r[0] == pytest.approx(case["expect_r"], abs=1e-15)
        assert bool(flag[0]) is c["expect_flag"], c


def test_boundary_closed_forms():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((2, 4, 16))
    f, r = boundary.boundary(q, q, 0.7)
    np.testing.assert_allclose(r, 1.0, atol=1e-15)
    assert not f.any()
    f, r = boundary.boundary(q, 3.5 * q, 0.7)
    np.testing.assert_allclose(r, 1.0, atol=1e-15)
    f, r = boundary.boundary(q, -q, 0.7)
    np.testing.assert_allclose(r, -1.0, atol=1e-15)
    assert f.all()


def test_boundary_known_angles():
    # rotate every head by a known angle theta_h inside a random 2-D plane;
    # cos = cos(theta_h) and r is their mean
    rng = np.random.default_rng(2)
    H, d = 8, 32
    thetas = np.linspace(0.1, 2.0, H)
    qp = np.empty((1, H, d))
    qc = np.empty((1, H, d))
    for h in range(H):
        u = rng.standard_normal(d)
        w = rng.standard_normal(d)
        w -= (w @ u) / (u @ u) * u
        w *= np.linalg.norm(u) / np.linalg.norm(w)
        qp[0, h] = u
        qc[0, h] = (math.cos(thetas[h]) * u + math.sin(thetas[h]) * w) * (h + 1)
    _, r = boundary.boundary(qp, qc, 0.7)
    assert r[0] == pytest.approx(np.cos(thetas).mean(), abs=1e-12)


def test_boundary_first_step_and_zero_norm():
    q = np.ones((3, 2, 4))
    f, r = boundary.boundary(None, q, 0.7)
    assert f.all() and np.isnan(r).all()
    z = np.zeros((1, 2, 4))
    z[0, 1, 0] = 1.0
    f, r = boundary.boundary(z, np.ones((1, 2, 4)), 0.7)
    # head 0 has zero norm -> cosine 0; head 1 cos = 1/2
    assert r[0] == pytest.approx(0.25)
    assert f[0]


def test_boundary_invariances():
    rng = np.random.default_rng(3)
    a, b = rng.standard_normal((2, 5, 6, 8))
    _, r1 = boundary.boundary(a, b, 0.7)
    _, r2 = boundary.boundary(b, a, 0.7)
    _, r3 = boundary.boundary(a * 2.0, b * 0.25, 0.7)
    perm = rng.permutation(6)
    _, r4 = boundary.boundary(a[:, perm], b[:, perm], 0.7)
    np.testing.assert_allclose(r1, r2, rtol=1e-14)
    np.testing.assert_allclose(r1, r3, rtol=1e-13)
    np.testing.assert_allclose(r1, r4, rtol=1e-13)
    assert (np.abs(r1) <= 1.0).all()


# ---------------------------------------------------------------- selection
def test_select_golden(tiny):
    case = tiny["select"]
    for c in case["cases"]:
        got = select.select_prefix(np.array(case["scores"]), np.array(case["sizes"]), c["budget"])
        assert got.tolist() == c["expect"], c


def _brute_force_select(scores, sizes, budget):
    # u is selected iff u is non-empty and the total size of every non-empty
    # unit ranked at or before u (score higher, or equal with id <= u) fits.
    U = len(scores)
    out = []
    for u in range(U):
        if sizes[u] <= 0:
            continue
        tot = 0
        for v in range(U):
            if sizes[v] > 0 and (scores[v] > scores[u] or (scores[v] == scores[u] and v <= u)):
                tot += sizes[v]
        if tot <= budget:
            out.append(u)
    return out


@pytest.mark.parametrize("seed", range(20))
def test_select_matches_brute_force(seed):
    rng = np.random.default_rng(seed)
    U = int(rng.integers(1, 60))
    scores = np.round(rng.standard_normal(U), 1)  # rounding creates ties
    sizes = rng.integers(0, 12, U)
    budget = int(rng.integers(0, 80))
    got = select.select_prefix(scores, sizes, budget).tolist()
    assert got == _brute_force_select(scores.tolist(), sizes.tolist(), budget)
    # budget never exceeded; maximal prefix: the next ranked unit overflows
    tot = int(sizes[got].sum()) if got else 0
    assert tot <= budget
    ranked = select.rank_units(scores, sizes)
    if len(got) < len(ranked):
        nxt = ranked[len(got)]
        assert tot + sizes[nxt] > budget
        assert set(got) == set(ranked[:len(got)].tolist())


def test_select_full_budget_takes_all_nonempty():
    rng = np.random.default_rng(5)
    sizes = rng.integers(0, 5, 100)
    got = select.select_prefix(rng.standard_normal(100), sizes, int(sizes.sum()))
    assert got.tolist() == np.nonzero(sizes)[0].tolist()


def test_group_scores_linear_and_basis():
    rng = np.random.default_rng(6)
    q = rng.standard_normal((4, 8))
    idx = np.eye(8)
    # basis index vectors pick coordinates: s_u = sum_h q_h[u]
    np.testing.assert_allclose(select.group_scores(q, idx), q.sum(axis=0), rtol=1e-15)
    idx = rng.standard_normal((30, 8))
    s_all = select.group_scores(q, idx)
    s_parts = sum(select.group_scores(q[h:h + 1], idx) for h in range(4))
    np.testing.assert_allclose(s_all, s_parts, rtol=1e-13)
    np.testing.assert_allclose(select.group_scores(2 * q, idx), 2 * s_all, rtol=1e-14)


# ---------------------------------------------------------------- attention
def test_attend_golden(tiny):
    c = tiny["attend"]
    out = attend.attend_exact(np.array(c["q"]), np.array(c["k"]), np.array(c["v"]), c["scale"])
    np.testing.assert_allclose(out, c["expect"], rtol=1e-14)


def test_attend_pure_python_dense():
    rng = np.random.default_rng(7)
    q = rng.standard_normal((3, 5))
    K = rng.standard_normal((9, 5))
    V = rng.standard_normal((9, 5))
    out = attend.attend_exact(q, K, V, 0.4)
    for h in range(3):
        w = [math.exp(0.4 * sum(q[h, j] * K[i, j] for j in range(5))) for i in range(9)]
        tot = sum(w)
        ref = [sum(w[i] * V[i, j] for i in range(9)) / tot for j in range(5)]
        np.testing.assert_allclose(out[h], ref, rtol=1e-12)


def test_attend_special_cases():
    rng = np.random.default_rng(8)
    q = rng.standard_normal((2, 6))
    K = rng.standard_normal((1, 6))
    V = rng.standard_normal((1, 6))
    np.testing.assert_allclose(attend.attend_exact(q, K, V, 1.0), np.repeat(V, 2, 0), rtol=1e-15)
    K = np.repeat(rng.standard_normal((1, 6)), 7, 0)
    V = rng.standard_normal((7, 6))
    np.testing.assert_allclose(attend.attend_exact(q, K, V, 1.0), np.repeat(V.mean(0, keepdims=True), 2, 0),
                               rtol=1e-12)
    assert (attend.attend_exact(q, np.zeros((0, 6)), np.zeros((0, 6)), 1.0) == 0).all()


def test_attend_invariances():
    rng = np.random.default_rng(9)
    q = rng.standard_normal((4, 16))
    K = rng.standard_normal((50, 16))
    V = rng.standard_normal((50, 16))
    base = attend.attend_exact(q, K, V, 0.25)
    perm = rng.permutation(50)
    np.testing.assert_allclose(attend.attend_exact(q, K[perm], V[perm], 0.25), base, rtol=1e-12)
    # a common offset on every key shifts each head's scores uniformly
    np.testing.assert_allclose(attend.attend_exact(q, K + rng.standard_normal(16), V, 0.25), base,
                               rtol=1e-10, atol=1e-12)
    # a very large scale concentrates all weight on the best row
    big = attend.attend_exact(q, K, V, 1e6)
    np.testing.assert_allclose(big, V[np.argmax(K @ q.T, axis=0)], rtol=1e-12)
