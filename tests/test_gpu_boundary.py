"""GPU parity: kv_boundary against the oracle (bit-exact flags).

LouisKV note, key design 1: r_t = mean over heads of cos(q_{t-1}, q_t);
retrieve when r_t < tau (strict).
"""
import numpy as np
import pytest
import torch

import long_context_kv_kmeans_amd as kvc
import workloads as wl
from oracle import boundary as ob
from tests.gpu_util import to_dev

pytestmark = pytest.mark.gpu


def _gpu_boundary(q_prev, q_cur, tau):
    B = q_cur.shape[0]
    flag = torch.zeros(B, dtype=torch.uint8, device="cuda")
    r = torch.zeros(B, dtype=torch.float32, device="cuda")
    kvc.kv_boundary(q_prev, q_cur, tau, flag, r)
    torch.cuda.synchronize()
    return flag.cpu().numpy().astype(bool), r.cpu().numpy()


@pytest.mark.parametrize("cfg_idx,steps", [(0, None), (1, None), (2, 16384), (3, None), (4, 512)])
def test_boundary_configs_bit_exact(cfg_idx, steps):
    cfg = wl.get_config(cfg_idx)
    seqs = range(min(cfg.batch, 4))
    q, jumps = wl.layer_queries(cfg, 0, steps, seqs=seqs)  # [T, B, Hq, d]
    T, B = q.shape[:2]
    # all steps of all sequences in one launch: batch index = (t, b)
    qd = to_dev(q, cfg.dtype)
    flag, r = _gpu_boundary(qd[:-1].reshape(-1, *q.shape[2:]).contiguous(),
                            qd[1:].reshape(-1, *q.shape[2:]).contiguous(), cfg.tau)
    of, orr = ob.boundary(q[:-1].reshape(-1, *q.shape[2:]), q[1:].reshape(-1, *q.shape[2:]), cfg.tau)
    np.testing.assert_array_equal(flag, of)
    np.testing.assert_allclose(r, orr, atol=2e-6)
    # the flags follow the walk's jumps
    assert (of.reshape(T - 1, B) == jumps[1:]).all()


def test_boundary_first_step():
    q = to_dev(np.ones((3, 4, 64), np.float32), "fp32")
    flag, r = _gpu_boundary(None, q, 0.7)
    assert flag.all() and np.isnan(r).all()


def test_boundary_golden_strict(tiny):
    case = tiny["boundary"]
    qp = np.zeros((1, 2, 64), np.float32)
    qc = np.zeros((1, 2, 64), np.float32)
    qp[..., :2] = case["q_prev"]
    qc[..., :2] = case["q_cur"]
    for c in case["cases"]:
        flag, r = _gpu_boundary(to_dev(qp, "fp32"), to_dev(qc, "fp32"), c["tau"])
        assert r[0] == pytest.approx(case["expect_r"], abs=1e-6)
        assert bool(flag[0]) is c["expect_flag"], c


def test_boundary_zero_norm_and_opposite():
    qp = np.zeros((2, 4, 128), np.float32)
    qc = np.ones((2, 4, 128), np.float32)
    qp[1] = -1.0
    flag, r = _gpu_boundary(to_dev(qp, "bf16"), to_dev(qc, "bf16"), 0.7)
    assert r[0] == 0.0 and r[1] == pytest.approx(-1.0, abs=1e-6)
    assert flag.all()
