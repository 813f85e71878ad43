"""The seeded input generators: shapes, determinism and dtype exactness."""
import numpy as np
import pytest

import workloads as wl


def test_configs_shapes():
    c = wl.get_config(1)
    assert (c.n_q_heads, c.n_kv_heads, c.head_dim, c.group) == (32, 8, 128, 4)
    assert wl.get_config(0).dtype == "fp32" and wl.get_config(3).layers == 36
    assert wl.get_config(4).batch == 16 and wl.get_config(2).buf_cap == 1024


def test_layer_inputs_deterministic_and_exact():
    cfg = wl.get_config(1, n_keys=512, n_clusters=32, n_components=16)
    a = wl.layer_inputs(cfg, heads=[0, 3])
    b = wl.layer_inputs(cfg, heads=[3])
    np.testing.assert_array_equal(a["keys"][0, 1], b["keys"][0, 0])
    assert a["keys"].shape == (1, 2, 512, 128)
    bits = a["keys"].view(np.uint32)
    assert (bits & 0xFFFF == 0).all()  # bf16-exact
    for h in range(2):
        idx = a["init_idx"][0, h]
        assert len(set(idx.tolist())) == 32 and idx.min() >= 0 and idx.max() < 512


def test_layer_inputs_threads_give_the_same_arrays():
    cfg = wl.get_config(4, n_keys=256, n_clusters=16, n_components=8, batch=2)
    a = wl.layer_inputs(cfg, 1)
    b = wl.layer_inputs(cfg, 1, threads=5)
    for k in ("keys", "values", "init_idx", "components"):
        np.testing.assert_array_equal(a[k], b[k])


def test_query_walk_structure():
    cfg = wl.get_config(0)
    q, jumps = wl.query_walk(cfg, 0, 0)
    assert q.shape == (64, 4, 64) and not jumps[0]
    # drift steps stay close, jumps move far
    step = np.linalg.norm(np.diff(q, axis=0), axis=-1).mean(axis=-1)
    assert (step[~jumps[1:]] < 1.0).all() and (step[jumps[1:]] > 5.0).all()


def test_decode_kv_shapes():
    cfg = wl.get_config(2, steps=20)
    k, v = wl.layer_decode_kv(cfg)
    assert k.shape == (20, 1, 8, 128) and v.shape == (20, 1, 8, 128)


def test_retrieval_schedules_and_page_labels():
    assert wl.retrieval_schedule("boundary", 5) is None
    assert wl.retrieval_schedule("per-token", 3).tolist() == [True] * 3
    assert wl.retrieval_schedule("stride:3", 7).tolist() == [True, False, False, True, False,
                                                             False, True]
    for bad in ("stride:0", "every-step"):
        with pytest.raises(ValueError):
            wl.retrieval_schedule(bad, 4)
    lab = wl.page_labels(2, 3, 10, 4)
    assert lab.shape == (2, 3, 10) and lab.dtype == np.int32
    assert lab[1, 2].tolist() == [0, 0, 0, 0, 1, 1, 1, 1, 2, 2]
