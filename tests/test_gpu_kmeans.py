"""GPU parity: K-means assign / update / cluster build against the oracle.

LouisKV note, key design 2 (K-means over keys, centroid = member mean).
Gate (lock-step): at each Lloyd round the GPU assignment on the oracle's
centroids agrees with the oracle (parity mode: distances to bf16(fp32 c))
on >= 99.9% of keys, and the GPU update on the oracle's labels matches the
oracle's centroids to relative error <= 1e-3 (max_k |c_k - c_k^o| / |c_k^o|).
Integer outputs of the pack (unit tables, row order) are bit-exact.
"""
import numpy as np
import pytest
import torch

import long_context_kv_kmeans_amd as kvc
import workloads as wl
from oracle import kmeans as okm
from tests.gpu_util import make_pool, to_dev, to_np

pytestmark = pytest.mark.gpu

AGREE = 0.999
CENT_RTOL = 1e-3


def _keys(cfg, heads, seqs=(0,)):
    inp = wl.layer_inputs(cfg, 0, heads=heads, seqs=seqs)
    B, H, N, d = inp["keys"].shape
    return inp, inp["keys"].reshape(B * H, N, d), inp["init_idx"].reshape(B * H, -1)


def _gpu_assign(keys_d, cents64):
    cent = torch.from_numpy(cents64.astype(np.float32)).cuda()
    lab = torch.zeros(keys_d.shape[:2], dtype=torch.int32, device="cuda")
    kvc.kv_kmeans_assign(keys_d, cent, lab)
    torch.cuda.synchronize()
    return lab.cpu().numpy()


def _gpu_update(keys_d, labels, cents64):
    cin = torch.from_numpy(cents64.astype(np.float32)).cuda()
    cout = torch.empty_like(cin)
    counts = torch.zeros(cin.shape[:2], dtype=torch.int32, device="cuda")
    kvc.kv_kmeans_update(keys_d, torch.from_numpy(labels.astype(np.int32)).cuda(), cin, cout, counts)
    torch.cuda.synchronize()
    return cout.cpu().numpy().astype(np.float64), counts.cpu().numpy()


def _rel_err(c, ref):
    num = np.linalg.norm(c - ref, axis=-1)
    den = np.maximum(np.linalg.norm(ref, axis=-1), 1e-30)
    return float((num / den).max())


CASES = [
    # (cfg, overrides, heads) -- several MFMA tiles, ragged key and cluster tails
    (0, {}, [0, 1]),
    (1, dict(n_keys=4096, n_clusters=256, n_components=64), [0, 5]),
    (1, dict(n_keys=4133, n_clusters=250, n_components=64), [2]),
    (1, dict(n_keys=3000, n_clusters=77, n_components=20, head_dim=64), [1]),
    (4, dict(n_keys=4096, n_clusters=256, n_components=64), [3]),
]


@pytest.mark.parametrize("cfg_idx,over,heads", CASES)
def test_lockstep_assign_update(cfg_idx, over, heads):
    cfg = wl.get_config(cfg_idx, **over)
    inp, keys, init = _keys(cfg, heads)
    keys_d = to_dev(keys, cfg.dtype)
    BH, N, d = keys.shape
    c = np.stack([keys[h][init[h]].astype(np.float64) for h in range(BH)])
    for it in range(4):
        c_in = c.astype(np.float32).astype(np.float64)  # the GPU receives fp32 centroids
        gl = _gpu_assign(keys_d, c_in)
        ol = np.stack([okm.assign(keys[h], okm.centroid_for_distance(c_in[h], "parity", cfg.dtype))
                       for h in range(BH)])
        agree = (gl == ol).mean()
        assert agree >= AGREE, (it, agree)
        new = []
        for h in range(BH):
            cn, _ = okm.update(keys[h], ol[h], c_in[h])
            new.append(cn)
        new = np.stack(new)
        gc, gcnt = _gpu_update(keys_d, ol, c_in)
        assert _rel_err(gc, new) <= CENT_RTOL
        assert _rel_err(gc, new) <= 1e-5  # fp32 sums of <= N bf16 values
        for h in range(BH):
            np.testing.assert_array_equal(gcnt[h], np.bincount(ol[h], minlength=cfg.n_clusters))
        c = new


def test_assign_ties_and_padding():
    # keys equidistant from two identical centroids -> lowest index; C not a multiple of 32
    rng = np.random.default_rng(5)
    d, C, N = 128, 45, 300
    cents = rng.standard_normal((1, C, d)).astype(np.float32)
    cents[0, 20] = cents[0, 7]
    cents[0, 44] = cents[0, 7]
    keys = (cents[0, rng.integers(0, C, N)] + 0.05 * rng.standard_normal((N, d))).astype(np.float32)
    keys = wl.to_dtype(keys, "bf16")[None]
    cb = wl.to_dtype(cents, "bf16").astype(np.float64)
    gl = _gpu_assign(to_dev(keys, "bf16"), cb)
    ol = okm.assign(keys[0], okm.centroid_for_distance(cb[0], "parity", "bf16"))
    np.testing.assert_array_equal(gl[0], ol)
    assert not np.isin(gl[0], [20, 44]).any()


@pytest.mark.parametrize("cfg_idx,over", [(0, {}), (1, dict(n_keys=4133, n_clusters=250,
                                                              n_components=64))])
def test_prepared_assign_matches_assign(cfg_idx, over):
    # one prepared workspace labels two key sets (the second shorter) exactly as
    # kv_kmeans_assign does, and the workspace is not consumed by the calls
    cfg = wl.get_config(cfg_idx, **over)
    _, keys, init = _keys(cfg, [0, 1])
    BH, N, d = keys.shape
    c = np.stack([keys[h][init[h]].astype(np.float64) for h in range(BH)])
    c = c + 0.01 * np.random.default_rng(3).standard_normal(c.shape)
    cent = torch.from_numpy(c.astype(np.float32)).cuda()
    dt = torch.float32 if cfg.dtype == "fp32" else torch.bfloat16
    ws = kvc.workspace(kvc.lib().kv_kmeans_assign_workspace(BH, cfg.n_clusters, d,
                                                            kvc.dtype_code(dt)))
    kvc.kv_kmeans_prepare(cent, dt, ws)
    for n in (N, N // 3 + 5):
        kd = to_dev(np.ascontiguousarray(keys[:, :n]), cfg.dtype)
        lab_p = torch.full((BH, n), -1, dtype=torch.int32, device="cuda")
        kvc.kv_kmeans_assign_prepared(kd, cent, lab_p, ws)
        lab_a = torch.full((BH, n), -1, dtype=torch.int32, device="cuda")
        kvc.kv_kmeans_assign(kd, cent, lab_a)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(lab_p.cpu().numpy(), lab_a.cpu().numpy())
        c_in = c.astype(np.float32).astype(np.float64)
        ol = np.stack([okm.assign(keys[h, :n], okm.centroid_for_distance(c_in[h], "parity",
                                                                          cfg.dtype))
                       for h in range(BH)])
        assert (lab_p.cpu().numpy() == ol).mean() >= AGREE


def test_update_empty_cluster_keeps_centroid(tiny):
    case = tiny["kmeans_empty"]
    keys = np.zeros((1, 2, 64), np.float32)
    keys[0, :, 0] = np.array(case["keys"])[:, 0]
    cin = np.zeros((1, 2, 64))
    cin[0, :, 0] = np.array(case["init_centroids"])[:, 0]
    gc, cnt = _gpu_update(to_dev(keys, "fp32"), np.array([[0, 0]]), cin)
    np.testing.assert_array_equal(gc[0, :, 0], np.array(case["expect_centroids"])[:, 0])
    assert cnt[0].tolist() == case["expect_counts"]


def _cluster_build(cfg, heads, iters, seqs=(0,), rounds=None, dup=0, sweeps=None):
    inp = wl.layer_inputs(cfg, 0, heads=heads, seqs=seqs)
    if dup:  # exact copies: key i repeats key i - i % dup (ties between keys and centroids)
        src = np.arange(inp["keys"].shape[2])
        inp["keys"] = inp["keys"][:, :, src - src % dup].copy()
    B, H, N, d = inp["keys"].shape
    pool = make_pool(B, H, d, cfg.dtype, N, cfg.n_clusters)
    keys = to_dev(inp["keys"], cfg.dtype)
    vals = to_dev(inp["values"], cfg.dtype)
    init = torch.from_numpy(inp["init_idx"]).cuda()
    lab = torch.zeros(B, H, N, dtype=torch.int32, device="cuda")
    kvc.kv_cluster_build(pool, keys, vals, cfg.n_clusters, iters, init, assign_out=lab,
                         rounds_out=rounds, sweeps_out=sweeps)
    torch.cuda.synchronize()
    return inp, pool, lab.cpu().numpy()


# several chunks of the counting sort with a ragged last one, for
# 1024 < C <= 4096 and for C > 4096 (two ranking waves per chunk)
BIG_C = [
    (1, dict(n_keys=9000, n_clusters=1500, n_components=64), [0]),
    (1, dict(n_keys=17001, n_clusters=5000, n_components=128), [1]),
]


@pytest.mark.parametrize("cfg_idx,over,heads", CASES[:3] + BIG_C)
def test_cluster_build_invariants_and_pack(cfg_idx, over, heads):
    cfg = wl.get_config(cfg_idx, **over)
    inp, pool, lab = _cluster_build(cfg, heads, cfg.iters)
    keys, vals = inp["keys"][0], inp["values"][0]
    C = cfg.n_clusters
    for g in range(len(heads)):
        l = lab[0, g]
        counts = np.bincount(l, minlength=C)
        np.testing.assert_array_equal(pool.unit_size[0, g].cpu().numpy(), counts)
        np.testing.assert_array_equal(pool.unit_start[0, g].cpu().numpy(),
                                      np.concatenate([[0], np.cumsum(counts)[:-1]]))
        # pool rows are the keys/values in stable cluster order (bit-exact)
        order = np.argsort(l, kind="stable")
        np.testing.assert_array_equal(to_np(pool.k[0, g]), keys[g][order])
        np.testing.assert_array_equal(to_np(pool.v[0, g]), vals[g][order])
        # centroids are the member means of the final labels
        means, _ = okm.update(keys[g], l, np.zeros((C, cfg.head_dim)))
        um = to_np(pool.unit_mean[0, g])
        nz = counts > 0
        assert _rel_err(um[nz], means[nz]) <= 1e-5
        # the scoring copy is the storage-dtype rounding of the fp32 mean
        from oracle.precision import to_storage
        np.testing.assert_array_equal(to_np(pool.unit_index[0, g]), to_storage(um, cfg.dtype))
        # every key sits with a nearest centroid of the previous round's centroids is not
        # checkable here; the objective must be close to the oracle's own run
    assert pool.n_rows.cpu().tolist() == [cfg.n_keys]
    assert pool.n_units.cpu().tolist() == [C] and pool.n_cand.cpu().tolist() == [C]


# many heads converging at different rounds (a mix of whole and incremental
# sweeps in one launch, queued keys of several heads); head_dim 64; copied keys
EQ_EXTRA = [
    (1, dict(n_keys=16384, n_clusters=1024, n_components=128), list(range(8)), 0),
    (CASES[3][0], CASES[3][1], CASES[3][2], 0),
    (1, dict(n_keys=8192, n_clusters=700, n_components=96), [0, 1, 2], 3),
    # more shapes: few components (clusters split one mixture component),
    # C above a third of a small key set, head_dim 64 with many heads
    (1, dict(n_keys=6000, n_clusters=333, n_components=12), [0, 1, 2, 3], 0),
    (1, dict(n_keys=12000, n_clusters=3000, n_components=200), [4, 5], 0),
    (4, dict(n_keys=2500, n_clusters=100, n_components=30, head_dim=64), list(range(8)), 2),
]


def _check_build_equals_rounds(cfg, heads, iters, dup=0, seqs=(0,)):
    rounds = torch.full((len(seqs), len(heads)), -1, dtype=torch.int32, device="cuda")
    sweeps = torch.full((len(seqs), len(heads)), -1.0, dtype=torch.float32, device="cuda")
    inp, pool, lab = _cluster_build(cfg, heads, iters, seqs=seqs, rounds=rounds, dup=dup,
                                    sweeps=sweeps)
    rounds, sweeps = rounds.cpu().numpy(), sweeps.cpu().numpy()
    # assignments run per head: iters, or (bf16) fewer for a head whose
    # assignment in some round 2.. changed no label; their work in whole
    # sweeps: rounds 1 and 2 sweep everything, later rounds at most a third of
    # the centroids for every key plus all of them for the queued keys
    if cfg.dtype == "fp32":
        assert (rounds == iters).all() and (sweeps == iters).all()
    else:
        assert ((rounds >= 2) & (rounds <= iters)).all(), rounds
        assert ((sweeps >= 2 - 1e-6) & (sweeps <= 2 + (rounds - 2) * 4 / 3 + 1e-3)).all(), sweeps
    print(f"rounds run per head: {rounds.tolist()} of {iters}; sweeps {sweeps.round(3).tolist()}")
    B, H, N, d = inp["keys"].shape
    keys_d = to_dev(inp["keys"], cfg.dtype).reshape(B * H, N, d)
    idx = torch.from_numpy(inp["init_idx"]).cuda().reshape(B * H, -1).long()
    cent = torch.gather(keys_d.float(), 1, idx[..., None].expand(-1, -1, d)).contiguous()
    labels = torch.zeros(B * H, N, dtype=torch.int32, device="cuda")
    counts = torch.zeros(B * H, cfg.n_clusters, dtype=torch.int32, device="cuda")
    for _ in range(iters):
        kvc.kv_kmeans_assign(keys_d, cent, labels)
        nxt = torch.empty_like(cent)
        kvc.kv_kmeans_update(keys_d, labels, cent, nxt, counts)
        cent = nxt
    torch.cuda.synchronize()
    np.testing.assert_array_equal(lab.reshape(B * H, N), labels.cpu().numpy())
    um = pool.unit_mean[:, :, :cfg.n_clusters].reshape(B * H, cfg.n_clusters, d)
    assert torch.equal(um, cent)


@pytest.mark.parametrize("iters", [4, 14])
@pytest.mark.parametrize("cfg_idx,over,heads,dup",
                         [c + (0,) for c in [CASES[0], CASES[2]] + BIG_C] + EQ_EXTRA)
def test_cluster_build_equals_assign_update_rounds(cfg_idx, over, heads, dup, iters):
    """kv_cluster_build's rounds (the two-launch update of every round but the
    last; heads that reach a fixed point skip their later rounds; from the
    third round on, the sweep covers only the centroids that moved, plus every
    centroid for the keys whose own centroid moved; intermediate updates skip
    the member sums of untouched clusters) give the same labels and
    centroids, bit for bit, as running kv_kmeans_assign and kv_kmeans_update
    round by round from the same start. 14 rounds take these heads past their
    fixed points."""
    _check_build_equals_rounds(wl.get_config(cfg_idx, **over), heads, iters, dup=dup)


def test_cluster_build_equals_rounds_128_heads():
    """16 sequences x 8 KV heads in one build: the served-head lists and the
    queued-key groups span two 64-head chunks."""
    cfg = wl.get_config(4, n_keys=4096, n_clusters=256, n_components=64)
    _check_build_equals_rounds(cfg, list(range(8)), cfg.iters, seqs=tuple(range(16)))


@pytest.mark.parametrize("cfg_idx", [3, 1])
def test_cluster_build_equals_rounds_full_size(cfg_idx):
    """One layer at the full sizes of the 36-layer and the single-layer
    workloads (8 heads x 131072 keys, C = 8192; 8 x 32768, C = 2048), the
    rounds the bench runs."""
    cfg = wl.get_config(cfg_idx)
    _check_build_equals_rounds(cfg, list(range(cfg.n_kv_heads)), cfg.iters)


def test_cluster_build_free_running_tiny_fp32():
    cfg = wl.get_config(0)
    inp, pool, lab = _cluster_build(cfg, [0, 1], cfg.iters)
    for g in range(2):
        o = okm.lloyd(inp["keys"][0, g], inp["init_idx"][0, g], cfg.iters, mode="parity", dtype="fp32")
        agree = (lab[0, g] == o["labels"]).mean()
        assert agree >= AGREE
        J_gpu = okm.objective(inp["keys"][0, g], lab[0, g], to_np(pool.unit_mean[0, g]))
        J_ora = okm.objective(inp["keys"][0, g], o["labels"], o["centroids"])
        assert J_gpu <= J_ora * (1 + 1e-3)


def test_cluster_build_free_running_report_qwen3_layer_small():
    cfg = wl.get_config(1, n_keys=4096, n_clusters=256, n_components=64)
    inp, pool, lab = _cluster_build(cfg, [0], cfg.iters)
    o = okm.lloyd(inp["keys"][0, 0], inp["init_idx"][0, 0], cfg.iters, mode="parity", dtype="bf16")
    agree = (lab[0, 0] == o["labels"]).mean()
    J_gpu = okm.objective(inp["keys"][0, 0], lab[0, 0], to_np(pool.unit_mean[0, 0]))
    J_ora = okm.objective(inp["keys"][0, 0], o["labels"], o["centroids"])
    print(f"free-running agreement {agree:.5f}, J_gpu/J_oracle {J_gpu / J_ora:.6f}")
    assert J_gpu <= J_ora * (1 + 1e-2)  # chaotic trajectory: reported, loosely bounded


def test_cluster_build_deterministic():
    cfg = wl.get_config(1, n_keys=4096, n_clusters=256, n_components=64)
    _, p1, l1 = _cluster_build(cfg, [0, 1], 3)
    _, p2, l2 = _cluster_build(cfg, [0, 1], 3)
    np.testing.assert_array_equal(l1, l2)
    assert torch.equal(p1.unit_mean, p2.unit_mean)
    assert torch.equal(p1.k, p2.k)


def test_cluster_build_beside_gemms_on_another_stream():
    # K-means overlapped with a prefill forward (the note's asynchronous
    # pipeline): kv_cluster_build on its own stream while large GEMMs run on
    # another gives the same clustering and pool, bit for bit, as alone
    cfg = wl.get_config(1, n_keys=8192, n_clusters=512, n_components=128)
    inp, ref_pool, ref_lab = _cluster_build(cfg, [0, 1, 2, 3], 4)
    B, H, N, d = inp["keys"].shape
    keys = to_dev(inp["keys"], cfg.dtype)
    vals = to_dev(inp["values"], cfg.dtype)
    init = torch.from_numpy(inp["init_idx"]).cuda()
    x = torch.randn(8192, 4096, device="cuda").bfloat16()
    w = torch.randn(4096, 8192, device="cuda").bfloat16()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    for _ in range(2):
        pool = make_pool(B, H, d, cfg.dtype, N, cfg.n_clusters)
        lab = torch.zeros(B, H, N, dtype=torch.int32, device="cuda")
        torch.cuda.synchronize()
        with torch.cuda.stream(sa):
            y = [x @ w for _ in range(4)]
        kvc.kv_cluster_build(pool, keys, vals, cfg.n_clusters, 4, init, assign_out=lab, stream=sb)
        torch.cuda.synchronize()
        del y
        np.testing.assert_array_equal(lab.cpu().numpy(), ref_lab)
        for name in ("k", "v", "unit_start", "unit_size", "unit_mean", "unit_index"):
            assert torch.equal(getattr(pool, name), getattr(ref_pool, name)), name


def test_kmeans_beside_gemms_matches_the_oracle():
    """The K-means steps on their own stream while large GEMMs run on another
    (the note's K-means overlapped with the prefill forward), checked against
    the oracle with the lock-step gate: each round's assignment on the oracle's
    previous centroids agrees on >= 99.9% of keys, each update on the oracle's
    labels is within 1e-3 of the oracle's centroids. The full build beside the
    GEMMs must then reach the oracle's free-running objective (within 1%, the
    trajectory being chaotic)."""
    cfg = wl.get_config(1, n_keys=8192, n_clusters=512, n_components=128)
    inp, keys, init = _keys(cfg, [0, 1, 2, 3])
    BH, N, d = keys.shape
    keys_d = to_dev(keys, cfg.dtype)
    x = torch.randn(8192, 4096, device="cuda").bfloat16()
    w = torch.randn(4096, 8192, device="cuda").bfloat16()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()

    def beside_gemms(fn):
        torch.cuda.synchronize()
        with torch.cuda.stream(sa):
            y = [x @ w for _ in range(4)]
        with torch.cuda.stream(sb):
            fn()
        torch.cuda.synchronize()
        del y

    c = np.stack([keys[h][init[h]].astype(np.float64) for h in range(BH)])
    for it in range(4):
        c_in = c.astype(np.float32).astype(np.float64)
        cent = torch.from_numpy(c_in.astype(np.float32)).cuda()
        lab = torch.zeros(BH, N, dtype=torch.int32, device="cuda")
        beside_gemms(lambda: kvc.kv_kmeans_assign(keys_d, cent, lab, stream=sb))
        gl = lab.cpu().numpy()
        ol = np.stack([okm.assign(keys[h], okm.centroid_for_distance(c_in[h], "parity", cfg.dtype))
                       for h in range(BH)])
        assert (gl == ol).mean() >= AGREE, it
        cout = torch.empty_like(cent)
        ol_d = torch.from_numpy(ol.astype(np.int32)).cuda()
        beside_gemms(lambda: kvc.kv_kmeans_update(keys_d, ol_d, cent, cout, stream=sb))
        new = np.stack([okm.update(keys[h], ol[h], c_in[h])[0] for h in range(BH)])
        assert _rel_err(cout.cpu().numpy().astype(np.float64), new) <= CENT_RTOL, it
        c = new

    B, H = 1, BH
    pool = make_pool(B, H, d, cfg.dtype, N, cfg.n_clusters)
    lab = torch.zeros(B, H, N, dtype=torch.int32, device="cuda")
    beside_gemms(lambda: kvc.kv_cluster_build(
        pool, keys_d.reshape(B, H, N, d), to_dev(inp["values"], cfg.dtype), cfg.n_clusters,
        cfg.iters, torch.from_numpy(inp["init_idx"]).cuda(), assign_out=lab, stream=sb))
    lab = lab.cpu().numpy()[0]
    for h in range(H):
        o = okm.lloyd(keys[h], init[h], cfg.iters, mode="parity", dtype=cfg.dtype)
        J_gpu = okm.objective(keys[h], lab[h], to_np(pool.unit_mean[0, h]))
        J_ora = okm.objective(keys[h], o["labels"], o["centroids"])
        print(f"head {h}: free-running agreement {(lab[h] == o['labels']).mean():.5f}, "
              f"J_gpu/J_oracle {J_gpu / J_ora:.6f}")
        assert J_gpu <= J_ora * (1 + 1e-2)


@pytest.mark.parametrize("cfg_idx,heads,sample", [(1, [0, 7], 4000), (3, [0], 3000), (4, [0], 3000)])
def test_full_size_sampled(cfg_idx, heads, sample):
    """Full-size heads: GPU round on its own centroids, checked on sampled keys/clusters."""
    cfg = wl.get_config(cfg_idx)
    inp, keys, init = _keys(cfg, heads)
    BH, N, d = keys.shape
    keys_d = to_dev(keys, cfg.dtype)
    rng = np.random.default_rng(0)
    c = np.stack([keys[h][init[h]].astype(np.float64) for h in range(BH)])
    for it in range(2):
        gl = _gpu_assign(keys_d, c)
        idx = rng.choice(N, sample, replace=False)
        for h in range(BH):
            ol = okm.assign(keys[h][idx], okm.centroid_for_distance(c[h], "parity", cfg.dtype))
            assert (gl[h][idx] == ol).mean() >= AGREE - 1.0 / sample
        gc, cnt = _gpu_update(keys_d, gl, c)
        for h in range(BH):
            ks = rng.choice(cfg.n_clusters, 200, replace=False)
            for k in ks:
                mem = keys[h][gl[h] == k]
                ref = mem.astype(np.float64).mean(0) if len(mem) else c[h][k]
                assert np.linalg.norm(gc[h][k] - ref) <= 1e-5 * max(np.linalg.norm(ref), 1e-30)
            assert cnt[h].sum() == N
        c = gc


def test_update_many_heads_long_chunks():
    """128 heads x 32773 keys, C = 2048: enough keys (>= 4096 x 1024) for the
    counting sort's 4096-key chunks, with a ragged last chunk. Counts are exact
    for every head; centroids of sampled heads match the oracle's update."""
    BH, N, d, C = 128, 32773, 128, 2048
    g = torch.Generator(device="cuda").manual_seed(11)
    keys_d = torch.randn(BH, N, d, generator=g, device="cuda").to(torch.bfloat16)
    lab_d = torch.randint(0, C, (BH, N), generator=g, device="cuda", dtype=torch.int32)
    idx = torch.randint(0, N, (BH, C), generator=g, device="cuda")
    cin = torch.gather(keys_d.float(), 1, idx[..., None].expand(BH, C, d)).contiguous()
    cout = torch.empty_like(cin)
    counts = torch.zeros(BH, C, dtype=torch.int32, device="cuda")
    kvc.kv_kmeans_update(keys_d, lab_d, cin, cout, counts)
    torch.cuda.synchronize()
    lab = lab_d.cpu().numpy()
    cnt = counts.cpu().numpy()
    for h in range(BH):
        np.testing.assert_array_equal(cnt[h], np.bincount(lab[h], minlength=C))
    for h in (0, 77, 127):
        kh = keys_d[h].float().cpu().numpy()
        ref, rc = okm.update(kh, lab[h], cin[h].cpu().numpy().astype(np.float64))
        np.testing.assert_array_equal(cnt[h], rc)
        assert _rel_err(cout[h].cpu().numpy().astype(np.float64), ref) <= 1e-5


def test_out_of_range_labels_and_init_indices_are_ignored_and_reported():
    """Labels outside [0, C) given to the update (or to kv_cluster_build as
    assign_in) leave their keys out of every cluster; init indices outside
    [0, N) are clamped into the head's keys. kv_cluster_build reports either
    case as KV_ERR_INVALID_ARG in the pool's status word. The clusters the
    valid labels define must equal the oracle's update over those keys alone."""
    cfg = wl.get_config(1, n_keys=2100, n_clusters=64, n_components=16)
    inp, keys, init = _keys(cfg, [0, 1])
    BH, N, d = keys.shape
    C = cfg.n_clusters
    keys_d = to_dev(keys, cfg.dtype)
    g = np.random.default_rng(5)
    lab = g.integers(0, C, (BH, N)).astype(np.int64)
    bad = g.random((BH, N)) < 0.05
    lab_bad = lab.copy()
    lab_bad[bad] = np.where(g.random(bad.sum()) < 0.5, -3, C + np.arange(bad.sum()) % 7)
    c0 = np.stack([keys[h][init[h]].astype(np.float64) for h in range(BH)])
    cg, cnt = _gpu_update(keys_d, lab_bad, c0)
    for h in range(BH):
        ok = ~bad[h]
        ref, rc = okm.update(keys[h][ok], lab[h][ok], c0[h])
        assert (cnt[h] == rc).all()
        assert _rel_err(cg[h], ref) <= 1e-5

    # through kv_cluster_build: status word, unit sizes, valid rows packed
    B, H = 1, BH
    pool = make_pool(B, H, d, cfg.dtype, N, C)
    vals_d = to_dev(inp["values"], cfg.dtype)
    rounds = torch.full((B, H), -1, dtype=torch.int32, device="cuda")
    kvc.kv_cluster_build(pool, keys_d.reshape(B, H, N, d), vals_d, C, 1,
                         torch.from_numpy(init.reshape(B, H, C)).cuda(),
                         assign_in=torch.from_numpy(lab_bad.astype(np.int32).reshape(B, H, N)).cuda(),
                         rounds_out=rounds)
    torch.cuda.synchronize()
    assert int(pool.status.item()) == kvc.KV_ERR_INVALID_ARG
    assert (rounds.cpu().numpy() == 0).all()  # a given clustering runs no round
    sizes = pool.unit_size[0].cpu().numpy()
    starts = pool.unit_start[0].cpu().numpy()
    pk = to_np(pool.k[0])
    for h in range(H):
        ok = ~bad[h]
        assert (sizes[h] == np.bincount(lab[h][ok], minlength=C)).all()
        order = np.argsort(lab[h][ok], kind="stable")
        np.testing.assert_array_equal(pk[h][:ok.sum()], keys[h][ok][order])
        assert starts[h][0] == 0

    # init indices out of range: clamped, reported, the rest of the build unchanged
    pool2 = make_pool(B, H, d, cfg.dtype, N, C)
    init_bad = init.copy().reshape(B, H, C)
    init_bad[0, 0, 3], init_bad[0, 1, 5] = -1, N + 10
    lab_out = torch.zeros(B, H, N, dtype=torch.int32, device="cuda")
    kvc.kv_cluster_build(pool2, keys_d.reshape(B, H, N, d), vals_d, C, 2,
                         torch.from_numpy(init_bad).cuda(), assign_out=lab_out)
    torch.cuda.synchronize()
    assert int(pool2.status.item()) == kvc.KV_ERR_INVALID_ARG
    lo = lab_out.cpu().numpy()
    assert lo.min() >= 0 and lo.max() < C
    assert int(pool2.unit_size.sum().item()) == H * N
