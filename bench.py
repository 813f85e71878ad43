#!/usr/bin/env python3
"""Benchmark of the centroid-indexed KV retrieval hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input. The
default workload (``--config 3``, long-in-long-out-128k-x36) is 36 layers of a
Qwen3-8B-shaped model (8 KV heads, 32 query heads, head dim 128, bf16, batch 1)
with 131072 prefill keys per KV head, C = 8192 clusters, 10 Lloyd rounds,
budget 2048 rows and 1024 decode steps:
  prefill : per layer, kv_cluster_build (K-means assign/update x10, then the
            pack of K/V into cluster-contiguous rows; a head whose assignment
            changes no label has reached a fixed point and skips the rounds
            left, and from the third round on only the centroids that moved
            are rescored, all with the result of ten whole rounds);
  decode  : 1024 steps x 36 layers of kv_decode_step, one launch per
            layer-step: the boundary test on the query pair; on a retrieval
            step, scoring of the centroids, the budgeted top-k selection and
            the copy of the selected rows into an HBM working set; then
            attention over the working set. The loop is replayed from captured
            HIP graphs on the seeded query walks.
Every layer draws its own prefill keys/values and query walk and clusters
into a pool of its own, so each layer-step reads its KV from HBM as in a real
model. Inputs are synthetic (seeded Gaussian-mixture keys, random values and
query walks) and resident in HBM before timing starts.

``--config`` selects another workload of the same family: 0 (tiny, fp32),
1 (one layer of 32768 keys, C = 2048, budget 512, 256 decode steps),
2 (long output: 2048 prefill keys, 16384 decode steps with temporal segments
and a 1024-token local buffer; the decode step is kv_boundary_segment_append
(boundary test + append in one launch) -> kv_select -> kv_gather_attend),
4 (16 sequences of 32768 keys, C = 2048, budget 1024, 512 decode steps).
``--launches two`` splits the layer-step into kv_boundary_select and
kv_fetch_attend; ``--attend pool`` attends the pool's rows directly
(kv_gather_attend reading the selection's row spans).

Printed JSON (one line): value = prefill keys clustered per second of whole
steps (the decode loop included); the split into prefill time and decode
microseconds per layer-step, the decode bytes moved per layer-step and the
fraction of HBM peak are extra fields. ``roofline`` covers the dominant
kernel by total time per step: the MFMA K-means assignment at the default
workload, the decode step's attention kernel (HBM bound) where that
dominates; ``roofline_assign`` and ``roofline_attend`` carry both. Both kernels are
timed with HIP events on the stream they run on around back-to-back
launches queued behind a GPU sleep, so that host enqueue gaps do not enter
the interval. ``cpu_baseline`` times the CPU oracle on a bounded sample of the
same work.

Variants (single-layer workloads without segments; the printed line names
them in ``config``): ``--pool host`` keeps the pool's K/V rows in pinned
host memory, as the LouisKV note deploys it, and each retrieval step copies
the selected rows into an HBM working set that attention reads
(kv_fetch_attend: the copy fused into the attention launch) -- the line then
carries ``fetch`` (the stand-alone gather kernel's and the fused retrieval
step's GB/s against the host link); ``--pool host-direct`` lets attention read host memory every step;
``--policy per-token|stride:S`` replaces the boundary test's decision of when
to retrieve; ``--units page:P`` uses pages of P consecutive keys as units. ``--overlap``
adds ``prefill_overlap``: layer 0's K-means on a second stream beside a
stand-in prefill forward of the same tokens, and the overhead it adds.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
HOST_LINK_GBS = 64.0        # MI355X host interface: PCIe 5.0 x16, one direction


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def profiled_traffic(workload):
    """HBM bytes per dispatch from the committed rocprofv3 counter summary of
    this workload, or None when there is none or the kernel sources changed
    since the counters were taken."""
    import hashlib
    import re

    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.md")
    if not os.path.exists(path):
        return None
    m = re.search(r"```json\n(.*?)\n```", open(path).read(), re.S)
    if not m:
        return None
    data = json.loads(m.group(1))
    h = hashlib.sha256()
    for f in ("decode.hip", "kmeans.hip", "kvc_internal.hpp"):
        with open(os.path.join(ROOT, "long_context_kv_kmeans_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    if h.hexdigest()[:16] != data.get("source_sha256_16"):
        return None
    return data


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return "unknown"


def cpu_baseline(cfg, inp, q, lloyd_iters, dk=None, dv=None):
    """Time the oracle on a bounded sample and scale to one whole step.

    The sample is Lloyd on one KV head of layer 0 (all of its keys, all C
    clusters, ``lloyd_iters`` of the rounds), its pack, and 16 decode steps of
    that head; the figure is extrapolated to every head, round, decode step
    and layer of the workload. numpy's BLAS runs with the threads it was
    given (OMP_NUM_THREADS); ``cores`` reports those."""
    import numpy as np

    from oracle import kmeans as okm
    from oracle.decode import run_decode

    affinity = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()
                     if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        cores = affinity
    keys0, vals0, init0 = inp["keys"][0, 0], inp["values"][0, 0], inp["init_idx"][0, 0]
    t0 = time.perf_counter()
    o = okm.lloyd(keys0, init0, lloyd_iters, mode="parity", dtype=cfg.dtype)
    t_lloyd = (time.perf_counter() - t0) * cfg.iters / lloyd_iters
    t0 = time.perf_counter()
    pack = okm.pack(keys0, vals0, o["labels"], o["centroids"], cfg.dtype)
    t_pack = time.perf_counter() - t0
    dec_steps = min(64, cfg.steps)
    t0 = time.perf_counter()
    seg = {} if dk is None else dict(buf_cap=cfg.buf_cap, dec_k=dk[:dec_steps, 0, :1],
                                     dec_v=dv[:dec_steps, 0, :1])
    run_decode([pack], q[:dec_steps, 0, :cfg.group], cfg.tau, cfg.budget, cfg.scale, cfg.dtype,
               **seg)
    t_dec = (time.perf_counter() - t0) / dec_steps  # one KV head, one step
    heads = cfg.batch * cfg.n_kv_heads
    t_step = cfg.layers * (heads * (t_lloyd + t_pack) + cfg.steps * heads * t_dec)
    return {
        "value": cfg.layers * heads * cfg.n_keys / t_step,
        "unit": "keys/s",
        "cores": int(cores),
        "kind": "oracle",
        "sample": (f"numpy fp64 oracle on layer 0, KV head 0 of {heads}: Lloyd over its "
                   f"{cfg.n_keys} keys with C={cfg.n_clusters} ({lloyd_iters} of {cfg.iters} "
                   f"rounds timed), the pack, and {dec_steps} of {cfg.steps} decode steps; "
                   f"scaled to {heads} heads, {cfg.iters} rounds, {cfg.steps} decode steps"
                   + (f" and {cfg.layers} layers" if cfg.layers > 1 else "")),
        "sample_s": t_lloyd * lloyd_iters / cfg.iters + t_pack + t_dec * dec_steps,
        "step_s_extrapolated": t_step,
        "decode_us_per_layer_step": t_dec * heads * 1e6,
        "affinity_cores": affinity,
        "cpu_model": cpu_model(),
    }


def prefill_overlap(kvc, y, n_clusters, iters, n_tokens, reps=5):
    """K-means of one layer's keys (kv_cluster_build on a second stream) while a
    stand-in prefill forward runs on the first: the dense GEMMs of one
    Qwen3-8B layer (QKV and output projections, gated MLP) over the same
    tokens, with random weights, through torch's GEMMs. The stand-in leaves
    out the attention itself and the norms. Returns the median times of the
    stand-in alone, the clustering alone, both launched together, and the
    overhead of the pair over the stand-in alone."""
    import numpy as np
    import torch

    hid, inter, qkv = 4096, 12288, (32 + 2 * 8) * 128
    g = torch.Generator(device="cuda").manual_seed(0)

    def w(*shape):
        return (torch.randn(*shape, generator=g, device="cuda") / shape[0] ** 0.5).bfloat16()

    x = torch.randn(n_tokens, hid, generator=g, device="cuda").bfloat16()
    w_qkv, w_o, w_gu, w_d = w(hid, qkv), w(hid, hid), w(hid, 2 * inter), w(inter, hid)
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()

    def standin():
        with torch.cuda.stream(sa):
            h = x @ w_qkv
            o = h[:, :hid] @ w_o
            gu = o @ w_gu
            act = torch.nn.functional.silu(gu[:, :inter]) * gu[:, inter:]
            return act @ w_d

    def kmeans():
        kvc.kv_cluster_build(y.pool, y.keys, y.vals, n_clusters, iters, y.init,
                             assign_in=y.assign_in,
                             assign_out=None if y.assign_in is not None else y.labels,
                             ws=y.ws_build, stream=sb)

    def timed(parts):
        """Both streams start together behind a GPU sleep (so that the host has
        enqueued everything first); the interval ends when both are done."""
        cur = torch.cuda.current_stream()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(20_000_000)
        a.record(cur)
        sa.wait_event(a)
        sb.wait_event(a)
        for f in parts:
            f()
        for s_ in (sa, sb):
            e_ = torch.cuda.Event()
            e_.record(s_)
            cur.wait_event(e_)
        b.record(cur)
        torch.cuda.synchronize()
        return a.elapsed_time(b)

    for f in (standin, kmeans):
        timed([f])  # warm
    t_a = float(np.median([timed([standin]) for _ in range(reps)]))
    t_b = float(np.median([timed([kmeans]) for _ in range(reps)]))
    t_ab = float(np.median([timed([standin, kmeans]) for _ in range(reps)]))
    flops = 2.0 * n_tokens * hid * (qkv + hid + 2 * inter) + 2.0 * n_tokens * inter * hid
    return {"standin": "Qwen3-8B layer GEMMs (QKV, O, gate/up, down) over "
                       f"{n_tokens} tokens, bf16, torch matmul; no attention or norms",
            "standin_ms": t_a, "standin_tflops": flops / (t_a * 1e-3) / 1e12,
            "kmeans_ms": t_b, "both_ms": t_ab, "overhead_frac": t_ab / t_a - 1.0,
            "serial_overhead_frac": t_b / t_a}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", type=int, default=3,
                    help="workload (default 3: 36 layers x 131072 keys per KV head, the largest "
                         "that fits one GPU)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-lloyd-iters", type=int, default=None,
                    help="Lloyd rounds the CPU oracle is timed on (default 3)")
    ap.add_argument("--gen-threads", type=int, default=None,
                    help="host threads drawing the synthetic inputs (default: min(16, cores))")
    ap.add_argument("--decode-steps", type=int, default=None,
                    help="run fewer decode steps than the workload's (counter-profiling runs "
                         "only; the printed line then names the override)")
    ap.add_argument("--assign-reps", type=int, default=20)
    ap.add_argument("--attend-reps", type=int, default=100)
    ap.add_argument("--copy-calibration-mib", type=int, default=64)
    ap.add_argument("--cold-mib", type=int, default=512,
                    help="total size of the working-set copies the cold attention timing "
                         "cycles through")
    ap.add_argument("--pool", choices=("hbm", "host", "host-direct"), default="hbm",
                    help="where the pool's K/V rows live: hbm; host (pinned host memory, "
                         "retrieval steps fetch the selected rows into an HBM working set "
                         "that attention reads); host-direct (attention reads host memory "
                         "every step)")
    ap.add_argument("--attend", choices=("wset", "pool"), default="wset",
                    help="HBM pool without a local buffer: attend an HBM working set holding "
                         "the current selection's rows (kv_fetch_attend), or the pool's rows "
                         "through the selection's spans (kv_gather_attend)")
    ap.add_argument("--fetch", choices=("fused", "separate"), default="fused",
                    help="--pool host: the working-set copy inside the attention launch "
                         "(kv_fetch_attend) or as a launch of its own (kv_fetch_selected, "
                         "then kv_gather_attend)")
    ap.add_argument("--launches", choices=("one", "two"), default="one",
                    help="pools without a local buffer, fused working-set fetch, boundary "
                         "policy: one launch per layer-step (kv_decode_step: boundary test, "
                         "selection on retrieval steps, fetch and attention) or two "
                         "(kv_boundary_select, then kv_fetch_attend)")
    ap.add_argument("--policy", default="boundary",
                    help="when to retrieve: boundary (the cosine test), per-token, stride:S")
    ap.add_argument("--units", default="cluster",
                    help="retrieval units: cluster (K-means) or page:P (P consecutive keys)")
    ap.add_argument("--overlap", action="store_true",
                    help="also time layer 0's K-means on a second stream beside a stand-in "
                         "prefill forward (GEMMs of one layer) and report the overhead")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); this path has no "
              "multi-GPU mode", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import long_context_kv_kmeans_amd as kvc
    import workloads as wl

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    kvc.lib()  # fail loudly if the HIP library is missing
    torch.cuda.set_device(0)
    cfg = wl.get_config(args.config)
    if args.decode_steps is not None:
        cfg = cfg.replace(steps=args.decode_steps)
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    e = 2 if cfg.dtype == "bf16" else 4
    B, H, N, d = cfg.batch, cfg.n_kv_heads, cfg.n_keys, cfg.head_dim
    C, T, Hq, L = cfg.n_clusters, cfg.steps, cfg.n_q_heads, cfg.layers
    seg = cfg.buf_cap > 0
    host = args.pool != "hbm"
    # working set: always for a host pool ("host"); for an HBM pool without a
    # local buffer unless --attend pool
    fetch = args.pool == "host" or (args.pool == "hbm" and cfg.buf_cap == 0
                                    and args.attend == "wset")
    sched = wl.retrieval_schedule(args.policy, T)
    page = int(args.units.split(":", 1)[1]) if args.units.startswith("page:") else None
    if args.units != "cluster" and page is None:
        raise SystemExit(f"unknown --units {args.units!r}")
    variant = host or sched is not None or page is not None
    # the whole layer-step in one launch where the path is boundary test -> select ->
    # fused fetch + attention; per-token retrieval is that launch with a boundary
    # threshold no cosine reaches (every step retrieves)
    every = sched is not None and bool(sched.all())
    one = (fetch and args.fetch == "fused" and not seg and (sched is None or every)
           and args.launches == "one" and args.pool != "host-direct" and cfg.dtype == "bf16")
    tau_step = float("inf") if every else cfg.tau
    if seg and (sched is not None or page is not None or (fetch and args.fetch == "separate")):
        raise SystemExit("with decode segments (--config 2) only --pool host|host-direct "
                         "(fused fetch) applies")
    if page is not None:
        C = -(-N // page)  # one unit per page
    # units: clusters, plus (long-output) the segments closed during decode
    unit_cap = C + min(T, 8192 - C) if seg else C
    row_cap = N + (T if seg else 0)
    sel_cap = min(cfg.budget, unit_cap)

    class Layer:
        pass

    # Every layer draws its own prefill keys/values and query walk; the
    # (sequence, head) streams of a layer are drawn on several host threads and
    # the next layers' are drawn while the current one is uploaded.
    import concurrent.futures as cf

    gen_threads = args.gen_threads or max(1, min(16, len(os.sched_getaffinity(0))))
    per_layer = max(1, gen_threads // 2) if L > 1 else gen_threads

    def gen_layer(li):
        return wl.layer_inputs(cfg, li, threads=per_layer), wl.layer_queries(cfg, li)[0]

    layers = []
    t_gen = time.perf_counter()
    gen_ex = cf.ThreadPoolExecutor(max_workers=2 if L > 1 else 1)
    pending = [gen_ex.submit(gen_layer, li) for li in range(min(L, 2))]
    for li in range(L):
        inp_l, q_l = pending[li].result()
        pending[li] = None
        if li + 2 < L:
            pending.append(gen_ex.submit(gen_layer, li + 2))
        y = Layer()
        y.assign_in = None
        y.keys = torch.from_numpy(inp_l["keys"]).cuda().to(tdt)
        y.vals = torch.from_numpy(inp_l["values"]).cuda().to(tdt)
        y.init = torch.from_numpy(inp_l["init_idx"]).cuda()
        y.q = torch.from_numpy(q_l).to(tdt).cuda()  # [T, B, Hq, d]
        if seg:
            dk, dv = wl.layer_decode_kv(cfg, li)
            y.dk = torch.from_numpy(dk).to(tdt).cuda()  # [T, B, H, d]
            y.dv = torch.from_numpy(dv).to(tdt).cuda()
        y.pool = kvc.Pool(B, H, d, tdt, row_cap=row_cap, unit_cap=unit_cap, buf_cap=cfg.buf_cap,
                          host_kv=host)
        if fetch:  # HBM working set: the rows of the current selection, one span per head
            y.wset = kvc.Pool(B, H, d, tdt, row_cap=cfg.budget, unit_cap=1)
            y.wspans = torch.zeros(B, H, 1, 2, dtype=torch.int32, device="cuda")
            y.wn = torch.zeros(B, H, dtype=torch.int32, device="cuda")
        if sched is not None:
            y.sched = torch.from_numpy(np.repeat(sched[:, None], B, axis=1).astype(np.uint8)).cuda()
        if page is not None:
            y.assign_in = torch.from_numpy(wl.page_labels(B, H, N, page)).cuda()
            y.init = torch.from_numpy(np.broadcast_to(
                (np.arange(C) * page).astype(np.int32), (B, H, C)).copy()).cuda()
        y.labels = torch.zeros(B, H, N, dtype=torch.int32, device="cuda")
        y.rounds = torch.zeros(B, H, dtype=torch.int32, device="cuda")  # Lloyd rounds run per head
        y.sweeps = torch.zeros(B, H, dtype=torch.float32, device="cuda")  # assignment work
        y.flags = torch.zeros(T, B, dtype=torch.uint8, device="cuda")
        y.sel = torch.zeros(B, H, sel_cap, dtype=torch.int32, device="cuda")
        y.sel_n = torch.zeros(B, H, dtype=torch.int32, device="cuda")
        y.sel_rows = torch.zeros(B, H, dtype=torch.int32, device="cuda")
        y.sel_spans = torch.zeros(B, H, sel_cap, 2, dtype=torch.int32, device="cuda")
        y.out = torch.zeros(B, Hq, d, dtype=torch.float32, device="cuda")
        if li == 0:  # the layers run one after another on one stream: one set of workspaces
            ws_build = kvc.workspace(kvc.kv_cluster_build_workspace(B, H, N, d, C, tdt))
            ws_sel = kvc.workspace(kvc.kv_select_workspace(y.pool, Hq))
            ws_att = kvc.workspace(kvc.kv_gather_attend_workspace(y.pool, Hq, cfg.budget))
            ws_step = (kvc.workspace(kvc.kv_decode_step_workspace(y.pool, Hq, cfg.budget))
                       if one else None)
        y.ws_build, y.ws_sel, y.ws_att, y.ws_step = ws_build, ws_sel, ws_att, ws_step
        layers.append(y)
        if li == 0:  # layer 0, sequence 0, KV head 0 feeds the CPU baseline
            inp = {k: np.ascontiguousarray(inp_l[k][:1, :1]) for k in ("keys", "values",
                                                                       "init_idx")}
            q_np = q_l
            dk0, dv0 = (dk, dv) if seg else (None, None)
        del inp_l, q_l
        if L > 1 and (li + 1) % 6 == 0:
            log(f"inputs of {li + 1}/{L} layers generated and uploaded "
                f"({time.perf_counter() - t_gen:.0f}s)")
    gen_ex.shutdown()
    log(f"inputs generated in {time.perf_counter() - t_gen:.1f}s")
    y0 = layers[0]
    keys, pool, sel, sel_n, sel_rows, sel_spans = (y0.keys, y0.pool, y0.sel, y0.sel_n,
                                                   y0.sel_rows, y0.sel_spans)

    def prefill():
        for y in layers:
            kvc.kv_cluster_build(y.pool, y.keys, y.vals, C, cfg.iters, y.init,
                                 assign_in=y.assign_in,
                                 assign_out=None if y.assign_in is not None else y.labels,
                                 ws=y.ws_build, rounds_out=y.rounds, sweeps_out=y.sweeps)

    def decode_step(y, t):
        q_prev = y.q[t - 1] if t else None
        flag = y.flags[t]
        if one:
            kvc.kv_decode_step(y.pool, q_prev, y.q[t], tau_step, cfg.scale, cfg.budget, flag,
                               y.sel, y.sel_spans, y.sel_n, y.sel_rows, y.wset, y.wspans, y.wn,
                               y.out, ws=y.ws_step)
            return
        if seg:  # boundary + segment append -> selection -> attention
            kvc.kv_boundary_segment_append(y.pool, q_prev, y.q[t], cfg.tau, y.dk[t], y.dv[t],
                                           y.flags[t])
            kvc.kv_select(y.pool, y.q[t], cfg.budget, y.flags[t], y.sel, y.sel_n, y.sel_rows,
                          ws=y.ws_sel, sel_spans=y.sel_spans)
        elif sched is not None:  # the schedule decides; no boundary test
            flag = y.sched[t]
            kvc.kv_select(y.pool, y.q[t], cfg.budget, flag, y.sel, y.sel_n, y.sel_rows,
                          ws=y.ws_sel, sel_spans=y.sel_spans)
        else:
            kvc.kv_boundary_select(y.pool, q_prev, y.q[t], cfg.tau, cfg.budget, y.flags[t],
                                   y.sel, y.sel_n, y.sel_rows, ws=y.ws_sel,
                                   sel_spans=y.sel_spans)
        if fetch and args.fetch == "fused":  # working-set copy inside the attention
            kvc.kv_fetch_attend(y.pool, y.q[t], cfg.scale, flag, None, y.sel_n, cfg.budget,
                                y.wset, y.wspans, y.wn, y.out, ws=y.ws_att,
                                sel_spans=y.sel_spans)
        elif fetch:
            kvc.kv_fetch_selected(y.pool, flag, None, y.sel_n, y.wset, y.wspans, y.wn,
                                  sel_spans=y.sel_spans)
            kvc.kv_gather_attend(y.wset, y.q[t], cfg.scale, None, y.wn, cfg.budget, y.out,
                                 ws=y.ws_att, sel_spans=y.wspans)
        else:
            kvc.kv_gather_attend(y.pool, y.q[t], cfg.scale, None, y.sel_n, cfg.budget, y.out,
                                 ws=y.ws_att, sel_spans=y.sel_spans)

    def decode(t0, t1, record=None):
        for t in range(t0, t1):
            for y in layers:
                decode_step(y, t)
            if record is not None:
                record[0][t].copy_(y0.sel_rows)
                if seg:
                    record[1][t].copy_(y0.pool.n_rows - y0.pool.buf_begin)

    # eager pass: loads kernels and records the per-step work for the byte count
    prefill()
    rec = (torch.zeros(T, B, H, dtype=torch.int32, device="cuda"),
           torch.zeros(T, B, dtype=torch.int32, device="cuda"))
    decode(0, T, rec)
    torch.cuda.synchronize()
    rows = rec[0].cpu().numpy().astype(np.int64)   # [T, B, H] selected pool rows (layer 0)
    buf_rows = rec[1].cpu().numpy().astype(np.int64) if seg else np.zeros((T, B), np.int64)
    fl = (y0.flags if sched is None else y0.sched).cpu().numpy().astype(bool)  # [T, B]
    n_cand = C  # candidates scored on a retrieval step (clusters; segments add a few)
    bytes_steps = (2 * Hq * d * e * B
                   + fl.sum(1) * H * n_cand * (d * e + 4)
                   + (rows.sum((1, 2)) + H * buf_rows.sum(1)) * 2 * d * e
                   + B * Hq * d * 4)
    dec_bytes = float(bytes_steps.mean())
    log(f"retrieval steps: {int(fl.sum())} of {T} (layer 0); mean selected rows/head "
        f"{rows.mean():.1f}" + (f", mean buffer rows {buf_rows.mean():.1f}" if seg else ""))

    # capture the decode loop in graphs of at most ~4096 launches; replay per step
    stream = torch.cuda.Stream()
    calls = (1 if one else 3 if seg or (fetch and args.fetch == "separate") else 2) * L
    chunk = max(1, min(T, 4096 // calls))
    with torch.cuda.stream(stream):
        prefill()
        decode(0, T)  # warm on the capture stream
    torch.cuda.synchronize()
    graphs = []
    prefill()  # decode state as after a prefill
    torch.cuda.synchronize()
    for t0 in range(0, T, chunk):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            decode(t0, min(T, t0 + chunk))
        graphs.append(g)
    torch.cuda.synchronize()
    log(f"decode captured in {len(graphs)} graph(s) of up to {chunk} steps x {calls} launches")

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]

    def step(i=None):
        with torch.cuda.stream(stream):
            if i is not None:
                ev[i][0].record(stream)
            prefill()
            if i is not None:
                ev[i][1].record(stream)
            for g in graphs:
                g.replay()
            if i is not None:
                ev[i][2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_step = elapsed * 1e3 / args.steps
    pre_ms = float(np.mean([a.elapsed_time(b) for a, b, _ in ev]))
    dec_ms = float(np.mean([b.elapsed_time(c) for _, b, c in ev]))
    dec_us = dec_ms * 1e3 / (T * L)
    for y in layers:
        st = int(y.pool.status.item())
        if st != 0:
            raise SystemExit(f"pool status {st} ({kvc.lib().kv_status_string(st).decode()})")

    def launch_ms(fn, reps, name="launch"):
        """Mean GPU time per launch of fn: `reps` back-to-back launches on
        `stream` between two HIP events, all queued behind a GPU sleep so that
        the host's enqueue rate does not stretch the interval. If the first
        event has already completed when the last launch is queued, the GPU
        may have waited for the host: the sleep is lengthened and the
        measurement taken again."""
        cycles = 20_000_000
        t_host = 0.0
        for _ in range(5):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            with torch.cuda.stream(stream):
                fn()
                torch.cuda._sleep(cycles)
                a.record(stream)
                t0_host = time.perf_counter()
                for _ in range(reps):
                    fn()
                t_host = time.perf_counter() - t0_host
                starved = a.query()
                b.record(stream)
            torch.cuda.synchronize()
            if not starved:
                return a.elapsed_time(b) / reps
            cycles *= 4
        raise SystemExit(f"{name} timing: the host could not queue {reps} launches ahead of the "
                         f"GPU ({t_host * 1e3:.1f} ms to queue them)")

    # gather-attend on the final step's selection (the state the graph left)
    sel_units_n = int(sel_n.sum().item())
    att_rows = int(sel_rows.sum().item())
    q_extra = 0
    if one:
        # the whole layer-step on a step without retrieval for every sequence (the
        # boundary test, then the working set): two adjacent queries of a drift step
        if sched is None:
            drift = ~fl.any(1)
        else:  # the schedule retrieved every step: where would the boundary test not?
            fb = torch.zeros(T, B, dtype=torch.uint8, device="cuda")
            for t in range(1, T):
                kvc.kv_boundary(y0.q[t - 1], y0.q[t], cfg.tau, fb[t])
            drift = ~fb.cpu().numpy().astype(bool).any(1)
            drift[0] = False
        if not drift.any():
            raise SystemExit("no decode step without retrieval to time the plain layer-step on")
        t_nr = int(np.nonzero(drift)[0][-1])
        flag_tmp = torch.zeros(B, dtype=torch.uint8, device="cuda")

        def att_fn(wset=None):
            kvc.kv_decode_step(pool, y0.q[t_nr - 1], y0.q[t_nr], cfg.tau, cfg.scale, cfg.budget,
                               flag_tmp, sel, sel_spans, sel_n, sel_rows, wset or y0.wset,
                               y0.wspans, y0.wn, y0.out, ws=y0.ws_step)
        att_spans = int(y0.wn.sum().item())
        q_extra = B * Hq * d * e  # the previous query, read by the boundary test
    elif fetch:  # a step without retrieval: the working set (+ the local buffer's HBM copy)
        zeros = torch.zeros(B, dtype=torch.uint8, device="cuda")

        def att_fn(wset=None):
            kvc.kv_fetch_attend(pool, y0.q[T - 1], cfg.scale, zeros, None, sel_n, cfg.budget,
                                wset or y0.wset, y0.wspans, y0.wn, y0.out, ws=y0.ws_att,
                                sel_spans=sel_spans)
        att_spans = int(y0.wn.sum().item())
    else:
        def att_fn():
            kvc.kv_gather_attend(pool, y0.q[T - 1], cfg.scale, None, sel_n, cfg.budget, y0.out,
                                 ws=y0.ws_att, sel_spans=sel_spans)
        att_spans = sel_units_n
    att_ms = launch_ms(att_fn, args.attend_reps, "attention")
    # Cold: the same launch over copies of the rows it reads, more than
    # --cold-mib of them, taken in turn back to back, so that every launch
    # finds its rows in neither the L2s nor the Infinity Cache (256 MB).
    att_cold_ms, n_copies = None, 0
    per_copy = 2 * B * H * cfg.budget * d * e
    # (working sets under 1 MiB would need thousands of copies, more launches
    # than the host queues ahead of the GPU: no cold figure for those)
    if fetch and per_copy >= (1 << 20):
        n_copies = max(2, -(-(args.cold_mib << 20) // per_copy))
        copies = []
        for _ in range(n_copies):
            c = kvc.Pool(B, H, d, tdt, row_cap=cfg.budget, unit_cap=1)
            c.k.copy_(y0.wset.k)
            c.v.copy_(y0.wset.v)
            copies.append(c)
        it = [0]

        def cold_fn():
            c = copies[it[0] % n_copies]
            it[0] += 1
            att_fn(c)
        att_cold_ms = launch_ms(cold_fn, max(args.attend_reps, 2 * n_copies), "cold attention")
        del copies
    att_buf = int((pool.n_rows - pool.buf_begin).sum().item()) * H if seg else 0
    att_bytes = ((att_rows + att_buf) * 2 * d * e  # selected (and local-buffer) K and V rows
                 + B * Hq * d * e + q_extra    # queries
                 + B * Hq * d * 4              # fp32 output
                 + att_spans * 8)              # row span (start, size) per selected unit
    att_gbs = att_bytes / (att_ms * 1e-3) / 1e9
    att_peak = HOST_LINK_GBS if args.pool == "host-direct" else HBM_PEAK_GBS

    fetch_res = None
    if args.pool == "host":
        # the working-set fetch of the final selection, every sequence retrieving
        ones = torch.ones(B, dtype=torch.uint8, device="cuda")
        f_ms = launch_ms(lambda: kvc.kv_fetch_selected(pool, ones, None, sel_n, y0.wset,
                                                       y0.wspans, y0.wn, sel_spans=sel_spans),
                         args.attend_reps)
        f_bytes = att_rows * 2 * d * e  # K and V rows read over the host link
        # a retrieval step of the fused call: copy into the working set + attention
        fa_ms = launch_ms(lambda: kvc.kv_fetch_attend(pool, y0.q[T - 1], cfg.scale, ones, None,
                                                      sel_n, cfg.budget, y0.wset, y0.wspans,
                                                      y0.wn, y0.out, ws=y0.ws_att,
                                                      sel_spans=sel_spans),
                          args.attend_reps)
        # a plain pinned-host -> HBM copy of 64 MiB: the link's practical rate here
        hsrc = torch.ones(16 << 20, dtype=torch.float32, pin_memory=True)
        hdst = torch.empty(16 << 20, dtype=torch.float32, device="cuda")
        h2d_ms = launch_ms(lambda: hdst.copy_(hsrc, non_blocking=True), 5)
        del hsrc, hdst
        fetch_res = {"bound": "host-link", "kernel": "k_fetch_rows (kv_fetch_selected)",
                     "achieved": f_bytes / (f_ms * 1e-3) / 1e9, "peak": HOST_LINK_GBS,
                     "unit": "GB/s", "frac": f_bytes / (f_ms * 1e-3) / 1e9 / HOST_LINK_GBS,
                     "bytes_per_launch": f_bytes, "avg_launch_ms": f_ms,
                     "h2d_copy_gbs": (64 << 20) / (h2d_ms * 1e-3) / 1e9,
                     "fetch_attend_retrieval_ms": fa_ms,
                     "fetch_attend_gbs": f_bytes / (fa_ms * 1e-3) / 1e9}

    # Phases of a retrieval step, every sequence retrieving: the selection alone
    # (kv_select: scoring + budgeted selection, one launch) and, on the
    # one-launch path, the whole retrieval layer-step (kv_decode_step with a
    # threshold no cosine reaches: boundary test, scoring, selection, working-set
    # fetch, attention) beside the plain layer-step timed above. Last, since both
    # rewrite the selection and the working set.
    retrieval = None
    if fetch and not seg and cfg.dtype == "bf16" and args.pool != "host-direct":
        ws_sel0 = y0.ws_sel
        sel_ms = launch_ms(lambda: kvc.kv_select(pool, y0.q[T - 1], cfg.budget, None, sel, sel_n,
                                                 sel_rows, ws=ws_sel0, sel_spans=sel_spans),
                           args.attend_reps)
        retrieval = {"select_us": sel_ms * 1e3, "units_scored": B * H * C}
        if one:
            flag_r = torch.zeros(B, dtype=torch.uint8, device="cuda")
            ret_ms = launch_ms(lambda: kvc.kv_decode_step(
                pool, y0.q[T - 2], y0.q[T - 1], float("inf"), cfg.scale, cfg.budget, flag_r, sel,
                sel_spans, sel_n, sel_rows, y0.wset, y0.wspans, y0.wn, y0.out, ws=y0.ws_step),
                args.attend_reps)
            retrieval.update({"step_us": ret_ms * 1e3, "plain_step_us": att_ms * 1e3})
        retrieval["how"] = ("HIP events around back-to-back launches on the final step's "
                            "queries, every sequence retrieving; select_us: kv_select (scoring + "
                            "selection)" + ("; step_us: kv_decode_step retrieving (boundary, "
                                            "scoring, selection, working-set fetch, attention); "
                                            "plain_step_us: the same launch on a step without "
                                            "retrieval" if one else ""))

    # MFMA K-means assignment against prepared centroids (the kernel the
    # prefill runs once per Lloyd round)
    cents = pool.unit_mean[:, :, :C].reshape(B * H, C, d).contiguous()
    k3 = keys.reshape(B * H, N, d)
    lab2 = torch.zeros(B * H, N, dtype=torch.int32, device="cuda")
    ws_asg = kvc.workspace(kvc.lib().kv_kmeans_assign_workspace(B * H, C, d, kvc.dtype_code(tdt)))
    with torch.cuda.stream(stream):
        kvc.kv_kmeans_prepare(cents, tdt, ws_asg)
    asg_fn = lambda: kvc.kv_kmeans_assign_prepared(k3, cents, lab2, ws_asg)  # noqa: E731
    asg_ms = launch_ms(asg_fn, args.assign_reps)
    flops = 2.0 * B * H * N * C * d
    achieved = flops / (asg_ms * 1e-3) / 1e12
    # assignment work per step in whole sweeps (sweeps_out of each build): a
    # head at a fixed point of Lloyd's iteration skips its later rounds, and
    # rounds after the second score only the centroids that moved
    rounds_run = [float(y.rounds.float().mean().item()) for y in layers]
    sweeps_run = [float(y.sweeps.mean().item()) for y in layers]
    share = {"k_gather_attend": T * L * att_ms / ms_step,
             "k_assign_mfma": (0 if page is not None else sum(sweeps_run)) * asg_ms / ms_step}

    # What this machine reaches on plain work: a 1 GiB device copy (bytes read +
    # written) and a large bf16 GEMM through torch (hipBLASLt).
    big = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    big2 = torch.empty_like(big)
    copy_ms = launch_ms(lambda: big2.copy_(big), 10)
    del big, big2
    ga = torch.randn(8192, 8192, device="cuda").bfloat16()
    gb = torch.randn(8192, 8192, device="cuda").bfloat16()
    gemm_ms = launch_ms(lambda: torch.matmul(ga, gb), 10)
    del ga, gb
    achievable = {"copy_gbs": 2 * (1 << 30) / (copy_ms * 1e-3) / 1e9,
                  "gemm_bf16_tflops": 2.0 * 8192 ** 3 / (gemm_ms * 1e-3) / 1e12,
                  "how": "1 GiB device-to-device copy (read + write bytes); "
                         "8192^3 bf16 torch.matmul"}

    # the committed counter profile covers the default path only
    traffic = profiled_traffic(cfg.name) if (not variant and args.attend == "wset"
                                             and args.decode_steps is None) else None
    roof_attend = {"bound": "hbm" if args.pool != "host-direct" else "host-link",
                   "kernel": ("k_gather_attend_mfma (kv_decode_step: boundary test + "
                              "working set, step without retrieval)" if one else
                              "k_gather_attend_mfma (kv_fetch_attend, working set, step "
                              "without retrieval)" if fetch else
                              "k_gather_attend_mfma (kv_gather_attend)"),
                   "achieved": att_gbs, "peak": att_peak, "unit": "GB/s",
                   "frac": att_gbs / att_peak,
                   "traffic": traffic["k_gather_attend_mfma"]["bytes"] if traffic else None,
                   "bytes_per_launch": att_bytes, "avg_launch_ms": att_ms,
                   "cold": None if att_cold_ms is None else {
                       "avg_launch_ms": att_cold_ms,
                       "achieved": att_bytes / (att_cold_ms * 1e-3) / 1e9,
                       "frac": att_bytes / (att_cold_ms * 1e-3) / 1e9 / att_peak,
                       "how": f"back-to-back launches over {n_copies} copies of the working "
                              f"set taken in turn (>= {args.cold_mib} MiB, more than the "
                              "Infinity Cache holds)"},
                   "frac_of_achievable": (att_gbs / achievable["copy_gbs"]
                                          if args.pool != "host-direct" else None)}
    roof_assign = {"bound": "mfma", "kernel": "k_assign_mfma (kv_kmeans_assign_prepared)",
                   "achieved": achieved, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                   "frac": achieved / BF16_PEAK_TFLOPS,
                   "traffic": traffic["k_assign_mfma"]["bytes"] if traffic else None,
                   "flops_per_launch": flops, "avg_launch_ms": asg_ms,
                   "frac_of_achievable": achieved / achievable["gemm_bf16_tflops"]}
    # `roofline` is the kernel with the larger share of step time
    dominant = "assign" if share["k_assign_mfma"] >= share["k_gather_attend"] else "attend"
    keys_per_step = L * B * H * N
    res = {
        "metric": "prefill keys clustered/s; decode select+gather+attend us/layer-step, %HBM peak",
        "value": keys_per_step / (ms_step * 1e-3),
        "unit": "keys/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": cfg.name, "layers": L, "batch": B, "n_kv_heads": H,
                   "n_q_heads": Hq, "head_dim": d, "n_keys": N, "n_clusters": C,
                   "iters": cfg.iters, "decode_steps": T, "budget": cfg.budget,
                   "local_buffer": cfg.buf_cap, "tau": cfg.tau, "pool": args.pool,
                   "fetch": args.fetch if fetch else None,
                   "launches_per_layer_step": calls // L,
                   "attend": "wset" if fetch else "pool",
                   "policy": args.policy, "units": args.units,
                   "prefill_keys_shared_across_layers": False,
                   "decode_steps_overridden": args.decode_steps is not None},
        "retrieval_steps": int(fl.sum()),
        "lloyd_rounds_per_head": sum(rounds_run) / L,
        "assign_sweeps_per_head": sum(sweeps_run) / L,
        "retrieval": retrieval,
        "prefill_ms": pre_ms,
        "prefill_keys_per_s": keys_per_step / (pre_ms * 1e-3),
        "decode_us_per_layer_step": dec_us,
        "decode_bytes_per_layer_step": dec_bytes,
        "decode_hbm_frac": dec_bytes / (dec_us * 1e-6) / (HBM_PEAK_GBS * 1e9),
        "roofline": dict(roof_assign if dominant == "assign" else roof_attend),
        "roofline_assign": roof_assign,
        "roofline_attend": roof_attend,
        "achievable": achievable,
        "time_share_per_step": share,
    }
    if fetch_res is not None:
        res["fetch"] = fetch_res
    if args.overlap:
        log("timing K-means beside a stand-in prefill forward ...")
        res["prefill_overlap"] = prefill_overlap(kvc, y0, C, cfg.iters, B * N)
    # A plain copy of known size after the timed region: the reference that
    # scales rocprofv3's FETCH_SIZE / WRITE_SIZE counters to bytes.
    if args.copy_calibration_mib > 0:
        nb = args.copy_calibration_mib << 20
        src = torch.ones(nb // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if variant:
        res["cpu_baseline"] = None  # the oracle's sample covers the standard path only
    elif not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample ...")
        iters = args.cpu_lloyd_iters or 3
        res["cpu_baseline"] = cpu_baseline(cfg, inp, q_np, iters, dk0, dv0)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
