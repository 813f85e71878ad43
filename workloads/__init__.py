"""Seeded synthetic inputs for centroid-indexed KV retrieval.

This module only draws random numbers and stores them in the working dtype.
It holds none of the method's arithmetic (no distances, means, scores,
selection or attention), so both the CPU oracle and the HIP path can take
their inputs from it without sharing any of the computation under test.

Recipe (the same for every config; only the shape parameters change):

* Every random stream is ``numpy.random.default_rng([1000 + cfg, tag, layer,
  seq, head])`` (PCG64 seeded through ``SeedSequence``), with a distinct
  ``tag`` per quantity, so any (layer, sequence, head) can be regenerated on
  its own.
* Keys of one KV head: a Gaussian mixture. Component means ~ N(0, I_d);
  each key picks a component (uniformly, or with lognormal(0, 1) weights when
  ``lognormal_weights``) and adds ``sigma * N(0, I_d)`` (sigma = 0.3).
* Values ~ N(0, I_d).
* K-means init: ``n_clusters`` distinct key indices drawn uniformly without
  replacement.
* Query walk of one (layer, sequence): q_0 ~ N(0, I) for all query heads;
  at each later step one Bernoulli(p_jump) decides whether all heads jump to
  fresh N(0, I) vectors, otherwise q_t = q_{t-1} + walk_sigma * N(0, I).
* Decode keys (long-output config): drawn from the same mixture as that
  head's prefill keys; decode values ~ N(0, I).
* Every tensor is rounded once to the working dtype (bf16 by round to
  nearest even, through torch's own conversion) and returned as float32
  numpy arrays whose values are exactly representable in that dtype.

The five workloads mirror the pages' scenarios: long input/short output,
short input/long output (segments) and long input/long output, with
Qwen3-8B attention shapes (32 query heads, 8 KV heads, head dim 128).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

# Stream tags (part of the seed tuple).
TAG_MIX_MEANS = 1
TAG_KEYS = 2
TAG_VALUES = 3
TAG_INIT = 4
TAG_WALK = 5
TAG_DEC_KEYS = 6
TAG_DEC_VALUES = 7
TAG_MIX_WEIGHTS = 8


@dataclasses.dataclass(frozen=True)
class Config:
    """Shape and workload parameters of one synthetic configuration."""

    idx: int
    name: str
    layers: int
    batch: int
    n_kv_heads: int
    n_q_heads: int
    head_dim: int
    dtype: str  # "fp32" | "bf16"
    n_keys: int
    n_components: int
    key_sigma: float
    lognormal_weights: bool
    n_clusters: int
    iters: int
    steps: int
    walk_sigma: float
    p_jump: float
    tau: float
    budget: int
    buf_cap: int  # 0: no decode segments

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.head_dim))

    def replace(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


CONFIGS = [
    Config(0, "tiny-fp32", 1, 1, 2, 4, 64, "fp32", 2048, 64, 0.3, False,
           32, 10, 64, 0.05, 0.1, 0.7, 256, 0),
    Config(1, "qwen3-8b-layer-32k", 1, 1, 8, 32, 128, "bf16", 32768, 512, 0.3,
           False, 2048, 10, 256, 0.05, 0.02, 0.7, 512, 0),
    Config(2, "long-output-16k", 1, 1, 8, 32, 128, "bf16", 2048, 64, 0.3,
           False, 128, 10, 16384, 0.05, 0.02, 0.7, 1024, 1024),
    Config(3, "long-in-long-out-128k-x36", 36, 1, 8, 32, 128, "bf16", 131072,
           4096, 0.3, False, 8192, 10, 1024, 0.05, 0.02, 0.7, 2048, 0),
    Config(4, "batched-decode-b16-32k", 1, 16, 8, 32, 128, "bf16", 32768, 512,
           0.3, True, 2048, 10, 512, 0.05, 0.02, 0.7, 1024, 0),
]


def get_config(idx: int, **overrides) -> Config:
    cfg = CONFIGS[idx]
    return cfg.replace(**overrides) if overrides else cfg


def rng_for(cfg_idx: int, tag: int, layer: int = 0, seq: int = 0, head: int = 0):
    return np.random.default_rng([1000 + cfg_idx, tag, layer, seq, head])


def to_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    """Store ``x`` in the working dtype; returns float32 holding those values."""
    x32 = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "fp32":
        return x32
    if dtype == "bf16":
        import torch

        t = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float32)
        return t.numpy()
    raise ValueError(f"unknown dtype {dtype!r}")


def _mixture(cfg: Config, layer: int, seq: int, head: int):
    d = cfg.head_dim
    means = rng_for(cfg.idx, TAG_MIX_MEANS, layer, seq, head).standard_normal(
        (cfg.n_components, d))
    if cfg.lognormal_weights:
        w = np.exp(rng_for(cfg.idx, TAG_MIX_WEIGHTS, layer, seq, head)
                   .standard_normal(cfg.n_components))
        w = w / w.sum()
    else:
        w = None
    return means, w


def _draw_mixture(rng, means, weights, n, sigma):
    n_comp, d = means.shape
    if weights is None:
        comp = rng.integers(0, n_comp, size=n)
    else:
        comp = rng.choice(n_comp, size=n, p=weights)
    x = means[comp] + sigma * rng.standard_normal((n, d))
    return x, comp


def head_keys(cfg: Config, layer: int, seq: int, head: int):
    """Prefill keys [n_keys, d] of one KV head and their mixture components."""
    means, w = _mixture(cfg, layer, seq, head)
    rng = rng_for(cfg.idx, TAG_KEYS, layer, seq, head)
    x, comp = _draw_mixture(rng, means, w, cfg.n_keys, cfg.key_sigma)
    return to_dtype(x, cfg.dtype), comp


def head_values(cfg: Config, layer: int, seq: int, head: int) -> np.ndarray:
    rng = rng_for(cfg.idx, TAG_VALUES, layer, seq, head)
    return to_dtype(rng.standard_normal((cfg.n_keys, cfg.head_dim)), cfg.dtype)


def init_indices(cfg: Config, layer: int, seq: int, head: int) -> np.ndarray:
    rng = rng_for(cfg.idx, TAG_INIT, layer, seq, head)
    return rng.choice(cfg.n_keys, size=cfg.n_clusters, replace=False).astype(np.int32)


def query_walk(cfg: Config, layer: int, seq: int, steps: Optional[int] = None):
    """Queries [steps, n_q_heads, d] and the jump indicator [steps] (bool)."""
    steps = cfg.steps if steps is None else steps
    rng = rng_for(cfg.idx, TAG_WALK, layer, seq, 0)
    hq, d = cfg.n_q_heads, cfg.head_dim
    q = np.empty((steps, hq, d), dtype=np.float64)
    jumps = np.zeros(steps, dtype=bool)
    cur = rng.standard_normal((hq, d))
    q[0] = cur
    for t in range(1, steps):
        u = rng.random()
        noise = rng.standard_normal((hq, d))
        if u < cfg.p_jump:
            cur = noise
            jumps[t] = True
        else:
            cur = cur + cfg.walk_sigma * noise
        q[t] = cur
    return to_dtype(q, cfg.dtype), jumps


def decode_kv(cfg: Config, layer: int, seq: int, head: int, steps: Optional[int] = None):
    """Decode-time keys/values [steps, d] of one KV head (long-output config)."""
    steps = cfg.steps if steps is None else steps
    means, w = _mixture(cfg, layer, seq, head)
    rng = rng_for(cfg.idx, TAG_DEC_KEYS, layer, seq, head)
    k, _ = _draw_mixture(rng, means, w, steps, cfg.key_sigma)
    v = rng_for(cfg.idx, TAG_DEC_VALUES, layer, seq, head).standard_normal(
        (steps, cfg.head_dim))
    return to_dtype(k, cfg.dtype), to_dtype(v, cfg.dtype)


def layer_inputs(cfg: Config, layer: int = 0, heads=None, seqs=None, threads: int = 1):
    """All prefill inputs of one layer.

    Returns dict with keys [B, H, N, d], values [B, H, N, d], init_idx
    [B, H, C] (int32), components [B, H, N] (int64) -- float32 arrays hold
    values exact in ``cfg.dtype``. ``threads`` > 1 draws the (sequence, head)
    streams on that many threads; every stream has its own generator, so the
    arrays are the same whatever the thread count.
    """
    seqs = range(cfg.batch) if seqs is None else seqs
    heads = range(cfg.n_kv_heads) if heads is None else heads
    seqs, heads = list(seqs), list(heads)
    B, H, N, d, C = len(seqs), len(heads), cfg.n_keys, cfg.head_dim, cfg.n_clusters
    keys = np.empty((B, H, N, d), np.float32)
    vals = np.empty((B, H, N, d), np.float32)
    init = np.empty((B, H, C), np.int32)
    comp = np.empty((B, H, N), np.int64)

    def one(job):
        bi, hi = job
        b, h = seqs[bi], heads[hi]
        keys[bi, hi], comp[bi, hi] = head_keys(cfg, layer, b, h)
        vals[bi, hi] = head_values(cfg, layer, b, h)
        init[bi, hi] = init_indices(cfg, layer, b, h)

    jobs = [(bi, hi) for bi in range(B) for hi in range(H)]
    if threads > 1 and len(jobs) > 1:
        import concurrent.futures as cf

        with cf.ThreadPoolExecutor(max_workers=min(threads, len(jobs))) as ex:
            list(ex.map(one, jobs))
    else:
        for job in jobs:
            one(job)
    return {"keys": keys, "values": vals, "init_idx": init, "components": comp}


def layer_queries(cfg: Config, layer: int = 0, steps: Optional[int] = None, seqs=None):
    """Query walks [steps, B, Hq, d] and jump flags [steps, B] of one layer."""
    seqs = range(cfg.batch) if seqs is None else seqs
    qs, js = [], []
    for b in seqs:
        q, j = query_walk(cfg, layer, b, steps)
        qs.append(q)
        js.append(j)
    return np.stack(qs, axis=1), np.stack(js, axis=1)


def layer_decode_kv(cfg: Config, layer: int = 0, steps: Optional[int] = None, seqs=None):
    """Decode keys/values [steps, B, H, d] of one layer (long-output config)."""
    seqs = range(cfg.batch) if seqs is None else seqs
    ks, vs = [], []
    for b in seqs:
        kh, vh = [], []
        for h in range(cfg.n_kv_heads):
            k, v = decode_kv(cfg, layer, b, h, steps)
            kh.append(k)
            vh.append(v)
        ks.append(np.stack(kh, axis=1))
        vs.append(np.stack(vh, axis=1))
    return np.stack(ks, axis=1), np.stack(vs, axis=1)


def retrieval_schedule(policy: str, steps: int) -> Optional[np.ndarray]:
    """When to retrieve, for the comparison policies: None for "boundary" (the
    boundary test decides), all steps for "per-token" (retrieval at every
    decoded token, as the methods the LouisKV note's "Motivation" section
    discusses do), every S-th step from step 0 for "stride:S" (the
    fixed-stride policy of the note's ablation table). Returns [steps] bool."""
    if policy == "boundary":
        return None
    if policy == "per-token":
        return np.ones(steps, dtype=bool)
    if policy.startswith("stride:"):
        s = int(policy.split(":", 1)[1])
        if s < 1:
            raise ValueError(f"stride must be >= 1 (got {s})")
        return np.arange(steps) % s == 0
    raise ValueError(f"unknown retrieval policy {policy!r}")


def page_labels(batch: int, n_kv_heads: int, n_keys: int, page: int) -> np.ndarray:
    """Page-granularity units (the note's ablation of fine-grained units against
    pages): key i of every head belongs to unit i // page. [B, H, N] int32."""
    if page < 1:
        raise ValueError(f"page size must be >= 1 (got {page})")
    return np.broadcast_to((np.arange(n_keys) // page).astype(np.int32),
                           (batch, n_kv_heads, n_keys)).copy()
