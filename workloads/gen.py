"""Seeded input generators (numpy PCG64, one independent stream per slice).

Every (batch, KV head) slice draws from its own stream, keyed by
(seed, tag, b, h), so a test can regenerate any single slice of a large
workload without drawing the rest.  All draws are float32 and are rounded to
float16 (round-to-nearest-even) only at the end.

Per KV head h      (tag 1): outlier channel choice, or lognormal channel scales.
Per slice (b, h)   (tag 2): K [N, D], V [N, D], planted positions, planted unit direction
                            (zero on outlier channels, so that boosting the query along it
                            does not also inflate the logits of every other key).
Per query (b, hq)  (tag 3): Q [T, D]; the slice's planted direction times `peak` is added.
Per slice (b, h)   (tag 4): tail K/V [R, D] when a tail is requested.
Per step and query (tag 5): the queries of later decode steps (generate_step_queries): fresh
                     draws from the same distribution, the slice's planted direction added.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .configs import WorkloadConfig

_TAG_HEAD, _TAG_SLICE, _TAG_QUERY, _TAG_TAIL, _TAG_STEP_QUERY = 1, 2, 3, 4, 5


def _rng(seed: int, tag: int, *keys: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(seed), tag, *map(int, keys)]))


@dataclass
class SliceInputs:
    k: np.ndarray            # [N, D] float16
    v: np.ndarray            # [N, D] float16
    planted: np.ndarray      # [P] int64, ascending (empty without a peak)
    direction: np.ndarray    # [D] float32 unit vector (zeros without a peak)


def _channel_scales(cfg: WorkloadConfig, h: int, seed: int) -> np.ndarray:
    rng = _rng(seed, _TAG_HEAD, h)
    scales = np.ones(cfg.head_dim, dtype=np.float32)
    if cfg.lognormal_keys:
        scales = np.exp(rng.standard_normal(cfg.head_dim, dtype=np.float32)).astype(np.float32)
    elif cfg.n_outlier > 0:
        ch = rng.choice(cfg.head_dim, size=cfg.n_outlier, replace=False)
        scales[ch] = np.float32(cfg.outlier_scale)
    return scales


def generate_slice(cfg: WorkloadConfig, b: int, h: int, seed: int | None = None) -> SliceInputs:
    seed = cfg.seed if seed is None else seed
    n, d = cfg.seq_len, cfg.head_dim
    scales = _channel_scales(cfg, h, seed)
    rng = _rng(seed, _TAG_SLICE, b, h)
    k = rng.standard_normal((n, d), dtype=np.float32)
    k *= scales[None, :]
    v = rng.standard_normal((n, d), dtype=np.float32)
    planted = np.zeros(0, dtype=np.int64)
    u = np.zeros(d, dtype=np.float32)
    if cfg.n_planted > 0:
        planted = np.sort(rng.choice(n, size=cfg.n_planted, replace=False)).astype(np.int64)
        u = rng.standard_normal(d, dtype=np.float32)
        u[scales != 1] = 0          # keep the planted direction off the outlier channels
        u /= np.float32(np.linalg.norm(u))
        k[planted] = np.float32(np.sqrt(d)) * u[None, :]
    return SliceInputs(k=k.astype(np.float16), v=v.astype(np.float16), planted=planted, direction=u)


def planted_positions(cfg: WorkloadConfig, b: int, h: int, seed: int | None = None) -> np.ndarray:
    return generate_slice(cfg, b, h, seed).planted


def generate_query(cfg: WorkloadConfig, b: int, hq: int, direction: np.ndarray | None = None,
                   seed: int | None = None) -> np.ndarray:
    """Q rows [T, D] float16 of query head hq in batch b."""
    seed = cfg.seed if seed is None else seed
    rng = _rng(seed, _TAG_QUERY, b, hq)
    q = rng.standard_normal((cfg.n_tokens, cfg.head_dim), dtype=np.float32)
    if cfg.peak is not None:
        if direction is None:
            direction = generate_slice(cfg, b, hq // cfg.gqa, seed).direction
        q += np.float32(cfg.peak) * direction[None, :]
    return q.astype(np.float16)


def generate_step_queries(cfg: WorkloadConfig, n_steps: int, seed: int | None = None) -> np.ndarray:
    """Queries of n_steps decode steps, [n_steps, B, Hq, T, D] float16: every step draws new
    N(0,1) queries, plus `peak` times the slice's planted direction as in generate_query --
    the planted positions stay relevant to every step, the rest of each step's top-k set is
    its own."""
    seed = cfg.seed if seed is None else seed
    B, Hq, T, D, G = cfg.batch, cfg.n_q_heads, cfg.n_tokens, cfg.head_dim, cfg.gqa
    out = np.zeros((n_steps, B, Hq, T, D), dtype=np.float16)
    dirs = {}
    for b in range(B):
        for h in range(cfg.n_kv_heads):
            dirs[b, h] = generate_slice(cfg, b, h, seed).direction if cfg.peak is not None else None
    for s in range(n_steps):
        for b in range(B):
            for hq in range(Hq):
                rng = _rng(seed, _TAG_STEP_QUERY, s, b, hq)
                q = rng.standard_normal((T, D), dtype=np.float32)
                if cfg.peak is not None:
                    q += np.float32(cfg.peak) * dirs[b, hq // G][None, :]
                out[s, b, hq] = q.astype(np.float16)
    return out


def generate_tail(cfg: WorkloadConfig, b: int, h: int, seed: int | None = None):
    seed = cfg.seed if seed is None else seed
    rng = _rng(seed, _TAG_TAIL, b, h)
    r, d = cfg.tail_len, cfg.head_dim
    kt = rng.standard_normal((r, d), dtype=np.float32)
    vt = rng.standard_normal((r, d), dtype=np.float32)
    return kt.astype(np.float16), vt.astype(np.float16)


def generate_all(cfg: WorkloadConfig, seed: int | None = None, slices=None):
    """Full tensors: K, V [B, Hkv, N, D], Q [B, Hq, T, D] (float16), planted [B, Hkv, P],
    and tail K/V [B, Hkv, R, D] (None when tail_len == 0).

    `slices`, if given, is an iterable of (b, h) pairs; only those slices are
    drawn (the others stay zero) -- used to check sampled slices of large
    workloads against the oracle."""
    seed = cfg.seed if seed is None else seed
    B, Hkv, Hq, N, D, T = cfg.batch, cfg.n_kv_heads, cfg.n_q_heads, cfg.seq_len, cfg.head_dim, cfg.n_tokens
    G = cfg.gqa
    K = np.zeros((B, Hkv, N, D), dtype=np.float16)
    V = np.zeros((B, Hkv, N, D), dtype=np.float16)
    Q = np.zeros((B, Hq, T, D), dtype=np.float16)
    planted = np.zeros((B, Hkv, cfg.n_planted), dtype=np.int64)
    want = None if slices is None else set((int(b), int(h)) for b, h in slices)
    for b in range(B):
        for h in range(Hkv):
            if want is not None and (b, h) not in want:
                continue
            s = generate_slice(cfg, b, h, seed)
            K[b, h], V[b, h], planted[b, h] = s.k, s.v, s.planted
            for g in range(G):
                Q[b, h * G + g] = generate_query(cfg, b, h * G + g, s.direction, seed)
    KT = VT = None
    if cfg.tail_len > 0:
        KT = np.zeros((B, Hkv, cfg.tail_len, D), dtype=np.float16)
        VT = np.zeros_like(KT)
        for b in range(B):
            for h in range(Hkv):
                if want is not None and (b, h) not in want:
                    continue
                KT[b, h], VT[b, h] = generate_tail(cfg, b, h, seed)
    return K, V, Q, planted, KT, VT
