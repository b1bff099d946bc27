"""Oracle prefetch: copy the selected 16-bit rows out of the full cache.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Follows [SpeCache] §7 Algorithm 3, Pre-fetch(C_κ): the κ rows of the 16-bit
cache held in CPU memory are brought to the GPU.  A byte copy.

[SpeCache] §3 "prefetch and offload during decoding": after the attention the
rows of κ_{t+1} are prefetched while the used rows outside κ_{t+1} are
evicted, so a row in both κ_t and κ_{t+1} is already on the device and only
κ_{t+1} minus κ_t crosses the host link (resident_rows).
"""
from __future__ import annotations

import numpy as np


def gather_rows(k16: np.ndarray, v16: np.ndarray, idx: np.ndarray):
    """k16, v16: [B, Hkv, N, D]; idx: [B, Hkv, k] -> (K_sel, V_sel) [B, Hkv, k, D]."""
    B, Hkv = idx.shape[:2]
    ks = np.stack([np.stack([k16[b, h, idx[b, h]] for h in range(Hkv)]) for b in range(B)])
    vs = np.stack([np.stack([v16[b, h, idx[b, h]] for h in range(Hkv)]) for b in range(B)])
    return ks, vs


def resident_rows(idx: np.ndarray, idx_prev: np.ndarray) -> np.ndarray:
    """[B, Hkv, k] bool: row i of idx holds a position that idx_prev also holds (per slice),
    i.e. a row that need not be fetched again."""
    B, Hkv, k = idx.shape
    out = np.zeros((B, Hkv, k), dtype=bool)
    for b in range(B):
        for h in range(Hkv):
            prev = set(int(p) for p in idx_prev[b, h])
            out[b, h] = [int(p) in prev for p in idx[b, h]]
    return out
