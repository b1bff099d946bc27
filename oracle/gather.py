"""Oracle prefetch: copy the selected 16-bit rows out of the full cache.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Follows [SpeCache] §7 Algorithm 3, Pre-fetch(C_κ): the κ rows of the 16-bit
cache held in CPU memory are brought to the GPU.  A byte copy.
"""
from __future__ import annotations

import numpy as np


def gather_rows(k16: np.ndarray, v16: np.ndarray, idx: np.ndarray):
    """k16, v16: [B, Hkv, N, D]; idx: [B, Hkv, k] -> (K_sel, V_sel) [B, Hkv, k, D]."""
    B, Hkv = idx.shape[:2]
    ks = np.stack([np.stack([k16[b, h, idx[b, h]] for h in range(Hkv)]) for b in range(B)])
    vs = np.stack([np.stack([v16[b, h, idx[b, h]] for h in range(Hkv)]) for b in range(B)])
    return ks, vs
