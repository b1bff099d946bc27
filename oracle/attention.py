"""Oracle mixed attention over the low-bit cache with 16-bit replacements.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What it follows:
  * [SpeCache] quick read, "how it works" (third mechanism) and §3 "decoding":
    O = Attn([T_t, T'_{t+1}], C' ∪ C_κ), where C' ∪ C_κ means the 16-bit pairs
    C_κ take the place of their low-bit counterparts C'_κ in this computation.
  * [SpeCache] §7 Algorithm 3: K = [K' ∪ K_κ, K_t], V = [V' ∪ V_κ, V_t] and
    A = MaskedSoftmax(Q_t K^T); O = A V (the output projection is outside the path).

Readings where the pages are silent:
  * Logits carry the 1/sqrt(D) factor as `sm_scale`; query head hq reads KV head
    hq // G.
  * The optional 16-bit tail (the step's own new KV, the K_t of Algorithm 3) is
    visible to query row t at tail position j iff j <= R - T + t, so the real
    token T_t does not see the speculative token's entry.
"""
from __future__ import annotations

import numpy as np


def _mixed_keys_values(k_hat, v_hat, idx, k_sel, v_sel):
    kt = np.array(k_hat, dtype=np.float64, copy=True)
    vt = np.array(v_hat, dtype=np.float64, copy=True)
    if idx is not None and idx.shape[-1] > 0:
        B, Hkv = kt.shape[:2]
        for b in range(B):
            for h in range(Hkv):
                kt[b, h, idx[b, h]] = k_sel[b, h].astype(np.float64)
                vt[b, h, idx[b, h]] = v_sel[b, h].astype(np.float64)
    return kt, vt


def attention_probs(q16, k_hat, v_hat, idx=None, k_sel=None, v_sel=None,
                    k_tail=None, v_tail=None, sm_scale: float = 1.0):
    """(P, Kmix, Vmix): softmax probabilities P [B, Hq, T, N + R] (float64) and the
    mixed keys / values [B, Hkv, N + R, D] they weight."""
    B, Hq, T, D = q16.shape
    Hkv = k_hat.shape[1]
    G = Hq // Hkv
    kt, vt = _mixed_keys_values(k_hat, v_hat, idx, k_sel, v_sel)
    R = 0
    if k_tail is not None and k_tail.shape[2] > 0:
        R = k_tail.shape[2]
        kt = np.concatenate([kt, k_tail.astype(np.float64)], axis=2)
        vt = np.concatenate([vt, v_tail.astype(np.float64)], axis=2)
    N = k_hat.shape[2]
    q = q16.astype(np.float64).reshape(B, Hkv, G, T, D)
    logits = sm_scale * np.einsum("bhgtd,bhnd->bhgtn", q, kt)
    if R > 0:
        j = np.arange(R)
        for t in range(T):
            hidden = j > (R - T + t)
            logits[:, :, :, t, N:][..., hidden] = -np.inf
    m = logits.max(axis=-1, keepdims=True)
    e = np.exp(logits - m)
    p = e / e.sum(axis=-1, keepdims=True)
    return p.reshape(B, Hq, T, N + R), kt, vt


def mixed_attention(q16, k_hat, v_hat, idx=None, k_sel=None, v_sel=None,
                    k_tail=None, v_tail=None, sm_scale: float = 1.0) -> np.ndarray:
    """O [B, Hq, T, D] float64 = softmax(sm_scale Q K_mix^T) V_mix."""
    B, Hq, T, D = q16.shape
    Hkv = k_hat.shape[1]
    G = Hq // Hkv
    p, kt, vt = attention_probs(q16, k_hat, v_hat, idx, k_sel, v_sel, k_tail, v_tail, sm_scale)
    p = p.reshape(B, Hkv, G, T, -1)
    o = np.einsum("bhgtn,bhnd->bhgtd", p, vt)
    return o.reshape(B, Hq, T, D)
