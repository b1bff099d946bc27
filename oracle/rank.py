"""Oracle speculative ranking: which cached positions to fetch in 16 bits.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What it follows:
  * [SpeCache] quick read, "how it works" (second mechanism) and §3 "prefetch
    and offload during decoding": the speculative token T'_{t+1} is attended
    against the low-bit copy C', and the indices of its top-k KV pairs become
    the set fetched for the next step.
  * [SpeCache] §7 Algorithm 3: the set is ArgTopK over the speculative row of the
    attention matrix A = Softmax(Q K^T) (Algorithm 2 uses the single row of the
    pre-decoding step).
  * [SpeCache] §2 "attention sparsity": a fetched pair is worth the share of
    attention it receives ("hit rate" = attention mass captured).

Readings where the pages are silent:
  * The logits carry the usual 1/sqrt(D) factor, exposed as `sm_scale`.
  * Grouped-query attention: query head hq reads KV head hq // G.  The set is
    per (batch, KV head); a position's rank is the attention mass that the G
    query heads of the rank row put on it, r(p) = log sum_g softmax_g(p),
    i.e. the hit rate a fetched row buys.  (With G = 1 this is the ordinary
    ArgTopK of that head's logits.)
  * Scores are taken against C' alone (the quick-read wording), independent of
    which 16-bit rows happen to be resident (rank_scores).  Algorithm 3 instead
    writes ArgTopK over the speculative row of A = MaskedSoftmax(Q_t K^T) with
    K = [K' ∪ K_κ, K_t]: the fetched 16-bit keys replace their low-bit rows and
    the step's own new keys join the softmax (rank_scores_mixed).  In that
    reading the new keys count in each head's normalization, but only the N
    cached positions are candidates (the new keys are on the device already).
  * Ties: the lower position wins; the set is returned in ascending order.
"""
from __future__ import annotations

import numpy as np


def _logsumexp(x: np.ndarray, axis: int) -> np.ndarray:
    m = np.max(x, axis=axis, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    return np.squeeze(m, axis=axis) + np.log(np.sum(np.exp(x - m), axis=axis))


def rank_scores(q16: np.ndarray, k_hat: np.ndarray, rank_row: int, sm_scale: float) -> np.ndarray:
    """r(p) for every slice.

    q16:   [B, Hq, T, D] queries (float16).
    k_hat: [B, Hkv, N, D] dequantized low-bit keys (float64).
    Returns r [B, Hkv, N] float64: log of the total attention probability the
    G query heads of row `rank_row` put on each position."""
    B, Hq, T, D = q16.shape
    Hkv = k_hat.shape[1]
    G = Hq // Hkv
    q = q16[:, :, rank_row, :].astype(np.float64).reshape(B, Hkv, G, D)
    logits = sm_scale * np.matmul(q, np.swapaxes(k_hat, -1, -2))        # [B, Hkv, G, N]
    logp = logits - _logsumexp(logits, axis=-1)[..., None]              # log softmax per head
    return _logsumexp(logp, axis=2)                                     # log sum over the G heads


def rank_scores_mixed(q16: np.ndarray, k_hat: np.ndarray, rank_row: int, sm_scale: float,
                      idx=None, k_sel=None, k_tail=None) -> np.ndarray:
    """r(p) from Algorithm 3's A_{1,:}: the rank row's masked softmax over the mixed keys.

    q16:    [B, Hq, T, D] queries (float16).
    k_hat:  [B, Hkv, N, D] dequantized low-bit keys (float64).
    idx:    [B, Hkv, k] fetched positions (or None), k_sel [B, Hkv, k, D] their 16-bit keys.
    k_tail: [B, Hkv, R, D] the step's new keys (or None); tail entry j is visible to
            row t iff j <= R - T + t.
    Returns r [B, Hkv, N] float64 over the cached positions."""
    B, Hq, T, D = q16.shape
    Hkv, N = k_hat.shape[1], k_hat.shape[2]
    G = Hq // Hkv
    keys = np.array(k_hat, dtype=np.float64, copy=True)
    if idx is not None:
        for b in range(B):
            for h in range(Hkv):
                keys[b, h, idx[b, h]] = k_sel[b, h].astype(np.float64)
    q = q16[:, :, rank_row, :].astype(np.float64).reshape(B, Hkv, G, D)
    logits = sm_scale * np.matmul(q, np.swapaxes(keys, -1, -2))          # [B, Hkv, G, N]
    full = logits
    if k_tail is not None and k_tail.shape[2] > 0:
        R = k_tail.shape[2]
        visible = R - T + rank_row + 1                                     # entries j <= R - T + t
        if visible > 0:
            kt = k_tail[:, :, :visible].astype(np.float64)
            full = np.concatenate([logits, sm_scale * np.matmul(q, np.swapaxes(kt, -1, -2))], axis=-1)
    logp = logits - _logsumexp(full, axis=-1)[..., None]
    return _logsumexp(logp, axis=2)


def topk_positions(r: np.ndarray, k: int) -> np.ndarray:
    """ArgTopK per slice: the k largest r, ties to the lower position, ascending.

    r: [B, Hkv, N]; returns [B, Hkv, k] int32."""
    B, Hkv, N = r.shape
    if not 0 <= k <= N:
        raise ValueError("k out of range")
    out = np.empty((B, Hkv, k), dtype=np.int32)
    pos = np.arange(N)
    for b in range(B):
        for h in range(Hkv):
            order = np.lexsort((pos, -r[b, h]))     # primary: r descending; then position
            out[b, h] = np.sort(order[:k])
    return out


def score_topk(q16, k_hat, rank_row: int, sm_scale: float, k: int):
    """(idx [B, Hkv, k] int32, r [B, Hkv, N] float64)."""
    r = rank_scores(q16, k_hat, rank_row, sm_scale)
    return topk_positions(r, k), r
