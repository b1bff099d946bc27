"""GPU parity of the decode-time cache update (SpeCache summary §3 "decoding",
Algorithm 3: C' = [C', C'_t], C = [C, Offload(C_t)]) and of caches laid out
with spare capacity.

Bars: codes and float16 metadata bit-exact against the oracle's quantization
of the whole sequence; outputs of a cache with spare capacity bitwise equal to
those of a tight cache holding the same data; offloaded rows byte-exact and
nothing else written; a decode loop with a 16-bit residual window within the
attention tolerance of the oracle at every step.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from decode_attention_bit_kivi_amd import (
    quantize_pack, quantize_append, offload_fp16, score_topk, gather_fp16, decode_attn, decode_step,
)
from tests.layout import unpack_keys, unpack_values
from workloads import get_config, generate_all

pytestmark = pytest.mark.gpu

ATTN_TOL = 2e-3


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def _np(t):
    return t.cpu().numpy()


def _codes(cache, N):
    """Codes and metadata of positions [0, N) of a (possibly larger) cache."""
    kc, kz, ks = unpack_keys(_np(cache.k_codes), _np(cache.k_meta), cache.bits)
    vc, vz, vs = unpack_values(_np(cache.v_codes), _np(cache.v_meta), cache.v_bits or cache.bits)
    nb = N // cache.group
    return (kc[:, :, :N], kz[:, :, :nb], ks[:, :, :nb], vc[:, :, :N], vz[:, :, :N], vs[:, :, :N])


def _with_room(x, cap):
    out = np.zeros(x.shape[:2] + (cap,) + x.shape[3:], dtype=x.dtype)
    out[:, :, : x.shape[2]] = x
    return out


def test_cache_with_spare_capacity_gives_the_same_results():
    cfg = get_config("llama8k").with_(seq_len=4096, batch=2, seed=3)
    K, V, Q, _, _, _ = generate_all(cfg)
    N, cap = cfg.seq_len, 6144
    tight = quantize_pack(_dev(K), _dev(V), cfg.bits)
    roomy = quantize_pack(_dev(_with_room(K, cap)), _dev(_with_room(V, cap)), cfg.bits, seq_len=N)
    assert roomy.capacity == cap and roomy.seq_len == N
    for a, b in zip(_codes(tight, N), _codes(roomy, N)):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))
    q = _dev(Q)
    i_t, i_r = score_topk(q, tight, cfg.top_k), score_topk(q, roomy, cfg.top_k)
    assert torch.equal(i_t, i_r)
    hk, hv = torch.from_numpy(K).pin_memory(), torch.from_numpy(V).pin_memory()
    hk_r = torch.from_numpy(_with_room(K, cap)).pin_memory()
    hv_r = torch.from_numpy(_with_room(V, cap)).pin_memory()
    ks, vs = gather_fp16(i_t, hk, hv)
    ks_r, vs_r = gather_fp16(i_t, hk_r, hv_r, seq_len=N)
    assert torch.equal(ks.view(torch.int16), ks_r.view(torch.int16))
    o_t = decode_attn(q, tight, i_t, ks, vs)
    o_r = decode_attn(q, roomy, i_t, ks_r, vs_r)
    f_t, n_t = decode_step(q, tight, cfg.top_k, idx=i_t, k_sel=ks, v_sel=vs)
    f_r, n_r = decode_step(q, roomy, cfg.top_k, idx=i_t, k_sel=ks, v_sel=vs)
    torch.cuda.synchronize()
    assert torch.equal(o_t.view(torch.int16), o_r.view(torch.int16))
    assert torch.equal(f_t.view(torch.int16), f_r.view(torch.int16)) and torch.equal(n_t, n_r)


@pytest.mark.parametrize("bits,group", [(1, 32), (2, 32), (1, 64)])
def test_append_equals_quantizing_the_whole_sequence(bits, group):
    cfg = get_config("llama8k").with_(seq_len=2048 + 3 * group, bits=bits, seed=5)
    K, V, Q, _, _, _ = generate_all(cfg)
    N0, cap = 2048, 4096
    cache = quantize_pack(_dev(_with_room(K[:, :, :N0], cap)), _dev(_with_room(V[:, :, :N0], cap)), bits,
                          seq_len=N0, group=group)
    quantize_append(cache, _dev(K[:, :, N0:N0 + 2 * group]), _dev(V[:, :, N0:N0 + 2 * group]))
    quantize_append(cache, _dev(K[:, :, N0 + 2 * group:]), _dev(V[:, :, N0 + 2 * group:]))
    torch.cuda.synchronize()
    N = cfg.seq_len
    assert cache.seq_len == N
    kc, kz, ks = oracle.quantize_keys(K, bits, group)
    vc, vz, vs = oracle.quantize_values(V, bits, group)
    got = _codes(cache, N)
    for g, w in zip(got, (kc, kz, ks, vc, vz, vs)):
        assert np.array_equal(g.view(np.uint8) if g.dtype != np.float16 else g.view(np.uint16),
                              w.view(np.uint8) if w.dtype != np.float16 else w.view(np.uint16))
    whole = quantize_pack(_dev(K), _dev(V), bits, group=group)
    q = _dev(Q)
    o_a = decode_attn(q, cache)
    o_w = decode_attn(q, whole)
    torch.cuda.synchronize()
    assert torch.equal(o_a.view(torch.int16), o_w.view(torch.int16))


@pytest.mark.parametrize("device_dst", [False, True])
def test_offload_writes_exactly_the_new_rows(device_dst):
    B, H, cap, D = 2, 3, 128, 64
    rng = np.random.default_rng(8)
    new_k = rng.standard_normal((B, H, 5, D)).astype(np.float16)
    new_v = rng.standard_normal((B, H, 5, D)).astype(np.float16)
    if device_dst:
        hk = torch.zeros((B, H, cap, D), dtype=torch.float16, device="cuda")
        hv = torch.zeros_like(hk)
    else:
        hk = torch.zeros((B, H, cap, D), dtype=torch.float16).pin_memory()
        hv = torch.zeros_like(hk).pin_memory()
    offload_fp16(_dev(new_k), _dev(new_v), hk, hv, pos0=100)
    torch.cuda.synchronize()
    for got, new in ((hk.cpu().numpy(), new_k), (hv.cpu().numpy(), new_v)):
        assert np.array_equal(got[:, :, 100:105].view(np.uint16), new.view(np.uint16))
        rest = np.concatenate([got[:, :, :100], got[:, :, 105:]], axis=2)
        assert not rest.any()


def test_decode_loop_with_residual_window():
    """40 decode steps of one layer: each step's new K/V joins a 16-bit residual window (the
    attention's tail); once the window holds 32 + 8 tokens its oldest 32 are quantized into
    C' and offloaded to the pinned 16-bit cache.  Every step ranks, fetches from the host
    cache and attends; the output follows the oracle over the whole history."""
    cfg = get_config("tiny").with_(n_tokens=1, seq_len=256, seed=11)
    K0, V0, _, _, _, _ = generate_all(cfg)
    B, H, Hq, D, bits, k = cfg.batch, cfg.n_kv_heads, cfg.n_q_heads, cfg.head_dim, cfg.bits, cfg.top_k
    cap = 512
    rng = np.random.default_rng(12)
    hist_k = [K0[:, :, i] for i in range(cfg.seq_len)]       # the 16-bit history, one row per position
    hist_v = [V0[:, :, i] for i in range(cfg.seq_len)]
    host_k = torch.from_numpy(_with_room(K0, cap)).pin_memory()
    host_v = torch.from_numpy(_with_room(V0, cap)).pin_memory()
    cache = quantize_pack(host_k.cuda(), host_v.cuda(), bits, seq_len=cfg.seq_len)
    win_k, win_v = [], []
    for step in range(40):
        nk = rng.standard_normal((B, H, D)).astype(np.float16)
        nv = rng.standard_normal((B, H, D)).astype(np.float16)
        win_k.append(nk)
        win_v.append(nv)
        hist_k.append(nk)
        hist_v.append(nv)
        if len(win_k) == 40:
            blk_k, blk_v = np.stack(win_k[:32], axis=2), np.stack(win_v[:32], axis=2)
            pos = cache.seq_len
            offload_fp16(_dev(blk_k), _dev(blk_v), host_k, host_v, pos0=pos)
            quantize_append(cache, _dev(blk_k), _dev(blk_v))
            win_k, win_v = win_k[32:], win_v[32:]
        q = rng.standard_normal((B, Hq, 1, D)).astype(np.float16)
        tk, tv = np.stack(win_k, axis=2), np.stack(win_v, axis=2)
        N = cache.seq_len
        idx = score_topk(_dev(q), cache, k, rank_row=0)
        ks, vs = gather_fp16(idx, host_k, host_v, bits, seq_len=N)
        out = decode_attn(_dev(q), cache, idx, ks, vs, _dev(tk), _dev(tv))
        torch.cuda.synchronize()
        Kh = np.stack(hist_k[:N], axis=2)
        Vh = np.stack(hist_v[:N], axis=2)
        kc, kz, kss = oracle.quantize_keys(Kh, bits)
        vc, vz, vss = oracle.quantize_values(Vh, bits)
        kh, vh = oracle.dequantize_keys(kc, kz, kss), oracle.dequantize_values(vc, vz, vss)
        i = _np(idx)
        rk, rv = oracle.gather_rows(Kh, Vh, i)
        ref = oracle.mixed_attention(q, kh, vh, i, rk, rv, tk, tv, sm_scale=cfg.sm_scale)
        err = float(np.max(np.abs(_np(out).astype(np.float64) - ref)) / np.max(np.abs(ref)))
        assert err <= ATTN_TOL, (step, err)
    assert cache.seq_len == cfg.seq_len + 32
