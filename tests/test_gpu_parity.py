"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bars (fixed before the kernels were written):
  * quantize_pack: codes and float16 zero-points / scales bit-exact;
  * score_topk: same count, unique, ascending; every position in the symmetric
    difference with the oracle's set has an oracle rank within 1e-5 of the k-th
    largest (ties go to the lower position);
  * gather_fp16: bitwise copy;
  * decode_attn: max |O_gpu - O_ref| / max |O_ref| <= 2e-3 (float16 output);
  * decode_step: O bitwise equal to decode_attn's on the same inputs, and the
    next selection held to score_topk's bar.
Small cases are checked in full; the large workloads run at full size in the
launch configuration the benchmark uses, with a few seeded slices filled and
checked against the oracle (the other slices are left zero).
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
from decode_attention_bit_kivi_amd import (
    quantize_pack, score_topk, gather_fp16, decode_attn, decode_step, GatherStream, ComputeStream,
    SpecacheError, gather_reuse, gather_fp16_missing, decode_attn_fp16,
)
from tests.layout import unpack_keys, unpack_values
from tests.parity_log import record
from workloads import get_config, generate_all

pytestmark = pytest.mark.gpu

ATTN_TOL = 2e-3
TIE_BAND = 1e-5


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def _np(t):
    return t.cpu().numpy()


def _sampled(cfg, n=4, seed=123):
    rng = np.random.default_rng(seed)
    allp = [(b, h) for b in range(cfg.batch) for h in range(cfg.n_kv_heads)]
    if len(allp) <= n:
        return allp
    pick = rng.choice(len(allp), size=n, replace=False)
    return [allp[i] for i in sorted(pick)]


def _reference_cache(K, V, bits):
    kc, kz, ks = oracle.quantize_keys(K, bits)
    vc, vz, vs = oracle.quantize_values(V, bits)
    return (kc, kz, ks, vc, vz, vs), oracle.dequantize_keys(kc, kz, ks), oracle.dequantize_values(vc, vz, vs)


def _assert_quantize_exact(cache, ref, bits, slices=None):
    kc, kz, ks, vc, vz, vs = ref
    gk, gkz, gks = unpack_keys(_np(cache.k_codes), _np(cache.k_meta), bits)
    gv, gvz, gvs = unpack_values(_np(cache.v_codes), _np(cache.v_meta), bits)
    sel = (slice(None),) if slices is None else (tuple(b for b, _ in slices), tuple(h for _, h in slices))
    pairs = [(gk, kc), (gv, vc)]
    for got, want in pairs:
        assert np.array_equal(got[sel], want[sel]), "codes differ"
    for got, want in ((gkz, kz), (gks, ks), (gvz, vz), (gvs, vs)):
        assert np.array_equal(got[sel].view(np.uint16), want[sel].view(np.uint16)), "metadata differs"


def _assert_topk(idx_gpu, r_ref, k, slices, what=""):
    """Same count, strictly ascending, and every position in the symmetric difference with the
    oracle's set within the tie band of the k-th largest oracle rank.  Records the widest
    distance from the k-th rank over the symmetric difference (0 when the sets are equal)."""
    widest, n_diff = 0.0, 0
    for (b, h) in slices:
        got = idx_gpu[b, h]
        assert len(got) == k and np.all(np.diff(got) > 0), "not strictly ascending"
        want = oracle.topk_positions(r_ref[b:b + 1, h:h + 1], k)[0, 0]
        kth = np.sort(r_ref[b, h])[::-1][k - 1]
        diff = np.setxor1d(got, want)
        n_diff += len(diff)
        dist = [abs(r_ref[b, h, p] - kth) for p in diff]
        widest = max([widest] + dist)
        bad = [p for p, d in zip(diff, dist) if d >= TIE_BAND]
        assert not bad, f"slice {(b, h)}: positions {bad[:8]} outside the tie band"
    record("topk_tie_distance", widest, TIE_BAND, f"{what} ({n_diff} positions differ over {len(slices)} slices)")


def _attn_err(o_gpu, o_ref):
    return float(np.max(np.abs(o_gpu.astype(np.float64) - o_ref)) / np.max(np.abs(o_ref)))


def _check_attn(o_gpu, o_ref, what=""):
    """max |O_gpu - O_ref| / max |O_ref| within ATTN_TOL; the measured error is recorded."""
    err = _attn_err(o_gpu, o_ref)
    record("attention_rel_err", err, ATTN_TOL, what)
    assert err <= ATTN_TOL, f"attention relative error {err:.3e} > {ATTN_TOL} {what}"


def _check_rank_keys(rk_gpu, r_ref, what=""):
    err = float(np.max(np.abs(rk_gpu - r_ref)))
    record("rank_key_abs_err", err, 1e-4, what)
    assert err < 1e-4, f"r(p) error {err:.3e} {what}"


# ---------------------------------------------------------------- quantize_pack

@pytest.mark.parametrize("name,over", [
    ("tiny", {}),
    ("tiny", dict(bits=2)),
    ("tiny", dict(head_dim=128, seq_len=96, batch=2)),
    ("llama8k", {}),
    ("llama8k", dict(bits=1, seed=1)),
    ("llama8k", dict(head_dim=64, seq_len=32, seed=2)),
])
def test_quantize_bit_exact(gpu, name, over):
    cfg = get_config(name).with_(**over)
    K, V, _, _, _, _ = generate_all(cfg)
    cache = quantize_pack(_dev(K), _dev(V), cfg.bits)
    torch.cuda.synchronize()
    ref, _, _ = _reference_cache(K, V, cfg.bits)
    _assert_quantize_exact(cache, ref, cfg.bits)


@pytest.mark.parametrize("bits,D", [(1, 128), (2, 128), (1, 64)])
def test_group_64(gpu, bits, D):
    """Quantization groups of 64 (keys: 64 tokens per channel, values: 64 channels per
    token): codes and metadata bit-exact, ranking and attention against the oracle."""
    cfg = get_config("llama8k").with_(bits=bits, head_dim=D, seq_len=4096 + 64, seed=8)
    K, V, Q, _, _, _ = generate_all(cfg)
    cache = quantize_pack(_dev(K), _dev(V), bits, group=64)
    kc, kz, ks = oracle.quantize_keys(K, bits, 64)
    vc, vz, vs = oracle.quantize_values(V, bits, 64)
    gk, gkz, gks = unpack_keys(_np(cache.k_codes), _np(cache.k_meta), bits)
    gv, gvz, gvs = unpack_values(_np(cache.v_codes), _np(cache.v_meta), bits)
    assert np.array_equal(gk, kc) and np.array_equal(gv, vc)
    for got, want in ((gkz, kz), (gks, ks), (gvz, vz), (gvs, vs)):
        assert np.array_equal(got.view(np.uint16), want.view(np.uint16))
    kh = oracle.dequantize_keys(kc, kz, ks, 64)
    vh = oracle.dequantize_values(vc, vz, vs, 64)
    rng = np.random.default_rng(4)
    idx = _random_idx(rng, cfg.batch, cfg.n_kv_heads, cfg.seq_len, cfg.top_k)
    sk, sv = oracle.gather_rows(K, V, idx)
    rk = torch.empty((cfg.batch, cfg.n_kv_heads, cfg.seq_len), dtype=torch.float32, device="cuda")
    sel = score_topk(_dev(Q), cache, cfg.top_k, rank_key_out=rk)
    o = decode_attn(_dev(Q), cache, _dev(idx), _dev(sk), _dev(sv))
    of, nxt = decode_step(_dev(Q), cache, cfg.top_k, idx=_dev(idx), k_sel=_dev(sk), v_sel=_dev(sv))
    torch.cuda.synchronize()
    r_ref = oracle.rank_scores(Q, kh, 1, cfg.sm_scale)
    _check_rank_keys(_np(rk), r_ref)
    slices = [(0, h) for h in range(cfg.n_kv_heads)]
    _assert_topk(_np(sel), r_ref, cfg.top_k, slices)
    _assert_topk(_np(nxt), r_ref, cfg.top_k, slices)
    ref = oracle.mixed_attention(Q, kh, vh, idx, sk, sv, sm_scale=cfg.sm_scale)
    _check_attn(_np(o), ref)
    assert torch.equal(of.view(torch.int16), o.view(torch.int16))


@pytest.mark.parametrize("kbits,vbits", [(2, 1), (1, 2)])
def test_mixed_key_value_bits(gpu, kbits, vbits):
    """Keys and values with different code widths: codes bit-exact, attention and the fused
    step against the oracle with each half dequantized at its own width."""
    cfg = get_config("llama8k").with_(bits=kbits, seed=7, seq_len=4096 + 64)
    K, V, Q, _, _, _ = generate_all(cfg)
    cache = quantize_pack(_dev(K), _dev(V), kbits, v_bits=vbits)
    torch.cuda.synchronize()
    kc, kz, ks = oracle.quantize_keys(K, kbits)
    vc, vz, vs = oracle.quantize_values(V, vbits)
    gk, gkz, gks = unpack_keys(_np(cache.k_codes), _np(cache.k_meta), kbits)
    gv, gvz, gvs = unpack_values(_np(cache.v_codes), _np(cache.v_meta), vbits)
    assert np.array_equal(gk, kc) and np.array_equal(gv, vc)
    for got, want in ((gkz, kz), (gks, ks), (gvz, vz), (gvs, vs)):
        assert np.array_equal(got.view(np.uint16), want.view(np.uint16))
    kh, vh = oracle.dequantize_keys(kc, kz, ks), oracle.dequantize_values(vc, vz, vs)
    rng = np.random.default_rng(3)
    idx = _random_idx(rng, cfg.batch, cfg.n_kv_heads, cfg.seq_len, cfg.top_k)
    sk, sv = oracle.gather_rows(K, V, idx)
    o = decode_attn(_dev(Q), cache, _dev(idx), _dev(sk), _dev(sv))
    of, nxt = decode_step(_dev(Q), cache, cfg.top_k, idx=_dev(idx), k_sel=_dev(sk), v_sel=_dev(sv))
    torch.cuda.synchronize()
    ref = oracle.mixed_attention(Q, kh, vh, idx, sk, sv, sm_scale=cfg.sm_scale)
    _check_attn(_np(o), ref)
    assert torch.equal(of.view(torch.int16), o.view(torch.int16))
    r_ref = oracle.rank_scores(Q, kh, 1, cfg.sm_scale)
    _assert_topk(_np(nxt), r_ref, cfg.top_k, [(0, h) for h in range(cfg.n_kv_heads)])


@pytest.mark.parametrize("bits", [1, 2])
def test_quantize_adversarial_values(gpu, bits):
    """Exact ties, constant groups, signed zeros, float16 extremes and subnormals."""
    rng = np.random.default_rng(77 + bits)
    specials = np.array([0.0, -0.0, 1.0, -1.0, 0.5, -0.5, 0.25, 65504.0, -65504.0, 6e-8, -6e-8,
                         1e-4, 3.0, 1.5, 2.0, -2.0], dtype=np.float16)
    B, H, N, D = 2, 2, 256, 64
    K = rng.choice(specials, size=(B, H, N, D))
    V = rng.choice(specials, size=(B, H, N, D))
    K[0, 0, :32] = np.float16(0.75)                                   # constant key groups
    V[0, 1, 5] = np.float16(-3.0)                                     # constant value groups
    t = rng.integers(0, 7, size=(N, D)) / 2                           # exact half-way 2-bit codes
    K[1, 1] = (np.float16(-1.0) + np.float16(0.25) * t).astype(np.float16)
    K[1, 1, ::32] = np.float16(-1.0)
    K[1, 1, 1::32] = np.float16(-0.25)
    cache = quantize_pack(_dev(K), _dev(V), bits)
    torch.cuda.synchronize()
    ref, _, _ = _reference_cache(K, V, bits)
    _assert_quantize_exact(cache, ref, bits)


@pytest.mark.filterwarnings("ignore:invalid value encountered")  # the oracle's dequantized 0 * inf
@pytest.mark.parametrize("bits", [1, 2])
def test_quantize_infinite_scale_groups(gpu, bits):
    """Groups holding +inf have an infinite scale: the kernels then decide the codes by the
    correctly rounded division instead of the division-free comparisons (every code 0, the
    zero-point +inf), as the oracle's division does; the other groups are unaffected."""
    rng = np.random.default_rng(91 + bits)
    B, H, N, D = 1, 2, 128, 64
    K = rng.standard_normal((B, H, N, D)).astype(np.float16)
    V = rng.standard_normal((B, H, N, D)).astype(np.float16)
    K[0, 0, 5, 3] = np.float16(np.inf)      # key group (tokens 0-31, channel 3)
    K[0, 1, 70, 10] = np.float16(np.inf)
    V[0, 0, 9, 40] = np.float16(np.inf)     # value group (token 9, channels 32-63)
    V[0, 1, 100, 0] = np.float16(np.inf)
    cache = quantize_pack(_dev(K), _dev(V), bits)
    torch.cuda.synchronize()
    ref, _, _ = _reference_cache(K, V, bits)
    _assert_quantize_exact(cache, ref, bits)


FULL_SIZE_SLICES = 4   # seeded (batch, KV head) slices filled and checked per full-size workload


@pytest.mark.parametrize("name", ["mistral32k", "long128k", "layers32"])
def test_quantize_full_size_sampled(gpu, name):
    cfg = get_config(name)
    sl = _sampled(cfg, FULL_SIZE_SLICES)
    K, V, _, _, _, _ = generate_all(cfg, slices=sl)
    cache = quantize_pack(_dev(K), _dev(V), cfg.bits)
    torch.cuda.synchronize()
    for (b, h) in sl:
        ref, _, _ = _reference_cache(K[b:b + 1, h:h + 1], V[b:b + 1, h:h + 1], cfg.bits)
        sub = type(cache)(*(t[b:b + 1, h:h + 1] for t in (cache.k_codes, cache.k_meta, cache.v_codes, cache.v_meta)),
                          1, 1, cfg.seq_len, cfg.head_dim, cfg.bits)
        _assert_quantize_exact(sub, ref, cfg.bits)


# ---------------------------------------------------------------- score_topk

@pytest.mark.parametrize("name,over", [
    ("tiny", {}),
    ("tiny", dict(bits=2, seed=1, top_k=1)),
    ("tiny", dict(seq_len=96, top_k=96)),                   # k = N
    ("llama8k", {}),
    ("llama8k", dict(bits=1, seed=2)),
    ("llama8k", dict(seq_len=8192 + 160, seed=3)),           # ragged last split
    ("llama8k", dict(n_tokens=1)),                           # pre-decoding: one token, row 0
])
def test_score_topk_matches_oracle(gpu, name, over):
    cfg = get_config(name).with_(**over)
    K, V, Q, _, _, _ = generate_all(cfg)
    cache = quantize_pack(_dev(K), _dev(V), cfg.bits)
    row = 1 if cfg.n_tokens == 2 else 0
    rk = torch.empty((cfg.batch, cfg.n_kv_heads, cfg.seq_len), dtype=torch.float32, device="cuda")
    idx = score_topk(_dev(Q), cache, cfg.top_k, rank_row=row, rank_key_out=rk)
    torch.cuda.synchronize()
    _, kh, _ = _reference_cache(K, V, cfg.bits)
    r_ref = oracle.rank_scores(Q, kh, row, cfg.sm_scale)
    slices = [(b, h) for b in range(cfg.batch) for h in range(cfg.n_kv_heads)]
    _assert_topk(_np(idx), r_ref, cfg.top_k, slices)
    _check_rank_keys(_np(rk), r_ref)


@pytest.mark.parametrize("qscale", [0.0, 1e-3, 1.0])
def test_score_topk_crowded_and_tied_ranks(gpu, qscale):
    """qscale 0: every rank equal (one coarse bin holds all 20480 positions, more than the
    selection keeps in LDS): the k lowest positions.  1e-3: the ranks differ by less than a
    coarse bin, the threshold bin is crowded with distinct keys.  1: the ordinary spread."""
    cfg = get_config("llama8k").with_(seq_len=20480, top_k=300, seed=3)
    K, V, Q, _, _, _ = generate_all(cfg)
    Q = (Q.astype(np.float32) * qscale).astype(np.float16)
    cache = quantize_pack(_dev(K), _dev(V), cfg.bits)
    rk = torch.empty((cfg.batch, cfg.n_kv_heads, cfg.seq_len), dtype=torch.float32, device="cuda")
    idx = _np(score_topk(_dev(Q), cache, cfg.top_k, rank_key_out=rk))
    _, kh, _ = _reference_cache(K, V, cfg.bits)
    r_ref = oracle.rank_scores(Q, kh, 1, cfg.sm_scale)
    slices = [(0, h) for h in range(cfg.n_kv_heads)]
    if qscale == 0.0:
        assert np.array_equal(idx, np.broadcast_to(np.arange(cfg.top_k, dtype=np.int32), idx.shape))
    _assert_topk(idx, r_ref, cfg.top_k, slices)
    _check_rank_keys(_np(rk), r_ref)


@pytest.mark.parametrize("seq_len", [32768, 32768 + 64])
def test_selection_same_with_and_without_key_output(gpu, seq_len):
    """r(p) is written only when the caller asks for it (up to 32768 positions the selection
    forms the keys itself, beyond that a separate pass writes them to workspace): the selected
    sets do not depend on it, for score_topk and for the fused step (each against itself: the
    two compute the logits in different kernels)."""
    cfg = get_config("llama8k").with_(seq_len=seq_len, top_k=328, bits=1, seed=5)
    K, V, Q, _, _, _ = generate_all(cfg)
    cache = quantize_pack(_dev(K), _dev(V), cfg.bits)
    q = _dev(Q)
    rk = torch.empty((cfg.batch, cfg.n_kv_heads, cfg.seq_len), dtype=torch.float32, device="cuda")
    a = score_topk(q, cache, cfg.top_k, rank_key_out=rk)
    b = score_topk(q, cache, cfg.top_k)
    rk2 = torch.empty_like(rk)
    _, na = decode_step(q, cache, cfg.top_k, rank_key_out=rk2)
    _, nb = decode_step(q, cache, cfg.top_k)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(na, nb)


@pytest.mark.parametrize("k,qscale", [(1, 1.0), (300, 1.0), (1500, 1.0), (3000, 1.0), (300, 0.0), (300, 1e-3)])
def test_topk_long_slices_grouped_and_swept(gpu, k, qscale):
    """Slices longer than one selection workgroup holds (40960 + 96 positions): rank_keys writes
    r(p) and its maximum over every 16 positions, and the selection reads only the groups whose
    maximum reaches the threshold bin; when more than 2048 groups do (k = 3000, every rank equal,
    a bin crowded with distinct keys) it sweeps over every key instead.  score_topk and the fused
    step's next selection against the oracle; with every rank equal, the k lowest positions."""
    cfg = get_config("llama8k").with_(seq_len=40960 + 96, top_k=k, seed=7)
    K, V, Q, _, _, _ = generate_all(cfg)
    Q = (Q.astype(np.float32) * qscale).astype(np.float16)
    cache = quantize_pack(_dev(K), _dev(V), cfg.bits)
    q = _dev(Q)
    rk = torch.empty((cfg.batch, cfg.n_kv_heads, cfg.seq_len), dtype=torch.float32, device="cuda")
    a = _np(score_topk(q, cache, k, rank_key_out=rk))
    b = _np(score_topk(q, cache, k))
    _, nxt = decode_step(q, cache, k)
    nxt = _np(nxt)
    _, kh, _ = _reference_cache(K, V, cfg.bits)
    r_ref = oracle.rank_scores(Q, kh, 1, cfg.sm_scale)
    slices = [(0, h) for h in range(cfg.n_kv_heads)]
    what = f"N {cfg.seq_len} k {k} q x{qscale}"
    assert np.array_equal(a, b), "the selection depends on the key output"
    _assert_topk(a, r_ref, k, slices, f"score_topk {what}")
    _assert_topk(nxt, r_ref, k, slices, f"decode_step {what}")
    _check_rank_keys(_np(rk), r_ref, what)
    if qscale == 0.0:
        lowest = np.broadcast_to(np.arange(k, dtype=np.int32), a.shape)
        assert np.array_equal(a, lowest) and np.array_equal(nxt, lowest)


def test_topk_sweeps_over_two_chunks(gpu):
    """A crowded threshold bin on a slice longer than one compaction chunk (131072 positions):
    the sweeps mark and compact the selected positions chunk by chunk, the second chunk's bitmaps
    cleared by other threads than the ones that read the first's.  The selected positions fall in
    both chunks; score_topk and the fused step's next selection against the oracle."""
    k = 3000
    cfg = get_config("llama8k").with_(seq_len=131072 + 8192 + 96, top_k=k, seed=11)
    K, V, Q, _, _, _ = generate_all(cfg)
    Q = (Q.astype(np.float32) * 1e-3).astype(np.float16)
    cache = quantize_pack(_dev(K), _dev(V), cfg.bits)
    q = _dev(Q)
    a = _np(score_topk(q, cache, k))
    _, nxt = decode_step(q, cache, k)
    nxt = _np(nxt)
    _, kh, _ = _reference_cache(K, V, cfg.bits)
    r_ref = oracle.rank_scores(Q, kh, 1, cfg.sm_scale)
    slices = [(0, h) for h in range(cfg.n_kv_heads)]
    assert (a >= 131072).any() and (a < 131072).any(), "the selection should span both chunks"
    _assert_topk(a, r_ref, k, slices, "score_topk two chunks")
    _assert_topk(nxt, r_ref, k, slices, "decode_step two chunks")


@pytest.mark.parametrize("name,rank_row", [("mistral32k", 1), ("long128k", 1), ("layers32", 1),
                                           ("mistral32k", 0)])   # row 0 of two: the serial comparator's ranking
def test_score_topk_full_size_sampled(gpu, name, rank_row):
    cfg = get_config(name)
    sl = _sampled(cfg, FULL_SIZE_SLICES)
    K, V, Q, planted, _, _ = generate_all(cfg, slices=sl)
    cache = quantize_pack(_dev(K), _dev(V), cfg.bits)
    idx = _np(score_topk(_dev(Q), cache, cfg.top_k, rank_row=rank_row))
    for (b, h) in sl:
        G = cfg.gqa
        q = Q[b:b + 1, h * G:(h + 1) * G]
        _, kh, _ = _reference_cache(K[b:b + 1, h:h + 1], V[b:b + 1, h:h + 1], cfg.bits)
        r_ref = oracle.rank_scores(q, kh, rank_row, cfg.sm_scale)
        _assert_topk(idx[b:b + 1, h:h + 1], r_ref, cfg.top_k, [(0, 0)], f"{name} row {rank_row} slice {(b, h)}")
        if cfg.n_planted:
            assert np.isin(planted[b, h], idx[b, h]).mean() >= 0.9


# ---------------------------------------------------------------- gather_fp16

@pytest.mark.parametrize("pinned", [True, False])
def test_gather_bitwise(gpu, pinned):
    cfg = get_config("llama8k").with_(seq_len=2048, batch=2)
    K, V, _, _, _, _ = generate_all(cfg)
    rng = np.random.default_rng(5)
    k = 37
    idx = np.stack([np.stack([np.sort(rng.choice(cfg.seq_len, k, replace=False)) for _ in range(cfg.n_kv_heads)])
                    for _ in range(cfg.batch)]).astype(np.int32)
    src_k = torch.from_numpy(K).pin_memory() if pinned else _dev(K)
    src_v = torch.from_numpy(V).pin_memory() if pinned else _dev(V)
    ks, vs = gather_fp16(_dev(idx), src_k, src_v)
    torch.cuda.synchronize()
    wk, wv = oracle.gather_rows(K, V, idx)
    assert np.array_equal(_np(ks).view(np.uint16), wk.view(np.uint16))
    assert np.array_equal(_np(vs).view(np.uint16), wv.view(np.uint16))


def _overlapping_sets(rng, B, H, N, k, k_prev, overlap):
    """(idx, idx_prev) ascending per slice, with round(overlap * min(k, k_prev)) shared positions."""
    idx = np.zeros((B, H, k), dtype=np.int32)
    prev = np.zeros((B, H, k_prev), dtype=np.int32)
    for b in range(B):
        for h in range(H):
            perm = rng.permutation(N)
            shared = int(round(overlap * min(k, k_prev)))
            prev[b, h] = np.sort(perm[:k_prev])
            idx[b, h] = np.sort(np.concatenate([perm[:shared], perm[k_prev:k_prev + k - shared]]))
    return idx, prev


@pytest.mark.parametrize("k,k_prev,overlap", [
    (37, 37, 0.5), (64, 20, 0.9), (20, 64, 0.3), (33, 0, 0.0), (50, 50, 1.0), (50, 50, 0.0), (300, 280, 0.7),
])
def test_reuse_then_fetch_missing_equals_full_gather(gpu, k, k_prev, overlap):
    """Rows of the new set held by the previous set come from the previous buffers (marked
    here, to prove they were copied, not fetched); the rest from pinned host memory."""
    cfg = get_config("llama8k").with_(seq_len=2048, batch=2)
    K, V, _, _, _, _ = generate_all(cfg)
    B, H, N = cfg.batch, cfg.n_kv_heads, cfg.seq_len
    rng = np.random.default_rng(k * 1000 + k_prev)
    idx, prev = _overlapping_sets(rng, B, H, N, k, k_prev, overlap)
    pk, pv = oracle.gather_rows(K, V, prev) if k_prev else (np.zeros((B, H, 0, cfg.head_dim), np.float16),) * 2
    mark_k = (pk.astype(np.float32) + 1).astype(np.float16)
    mark_v = (pv.astype(np.float32) - 1).astype(np.float16)
    hk, hv = torch.from_numpy(K).pin_memory(), torch.from_numpy(V).pin_memory()
    ks = torch.full((B, H, k, cfg.head_dim), float("nan"), dtype=torch.float16, device="cuda")
    vs = torch.full_like(ks, float("nan"))
    ks, vs, fetch = gather_reuse(_dev(idx), _dev(prev), _dev(mark_k), _dev(mark_v), N, k_sel=ks, v_sel=vs)
    gather_fp16_missing(fetch, hk, hv, ks, vs)
    torch.cuda.synchronize()
    resident = oracle.resident_rows(idx, prev)
    assert np.array_equal(_np(fetch), np.where(resident, -1, idx))
    wk, wv = oracle.gather_rows(K, V, idx)
    for b in range(B):
        for h in range(H):
            j = np.searchsorted(prev[b, h], idx[b, h])
            r = resident[b, h]
            wk[b, h, r] = mark_k[b, h, j[r]]
            wv[b, h, r] = mark_v[b, h, j[r]]
    assert np.array_equal(_np(ks).view(np.uint16), wk.view(np.uint16))
    assert np.array_equal(_np(vs).view(np.uint16), wv.view(np.uint16))


def test_reuse_marks_out_of_range_rows_for_a_nan_fetch(gpu):
    K = np.ones((1, 1, 64, 64), dtype=np.float16)
    idx = _dev(np.array([[[3, 10, 64]]], dtype=np.int32))      # 64 is out of range
    prev = _dev(np.array([[[10, 64]]], dtype=np.int32))
    prow = torch.full((1, 1, 2, 64), 2.0, dtype=torch.float16, device="cuda")
    ks, vs, fetch = gather_reuse(idx, prev, prow, prow, 64)
    gather_fp16_missing(fetch, _dev(K), _dev(K), ks, vs)
    torch.cuda.synchronize()
    assert _np(fetch)[0, 0].tolist() == [3, -1, 64]
    out = _np(ks)[0, 0]
    assert np.all(out[0] == 1) and np.all(out[1] == 2) and np.all(np.isnan(out[2]))


def test_gather_rejects_pageable_source_and_flags_bad_rows(gpu):
    import ctypes
    from decode_attention_bit_kivi_amd import _lib
    K = np.ones((1, 1, 64, 64), dtype=np.float16)
    idx = _dev(np.array([[[0, 63, 64, -1]]], dtype=np.int32))
    dk = _dev(K)
    out_k = torch.empty((1, 1, 4, 64), dtype=torch.float16, device="cuda")
    out_v = torch.empty_like(out_k)
    shape = _lib.Shape(1, 1, 1, 64, 64, 1, 32)
    pageable = K.ctypes.data                      # plain host memory: not readable by the GPU
    st = _lib.load().specache_gather_fp16(ctypes.byref(shape), idx.data_ptr(), 4, pageable, dk.data_ptr(),
                                          out_k.data_ptr(), out_v.data_ptr(), None)
    assert st == _lib.SPECACHE_ERR_NOT_PINNED
    ks, vs = gather_fp16(idx, dk, dk)
    torch.cuda.synchronize()
    out = _np(ks)[0, 0]
    assert np.all(out[:2] == 1) and np.all(np.isnan(out[2:]))


# ---------------------------------------------------------------- decode_attn

def _random_idx(rng, B, H, N, k):
    return np.stack([np.stack([np.sort(rng.choice(N, k, replace=False)) for _ in range(H)])
                     for _ in range(B)]).astype(np.int32)


@pytest.mark.parametrize("name,over,mode", [
    ("tiny", {}, "none"),
    ("tiny", {}, "random"),
    ("tiny", dict(bits=2), "all"),
    ("tiny", {}, "tail"),
    ("tiny", dict(n_tokens=1), "random"),
    ("llama8k", {}, "topk"),
    ("llama8k", dict(bits=1, seed=1), "none"),
    ("llama8k", dict(seq_len=8192 + 96), "random"),
    ("llama8k", dict(n_q_heads=64, n_kv_heads=8), "random"),     # G = 8: 16 rows
])
def test_decode_attn_matches_oracle(gpu, name, over, mode):
    cfg = get_config(name).with_(**over)
    if mode == "tail":
        cfg = cfg.with_(tail_len=2)
    K, V, Q, _, KT, VT = generate_all(cfg)
    B, Hkv, N = cfg.batch, cfg.n_kv_heads, cfg.seq_len
    cache = quantize_pack(_dev(K), _dev(V), cfg.bits)
    _, kh, vh = _reference_cache(K, V, cfg.bits)
    rng = np.random.default_rng(9)
    idx = None
    if mode == "random" or mode == "tail":
        idx = _random_idx(rng, B, Hkv, N, cfg.top_k)
    elif mode == "all":
        idx = np.broadcast_to(np.arange(N, dtype=np.int32), (B, Hkv, N)).copy()
    elif mode == "topk":
        idx = _np(score_topk(_dev(Q), cache, cfg.top_k))
    ks = vs = None
    if idx is not None:
        ks, vs = oracle.gather_rows(K, V, idx)
    out = decode_attn(_dev(Q), cache, None if idx is None else _dev(idx),
                      None if ks is None else _dev(ks), None if vs is None else _dev(vs),
                      None if KT is None else _dev(KT), None if VT is None else _dev(VT))
    torch.cuda.synchronize()
    ref = oracle.mixed_attention(Q, kh, vh, idx, ks, vs, KT, VT, sm_scale=cfg.sm_scale)
    _check_attn(_np(out), ref, f"{name} {over} {mode}")


@pytest.mark.parametrize("name,over,mode", [
    ("tiny", {}, "none"),
    ("tiny", {}, "random"),
    ("tiny", dict(bits=2), "all"),                           # every low-bit row replaced
    ("tiny", dict(seq_len=96, top_k=96), "tail"),            # k_next = N
    ("tiny", dict(n_tokens=1, top_k=1), "random"),           # pre-decoding shape, row 0
    ("llama8k", {}, "random"),
    ("llama8k", dict(bits=1, seed=4, tail_len=3), "tail"),
    ("llama8k", dict(seq_len=8192 + 96, seed=5), "random"),  # ragged last split
    ("llama8k", dict(n_q_heads=64, n_kv_heads=8), "random"),  # G = 8: 16 rows
])
def test_fused_step_matches_separate_calls(gpu, name, over, mode):
    cfg = get_config(name).with_(**over)
    if mode == "tail" and cfg.tail_len == 0:
        cfg = cfg.with_(tail_len=2)
    K, V, Q, _, KT, VT = generate_all(cfg)
    B, Hkv, N = cfg.batch, cfg.n_kv_heads, cfg.seq_len
    cache = quantize_pack(_dev(K), _dev(V), cfg.bits)
    rng = np.random.default_rng(11)
    idx = None
    if mode in ("random", "tail"):
        idx = _random_idx(rng, B, Hkv, N, min(cfg.top_k, N))
    elif mode == "all":
        idx = np.broadcast_to(np.arange(N, dtype=np.int32), (B, Hkv, N)).copy()
    ks = vs = None
    if idx is not None:
        ks, vs = oracle.gather_rows(K, V, idx)
    args = (_dev(Q), cache, None if idx is None else _dev(idx), None if ks is None else _dev(ks),
            None if vs is None else _dev(vs), None if KT is None else _dev(KT), None if VT is None else _dev(VT))
    row = 1 if cfg.n_tokens == 2 else 0
    o_sep = decode_attn(*args)
    rk = torch.empty((B, Hkv, N), dtype=torch.float32, device="cuda")
    o_fused, idx_next = decode_step(args[0], cache, cfg.top_k, rank_row=row, idx=args[2], k_sel=args[3],
                                    v_sel=args[4], k_tail=args[5], v_tail=args[6], rank_key_out=rk)
    torch.cuda.synchronize()
    assert torch.equal(o_fused.view(torch.int16), o_sep.view(torch.int16))
    _, kh, vh = _reference_cache(K, V, cfg.bits)
    r_ref = oracle.rank_scores(Q, kh, row, cfg.sm_scale)
    slices = [(b, h) for b in range(B) for h in range(Hkv)]
    _assert_topk(_np(idx_next), r_ref, cfg.top_k, slices)
    _check_rank_keys(_np(rk), r_ref)
    ref = oracle.mixed_attention(Q, kh, vh, idx, ks, vs, KT, VT, sm_scale=cfg.sm_scale)
    _check_attn(_np(o_fused), ref)


@pytest.mark.parametrize("name,over,mode", [
    ("tiny", {}, "none"),
    ("tiny", {}, "random"),
    ("tiny", dict(bits=2), "all"),                           # every row fetched: 16-bit attention mass
    ("tiny", dict(seq_len=96, top_k=96), "tail"),            # k_next = N, tail in the normalization
    ("tiny", dict(n_tokens=1, top_k=1), "random"),
    ("llama8k", {}, "random"),
    ("llama8k", dict(bits=1, seed=4, tail_len=3), "tail"),
    ("llama8k", dict(seq_len=8192 + 96, seed=5), "random"),
    ("llama8k", dict(n_q_heads=64, n_kv_heads=8), "tail"),    # G = 8: 16 rows
])
def test_fused_step_mixed_cache_rank(gpu, name, over, mode):
    """Algorithm 3's reading: the next set ranked by the speculative row of the attention
    over C' with the fetched rows substituted and the visible tail."""
    cfg = get_config(name).with_(**over)
    if mode == "tail" and cfg.tail_len == 0:
        cfg = cfg.with_(tail_len=2)
    K, V, Q, _, KT, VT = generate_all(cfg)
    B, Hkv, N = cfg.batch, cfg.n_kv_heads, cfg.seq_len
    cache = quantize_pack(_dev(K), _dev(V), cfg.bits)
    rng = np.random.default_rng(12)
    idx = None
    if mode in ("random", "tail"):
        idx = _random_idx(rng, B, Hkv, N, min(cfg.top_k, N))
    elif mode == "all":
        idx = np.broadcast_to(np.arange(N, dtype=np.int32), (B, Hkv, N)).copy()
    ks = vs = None
    if idx is not None:
        ks, vs = oracle.gather_rows(K, V, idx)
    args = (_dev(Q), cache, None if idx is None else _dev(idx), None if ks is None else _dev(ks),
            None if vs is None else _dev(vs), None if KT is None else _dev(KT), None if VT is None else _dev(VT))
    row = 1 if cfg.n_tokens == 2 else 0
    o_sep = decode_attn(*args)
    rk = torch.empty((B, Hkv, N), dtype=torch.float32, device="cuda")
    o_fused, idx_next = decode_step(args[0], cache, cfg.top_k, rank_row=row, rank_mixed=True, idx=args[2],
                                    k_sel=args[3], v_sel=args[4], k_tail=args[5], v_tail=args[6], rank_key_out=rk)
    torch.cuda.synchronize()
    assert torch.equal(o_fused.view(torch.int16), o_sep.view(torch.int16))
    _, kh, _ = _reference_cache(K, V, cfg.bits)
    r_ref = oracle.rank_scores_mixed(Q, kh, row, cfg.sm_scale, idx=idx, k_sel=ks, k_tail=KT)
    _assert_topk(_np(idx_next), r_ref, cfg.top_k, [(b, h) for b in range(B) for h in range(Hkv)])
    _check_rank_keys(_np(rk), r_ref)


@pytest.mark.parametrize("seq_len", [32, 96, 32 * 7, 32 * 29, 8192 + 96])
@pytest.mark.parametrize("cus", [8, None])
@pytest.mark.parametrize("top_k", [64, 600])
def test_streamed_split_block_counts(gpu, seq_len, cus, top_k):
    """The LDS-streamed split kernel (head_dim 128, 1-bit codes, G * T = 8) with every count of
    low-bit blocks per wave it meets: none, fewer than its loads ahead, and each remainder of its
    four-step loop.  On 8 compute units the plan takes few, long splits; on the device many short
    ones.  decode_attn against the oracle; the fused step (ranking against C', and by the mixed
    cache) bit for bit against it, with its next selection against the oracle's ranking.  Ranking
    by the mixed cache, up to 512 fetched rows (4 heads) wait in LDS and overwrite their low-bit
    logits at the end; more (600) are stored position by position as they come."""
    cfg = get_config("llama8k").with_(bits=1, seq_len=seq_len, top_k=min(top_k, seq_len), tail_len=3, seed=7)
    K, V, Q, _, KT, VT = generate_all(cfg)
    B, Hkv, N = cfg.batch, cfg.n_kv_heads, cfg.seq_len
    rng = np.random.default_rng(seq_len)
    idx = _random_idx(rng, B, Hkv, N, cfg.top_k)
    ks, vs = oracle.gather_rows(K, V, idx)
    gs = GatherStream(cus) if cus else None
    comp = gs.torch if gs else torch.cuda.current_stream()
    comp.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(comp):
        cache = quantize_pack(_dev(K), _dev(V), cfg.bits)
        args = (_dev(Q), cache, _dev(idx), _dev(ks), _dev(vs), _dev(KT), _dev(VT))
        o_sep = decode_attn(*args)
        o_c, nxt_c = decode_step(args[0], cache, cfg.top_k, rank_row=1, idx=args[2], k_sel=args[3],
                                 v_sel=args[4], k_tail=args[5], v_tail=args[6])
        o_m, nxt_m = decode_step(args[0], cache, cfg.top_k, rank_row=1, rank_mixed=True, idx=args[2],
                                 k_sel=args[3], v_sel=args[4], k_tail=args[5], v_tail=args[6])
        comp.synchronize()
    if gs:
        gs.close()
    assert torch.equal(o_c.view(torch.int16), o_sep.view(torch.int16))
    assert torch.equal(o_m.view(torch.int16), o_sep.view(torch.int16))
    _, kh, vh = _reference_cache(K, V, cfg.bits)
    what = f"seq {seq_len} cus {cus} k {cfg.top_k}"
    ref = oracle.mixed_attention(Q, kh, vh, idx, ks, vs, KT, VT, sm_scale=cfg.sm_scale)
    _check_attn(_np(o_sep), ref, what)
    slices = [(b, h) for b in range(B) for h in range(Hkv)]
    _assert_topk(_np(nxt_c), oracle.rank_scores(Q, kh, 1, cfg.sm_scale), cfg.top_k, slices, what + " C'")
    r_mixed = oracle.rank_scores_mixed(Q, kh, 1, cfg.sm_scale, idx=idx, k_sel=ks, k_tail=KT)
    _assert_topk(_np(nxt_m), r_mixed, cfg.top_k, slices, what + " mixed")


def test_fused_step_next_selection_may_alias_current(gpu):
    cfg = get_config("llama8k").with_(seq_len=4096, seed=7)
    K, V, Q, _, _, _ = generate_all(cfg)
    cache = quantize_pack(_dev(K), _dev(V), cfg.bits)
    q = _dev(Q)
    idx = score_topk(q, cache, cfg.top_k)
    hk, hv = torch.from_numpy(K).pin_memory(), torch.from_numpy(V).pin_memory()
    ks, vs = gather_fp16(idx, hk, hv)
    o_sep = decode_attn(q, cache, idx, ks, vs)
    want_next = score_topk(q, cache, cfg.top_k).clone()
    o, nxt = decode_step(q, cache, cfg.top_k, idx=idx, k_sel=ks, v_sel=vs, idx_next_out=idx)
    torch.cuda.synchronize()
    assert nxt.data_ptr() == idx.data_ptr()
    assert torch.equal(o.view(torch.int16), o_sep.view(torch.int16))
    _, kh, _ = _reference_cache(K, V, cfg.bits)
    r_ref = oracle.rank_scores(Q, kh, 1, cfg.sm_scale)
    slices = [(0, h) for h in range(cfg.n_kv_heads)]
    _assert_topk(_np(nxt), r_ref, cfg.top_k, slices)
    _assert_topk(_np(want_next), r_ref, cfg.top_k, slices)


@pytest.mark.parametrize("name,mixed,stream,rank_row", [
    ("mistral32k", False, "device", 1), ("long128k", False, "device", 1), ("mistral32k", True, "device", 1),
    ("mistral32k", False, "bench", 1), ("layers32", False, "bench", 1), ("mistral32k", False, "bench", 0)])
def test_fused_step_full_size_sampled(gpu, name, mixed, stream, rank_row):
    """The fused step at full size: score_topk seeds the selection, the step gathers its rows
    from pinned host memory and returns the next selection (ranked against C', or by the
    mixed-cache attention row; by the speculative row, or by the real one).  stream = "bench":
    on the compute stream bench.py times (every compute unit but 32, so the split plan is the
    benchmark's); "device": the whole device."""
    cfg = get_config(name)
    sl = _sampled(cfg, FULL_SIZE_SLICES)
    K, V, Q, _, _, _ = generate_all(cfg, slices=sl)
    cs = ComputeStream(32) if stream == "bench" else None
    comp = cs.torch if cs else torch.cuda.current_stream()
    comp.wait_stream(torch.cuda.current_stream())
    hk, hv = torch.from_numpy(K).pin_memory(), torch.from_numpy(V).pin_memory()
    with torch.cuda.stream(comp):
        cache = quantize_pack(_dev(K), _dev(V), cfg.bits)
        q = _dev(Q)
        idx = score_topk(q, cache, cfg.top_k)
        ks, vs = gather_fp16(idx, hk, hv)
        out, nxt = decode_step(q, cache, cfg.top_k, rank_row=rank_row, rank_mixed=mixed, idx=idx, k_sel=ks,
                               v_sel=vs)
        comp.synchronize()
    idx_np, out, nxt = _np(idx), _np(out), _np(nxt)
    if cs:
        cs.close()
    G = cfg.gqa
    for (b, h) in sl:
        q1 = Q[b:b + 1, h * G:(h + 1) * G]
        _, kh, vh = _reference_cache(K[b:b + 1, h:h + 1], V[b:b + 1, h:h + 1], cfg.bits)
        i = idx_np[b:b + 1, h:h + 1]
        rks, rvs = oracle.gather_rows(K[b:b + 1, h:h + 1], V[b:b + 1, h:h + 1], i)
        ref = oracle.mixed_attention(q1, kh, vh, i, rks, rvs, sm_scale=cfg.sm_scale)
        what = f"{name} {'mixed' if mixed else 'lowbit'} {stream} row {rank_row} slice {(b, h)}"
        _check_attn(out[b:b + 1, h * G:(h + 1) * G], ref, what)
        if mixed:
            r_ref = oracle.rank_scores_mixed(q1, kh, rank_row, cfg.sm_scale, idx=i, k_sel=rks)
        else:
            r_ref = oracle.rank_scores(q1, kh, rank_row, cfg.sm_scale)
        _assert_topk(nxt[b:b + 1, h:h + 1], r_ref, cfg.top_k, [(0, 0)], what)


@pytest.mark.parametrize("name,over", [
    ("tiny", {}),
    ("tiny", dict(tail_len=3)),
    ("tiny", dict(n_tokens=1, head_dim=128, seq_len=96)),
    ("llama8k", {}),
    ("llama8k", dict(seq_len=8192 + 96, tail_len=2)),
    ("llama8k", dict(n_q_heads=64, n_kv_heads=8)),
])
def test_fp16_comparator_matches_oracle(gpu, name, over):
    """The 16-bit comparator: attention over the float16 cache (the oracle's mixed attention
    with every row fetched) -- and the same as decode_attn fetching every row."""
    cfg = get_config(name).with_(**over)
    K, V, Q, _, KT, VT = generate_all(cfg)
    B, H, N = cfg.batch, cfg.n_kv_heads, cfg.seq_len
    kt = None if KT is None else _dev(KT)
    vt = None if VT is None else _dev(VT)
    out = decode_attn_fp16(_dev(Q), _dev(K), _dev(V), k_tail=kt, v_tail=vt)
    torch.cuda.synchronize()
    ref = oracle.mixed_attention(Q, K.astype(np.float64), V.astype(np.float64), sm_scale=cfg.sm_scale, k_tail=KT,
                                 v_tail=VT)
    _check_attn(_np(out), ref)
    cache = quantize_pack(_dev(K), _dev(V), cfg.bits)
    idx = np.broadcast_to(np.arange(N, dtype=np.int32), (B, H, N)).copy()
    o_all = decode_attn(_dev(Q), cache, _dev(idx), _dev(K), _dev(V), kt, vt)
    torch.cuda.synchronize()
    assert _attn_err(_np(out), _np(o_all).astype(np.float64)) <= 1e-3


@pytest.mark.parametrize("name,stream", [("mistral32k", "device"), ("long128k", "device"), ("layers32", "bench"),
                                         ("mistral32k", "bench")])
def test_decode_step_full_size_sampled(gpu, name, stream):
    """The whole step at full size in four calls: score_topk -> gather from pinned host ->
    decode_attn (stream as in test_fused_step_full_size_sampled)."""
    cfg = get_config(name)
    sl = _sampled(cfg, FULL_SIZE_SLICES)
    K, V, Q, _, _, _ = generate_all(cfg, slices=sl)
    cs = ComputeStream(32) if stream == "bench" else None
    comp = cs.torch if cs else torch.cuda.current_stream()
    comp.wait_stream(torch.cuda.current_stream())
    hk, hv = torch.from_numpy(K).pin_memory(), torch.from_numpy(V).pin_memory()
    with torch.cuda.stream(comp):
        cache = quantize_pack(_dev(K), _dev(V), cfg.bits)
        idx = score_topk(_dev(Q), cache, cfg.top_k)
        ks, vs = gather_fp16(idx, hk, hv)
        out = decode_attn(_dev(Q), cache, idx, ks, vs)
        comp.synchronize()
    out, idx = _np(out), _np(idx)
    if cs:
        cs.close()
    G = cfg.gqa
    for (b, h) in sl:
        q = Q[b:b + 1, h * G:(h + 1) * G]
        _, kh, vh = _reference_cache(K[b:b + 1, h:h + 1], V[b:b + 1, h:h + 1], cfg.bits)
        i = idx[b:b + 1, h:h + 1]
        rks, rvs = oracle.gather_rows(K[b:b + 1, h:h + 1], V[b:b + 1, h:h + 1], i)
        ref = oracle.mixed_attention(q, kh, vh, i, rks, rvs, sm_scale=cfg.sm_scale)
        _check_attn(out[b:b + 1, h * G:(h + 1) * G], ref, f"{name} {stream} slice {(b, h)}")
        r_ref = oracle.rank_scores(q, kh, 1, cfg.sm_scale)
        _assert_topk(i, r_ref, cfg.top_k, [(0, 0)], f"{name} {stream} slice {(b, h)}")


def test_gather_on_cu_limited_stream(gpu):
    cfg = get_config("llama8k").with_(seq_len=4096, batch=2)
    K, V, _, _, _, _ = generate_all(cfg)
    rng = np.random.default_rng(6)
    idx = _dev(_random_idx(rng, cfg.batch, cfg.n_kv_heads, cfg.seq_len, 50))
    hk, hv = torch.from_numpy(K).pin_memory(), torch.from_numpy(V).pin_memory()
    gs = GatherStream(8)
    ev = torch.cuda.Event()
    ev.record()
    gs.torch.wait_event(ev)
    ks, vs = gather_fp16(idx, hk, hv, stream=gs)
    gs.torch.synchronize()
    wk, wv = oracle.gather_rows(K, V, _np(idx))
    assert np.array_equal(_np(ks).view(np.uint16), wk.view(np.uint16))
    assert np.array_equal(_np(vs).view(np.uint16), wv.view(np.uint16))
    gs.close()
    with pytest.raises(SpecacheError):
        GatherStream(100000)
    with pytest.raises(SpecacheError):
        GatherStream(4)
    with pytest.raises(SpecacheError):
        ComputeStream(4)
    with pytest.raises(SpecacheError):
        ComputeStream(100000)


@pytest.mark.parametrize("compute", ["torch", "exclusive"])
def test_overlapped_streams_match_serial(gpu, compute):
    """score_topk on the compute stream, gather on a side stream after an event,
    attention after the gather's event, then the fused step: bitwise equal to the
    same calls serialized on the same compute stream (the split plan follows the
    stream's compute units).  The compute stream is a plain torch stream or the
    library's stream on the compute units the gather stream leaves free."""
    cfg = get_config("llama8k").with_(batch=2)
    K, V, Q, _, _, _ = generate_all(cfg)
    cache = quantize_pack(_dev(K), _dev(V), cfg.bits)
    q = _dev(Q)
    hk, hv = torch.from_numpy(K).pin_memory(), torch.from_numpy(V).pin_memory()
    gs = GatherStream(8)
    side = gs.torch
    cs = ComputeStream(8) if compute == "exclusive" else None
    comp = cs.torch if cs else torch.cuda.Stream()   # non-default: the gather stream is a blocking stream
    comp.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(comp):
        idx0 = score_topk(q, cache, cfg.top_k)
        ks0, vs0 = gather_fp16(idx0, hk, hv)
        o0 = decode_attn(q, cache, idx0, ks0, vs0)
        of0, nx0 = decode_step(q, cache, cfg.top_k, idx=idx0, k_sel=ks0, v_sel=vs0)
        comp.synchronize()

        ks = torch.full_like(ks0, float("nan"))
        vs = torch.full_like(vs0, float("nan"))
        idx = score_topk(q, cache, cfg.top_k)
        ev = torch.cuda.Event()
        ev.record(comp)
        side.wait_event(ev)
        gather_fp16(idx, hk, hv, k_sel=ks, v_sel=vs, stream=side)
        ev2 = torch.cuda.Event()
        ev2.record(side)
        comp.wait_event(ev2)
        o1 = decode_attn(q, cache, idx, ks, vs)
        of1, nx1 = decode_step(q, cache, cfg.top_k, idx=idx, k_sel=ks, v_sel=vs)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx0)
    assert torch.equal(o1.view(torch.int16), o0.view(torch.int16))
    assert torch.equal(of1.view(torch.int16), of0.view(torch.int16))
    assert torch.equal(nx1, nx0)
    # the result on the default stream (whole device) agrees to the attention tolerance
    o_dev = decode_attn(q, cache, idx0, ks0, vs0)
    torch.cuda.synchronize()
    assert _attn_err(_np(o1), _np(o_dev).astype(np.float64)) <= ATTN_TOL
    gs.close()
    if cs:
        cs.close()


@pytest.mark.parametrize("name,over,qscale", [
    ("tiny", {}, 1.0),
    ("tiny", dict(top_k=64), 1.0),                         # k = N / 8: one position per bound group
    ("tiny", dict(top_k=65), 1.0),                         # k > N / 8: the unpruned selection
    ("llama8k", {}, 1.0),
    ("llama8k", dict(seq_len=8192 + 96, seed=5), 1.0),     # ragged last split
    ("llama8k", dict(seq_len=4096, top_k=256, bits=1), 1.0),
    ("llama8k", dict(seq_len=32768, top_k=328, bits=1, seed=2), 1.0),   # a 32K slice, k = 1%
    ("llama8k", dict(seq_len=20480, top_k=300, seed=3), 0.0),           # every rank equal
    ("llama8k", dict(seq_len=20480, top_k=300, seed=3), 1e-3),          # a crowded threshold bin
    ("llama8k", dict(n_tokens=1, top_k=40), 1.0),          # pre-decoding shape, row 0
    ("llama8k", dict(seq_len=8192 + 96, seed=6, tail_len=3), 1.0),   # a visible tail (mixed: in the LSE)
])
@pytest.mark.parametrize("mixed", [False, True])
def test_fused_step_selection_from_bounds(gpu, name, over, qscale, mixed):
    """Without a key output the fused step selects from per-8-position logit maxima: groups
    whose upper bound cannot reach the k-th rank are never read.  Ranking by the mixed cache
    (Algorithm 3's reading), the fetched rows' 16-bit logits replace the low-bit ones after the
    maxima are taken, so the groups holding them are always read and give no lower bound.  The
    set must be the oracle's (tie band) and the one the unpruned selection makes from the same
    logits (which runs when the keys are asked for)."""
    cfg = get_config(name).with_(**over)
    K, V, Q, _, KT, VT = generate_all(cfg)
    Q = (Q.astype(np.float32) * qscale).astype(np.float16)
    B, Hkv, N = cfg.batch, cfg.n_kv_heads, cfg.seq_len
    cache = quantize_pack(_dev(K), _dev(V), cfg.bits)
    rng = np.random.default_rng(21)
    idx = _random_idx(rng, B, Hkv, N, cfg.top_k)
    ks, vs = oracle.gather_rows(K, V, idx)
    row = 1 if cfg.n_tokens == 2 else 0
    args = dict(rank_row=row, rank_mixed=mixed, idx=_dev(idx), k_sel=_dev(ks), v_sel=_dev(vs))
    if KT is not None:
        args.update(k_tail=_dev(KT), v_tail=_dev(VT))
    o1, pruned = decode_step(_dev(Q), cache, cfg.top_k, **args)
    rk = torch.empty((B, Hkv, N), dtype=torch.float32, device="cuda")
    o2, full = decode_step(_dev(Q), cache, cfg.top_k, rank_key_out=rk, **args)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(pruned, full)
    _, kh, _ = _reference_cache(K, V, cfg.bits)
    if mixed:
        r_ref = oracle.rank_scores_mixed(Q, kh, row, cfg.sm_scale, idx=idx, k_sel=ks, k_tail=KT)
    else:
        r_ref = oracle.rank_scores(Q, kh, row, cfg.sm_scale)
    if qscale == 0.0 and not mixed:
        assert np.array_equal(_np(pruned), np.broadcast_to(np.arange(cfg.top_k, dtype=np.int32), pruned.shape))
    _assert_topk(_np(pruned), r_ref, cfg.top_k, [(b, h) for b in range(B) for h in range(Hkv)],
                 f"{name} {over} q x{qscale} {'mixed' if mixed else 'lowbit'} bounds")
