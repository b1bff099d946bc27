"""Pins of the CPU oracle against things other than itself.

Each test checks one oracle function against what the pages and the
mathematics fix: closed forms the SpeCache summary prints (§3 quantizer
equations), exact arithmetic with Python fractions, library routines
(torch.topk, torch scaled_dot_product_attention in float64 on the CPU),
invariants (probabilities sum to one) and brute force on tiny inputs.
They are chosen so that a plausible slip in the oracle -- a wrong coefficient,
a swapped group direction, half-to-even rounding, a transposed operand, a
wrong GQA head mapping, a dropped mask -- fails at least one of them.
"""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from workloads import get_config, generate_all

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _fr(x) -> Fraction:
    return Fraction(float(x))


# --------------------------------------------------------------------------
# Quantizer: closed forms of SpeCache §3
# --------------------------------------------------------------------------

def test_one_bit_closed_form_fixture():
    with open(os.path.join(GOLDEN, "quantizer_closed_forms.json")) as f:
        cases = json.load(f)["one_bit"]
    for case in cases:
        x = np.array(case["group"], dtype=np.float16).reshape(32, 1)
        codes, z, s = oracle.quantize_keys(x, bits=1)
        assert float(z[0, 0]) == case["z"] and float(s[0, 0]) == case["s"]
        deq = oracle.dequantize_keys(codes, z, s)[:, 0]
        assert deq.tolist() == case["dequantized"], case["cite"]


def _dyadic_groups(rng, n_groups, lo=-32, hi=32, den=8):
    return (rng.integers(lo, hi + 1, size=(n_groups, 32)) / den).astype(np.float16)


@pytest.mark.parametrize("direction", ["keys", "values"])
def test_one_bit_values_go_to_interval_centres(direction):
    """SpeCache §3: [min, mid) -> (3 min + max)/4, (mid, max] -> (min + 3 max)/4;
    the midpoint itself goes up (round half up).  Dyadic data keeps every step exact."""
    rng = np.random.default_rng(11)
    g = _dyadic_groups(rng, 200)
    if direction == "keys":
        codes, z, s = oracle.quantize_keys(g.T.copy(), bits=1)        # [32 tokens, 200 channels]
        deq = oracle.dequantize_keys(codes, z, s).T
    else:
        codes, z, s = oracle.quantize_values(g, bits=1)               # [200 tokens, 32 channels]
        deq = oracle.dequantize_values(codes, z, s)
    for i in range(g.shape[0]):
        xs = [_fr(v) for v in g[i]]
        mn, mx = min(xs), max(xs)
        lo_c, hi_c, mid = (3 * mn + mx) / 4, (mn + 3 * mx) / 4, (mn + mx) / 2
        for j, x in enumerate(xs):
            want = hi_c if x >= mid else lo_c
            if mn == mx:
                want = mn
            assert _fr(deq[i, j]) == want, (i, j, x, mn, mx)


def test_two_bit_levels_and_half_up():
    """KIVI at B = 2 (SpeCache §3): levels min + i (max - min)/3, nearest level,
    an exact half-way value rounds up."""
    rng = np.random.default_rng(12)
    mn = rng.integers(-40, 10, size=300) / 8
    step = rng.integers(1, 10, size=300) / 8
    t = rng.integers(0, 7, size=(300, 32)) / 2                  # multiples of 1/2 in [0, 3]
    t[:, 0], t[:, 1] = 0, 3
    x = (mn[:, None] + step[:, None] * t).astype(np.float16)
    codes, z, s = oracle.quantize_values(x, bits=2)
    deq = oracle.dequantize_values(codes, z, s)
    for i in range(300):
        assert _fr(z[i, 0]) == _fr(mn[i]) and _fr(s[i, 0]) == _fr(step[i])
        for j in range(32):
            tt = Fraction(t[i, j]).limit_denominator(2)
            want_code = min(3, math.floor(tt + Fraction(1, 2)))
            assert codes[i, j] == want_code, (i, j, tt)
            assert _fr(deq[i, j]) == _fr(mn[i]) + want_code * _fr(step[i])


@pytest.mark.parametrize("bits", [1, 2])
@pytest.mark.parametrize("direction", ["keys", "values"])
def test_codes_are_round_half_up_of_exact_ratio(bits, direction):
    """Random float16 data: every code equals round-half-up of the exact ratio
    (x - z16) / s16, clamped to [0, 2^B - 1], except within float32 rounding of a
    half-integer; z16 / s16 are the float16 roundings of the §3 expressions."""
    rng = np.random.default_rng(13 + bits)
    x = (rng.standard_normal((64, 96)) * rng.choice([0.01, 1.0, 30.0], size=(1, 96))).astype(np.float16)
    if direction == "keys":
        codes, z, s = oracle.quantize_keys(x, bits)
        zz, ss = np.repeat(z, 32, axis=0), np.repeat(s, 32, axis=0)
        groups = [x[32 * j:32 * j + 32, c] for j in range(2) for c in range(96)]
        metas = [(z[j, c], s[j, c]) for j in range(2) for c in range(96)]
    else:
        codes, z, s = oracle.quantize_values(x, bits)
        zz, ss = np.repeat(z, 32, axis=1), np.repeat(s, 32, axis=1)
        groups = [x[p, 32 * w:32 * w + 32] for p in range(64) for w in range(3)]
        metas = [(z[p, w], s[p, w]) for p in range(64) for w in range(3)]
    qmax = (1 << bits) - 1
    ambiguous = 0
    for idx in np.ndindex(x.shape):
        sv = _fr(ss[idx])
        if sv == 0:
            assert codes[idx] == 0
            continue
        ratio = (_fr(x[idx]) - _fr(zz[idx])) / sv
        frac = ratio - math.floor(ratio)
        decisive = 0 <= math.floor(ratio) < qmax     # boundary j + 1/2 with 0 <= j < qmax
        if decisive and abs(frac - Fraction(1, 2)) < Fraction(1, 1 << 20):
            ambiguous += 1
            continue
        want = min(qmax, max(0, math.floor(ratio + Fraction(1, 2))))
        assert codes[idx] == want, (idx, float(ratio))
    assert ambiguous < 0.001 * x.size
    off_by_rounding = 0
    for grp, (zv, sv) in zip(groups, metas):
        mn, mx = min(map(_fr, grp)), max(map(_fr, grp))
        if bits == 1:
            zx, sx = (3 * mn + mx) / 4, (mx - mn) / 2
        else:
            zx, sx = mn, (mx - mn) / 3
        for got, exact in ((zv, zx), (sv, sx)):
            r16 = np.float16(float(exact))
            if _fr(got) != _fr(r16):
                off_by_rounding += 1
                ulp = np.spacing(np.abs(r16)).astype(np.float64)
                assert abs(float(got) - float(exact)) <= 1.01 * float(ulp)
    assert off_by_rounding <= 0.01 * 2 * len(groups)


@pytest.mark.parametrize("group", [32, 64])
def test_group_directions(group):
    """SemKV §2.1: keys are grouped per channel along tokens, values per token
    along channels (SpeCache §4: groups of 32 or 64).  Changing one element moves
    only its own group's metadata."""
    rng = np.random.default_rng(3)
    x = rng.standard_normal((128, 128)).astype(np.float16)
    _, zk, sk = oracle.quantize_keys(x, 2, group)
    _, zv, sv = oracle.quantize_values(x, 2, group)
    assert sk.shape == (128 // group, 128) and sv.shape == (128, 128 // group)
    y = x.copy()
    y[77, 40] = np.float16(50.0)                # new maximum of its groups
    _, zk2, sk2 = oracle.quantize_keys(y, 2, group)
    _, zv2, sv2 = oracle.quantize_values(y, 2, group)
    changed_k = np.argwhere(sk2 != sk)
    changed_v = np.argwhere(sv2 != sv)
    assert changed_k.tolist() == [[77 // group, 40]]
    assert changed_v.tolist() == [[77, 40 // group]]
    assert np.array_equal(zk2, zk) and np.array_equal(zv2, zv)


def test_group_64_is_the_min_max_of_its_two_halves():
    """A 64-group's 1-bit zero-point and scale are those of the min and max over both of its
    32-element halves (SpeCache §3's formula applied to the larger group)."""
    rng = np.random.default_rng(9)
    x = rng.standard_normal((64, 8)).astype(np.float16)
    _, z64, s64 = oracle.quantize_keys(x, 1, 64)
    mn = np.minimum(x[:32].min(0), x[32:].min(0)).astype(np.float32)
    mx = np.maximum(x[:32].max(0), x[32:].max(0)).astype(np.float32)
    z, s = oracle.zero_point_scale(mn, mx, 1)
    assert np.array_equal(z64[0].view(np.uint16), z.view(np.uint16))
    assert np.array_equal(s64[0].view(np.uint16), s.view(np.uint16))


def test_constant_group_and_signed_zero():
    x = np.full((32, 2), 0.75, dtype=np.float16)
    x[:, 1] = np.float16(-0.0)
    for bits in (1, 2):
        codes, z, s = oracle.quantize_keys(x, bits)
        assert np.all(codes == 0) and np.all(s == 0)
        assert float(z[0, 0]) == 0.75
        assert np.signbit(z[0, 1]) == False  # noqa: E712  (stored as +0)
        assert np.array_equal(oracle.dequantize_keys(codes, z, s), x.astype(np.float64))


# --------------------------------------------------------------------------
# Ranking: ArgTopK over the speculative row (SpeCache Alg. 3)
# --------------------------------------------------------------------------

def _rand_case(rng, B=2, Hkv=2, G=2, T=2, N=96, D=16):
    q = rng.standard_normal((B, Hkv * G, T, D)).astype(np.float16)
    k = rng.standard_normal((B, Hkv, N, D))
    return q, k


def test_rank_mass_sums_to_group_size():
    rng = np.random.default_rng(4)
    q, k = _rand_case(rng, G=4)
    r = oracle.rank_scores(q, k, rank_row=1, sm_scale=0.25)
    assert np.allclose(np.exp(r).sum(axis=-1), 4.0, rtol=0, atol=1e-12)


def test_rank_single_head_is_torch_topk_of_logits():
    """G = 1: ArgTopK of the attention row is the top-k of that head's logits."""
    rng = np.random.default_rng(5)
    q, k = _rand_case(rng, B=2, Hkv=3, G=1, N=200, D=32)
    for row in (0, 1):
        idx = oracle.topk_positions(oracle.rank_scores(q, k, row, 0.125), 17)
        logits = torch.from_numpy(q[:, :, row, :].astype(np.float64)).unsqueeze(2) @ \
            torch.from_numpy(k).transpose(-1, -2)
        want = torch.topk(logits.squeeze(2), 17, dim=-1).indices.sort(dim=-1).values.numpy()
        assert np.array_equal(idx, want)


def test_rank_identical_heads_reduce_to_single_head():
    """G identical query heads: r = log(G) + log softmax, same order as one head."""
    rng = np.random.default_rng(6)
    q1, k = _rand_case(rng, B=1, Hkv=2, G=1, N=128, D=16)
    q4 = np.repeat(q1, 4, axis=1)
    r1 = oracle.rank_scores(q1, k, 1, 0.3)
    r4 = oracle.rank_scores(q4, k, 1, 0.3)
    assert np.allclose(r4, r1 + math.log(4), atol=1e-12)


def test_rank_gqa_head_mapping():
    """Query head hq reads KV head hq // G: plant a key in each KV head that only
    that head's G query heads point at."""
    B, Hkv, G, N, D = 1, 3, 2, 64, 8
    k = np.zeros((B, Hkv, N, D))
    q = np.zeros((B, Hkv * G, 2, D), dtype=np.float16)
    target = [5, 40, 17]
    for h in range(Hkv):
        k[0, h, target[h], h] = 4.0
        for g in range(G):
            q[0, h * G + g, :, h] = 3.0
    idx = oracle.topk_positions(oracle.rank_scores(q, k, 1, 1.0), 1)
    assert idx[0, :, 0].tolist() == target


def test_rank_uses_requested_row():
    B, Hkv, G, N, D = 1, 1, 2, 32, 4
    k = np.zeros((B, Hkv, N, D))
    k[0, 0, 3, 0] = 5.0
    k[0, 0, 30, 1] = 5.0
    q = np.zeros((B, 2, 2, D), dtype=np.float16)
    q[0, :, 0, 0] = 2.0      # real row looks at position 3
    q[0, :, 1, 1] = 2.0      # speculative row looks at position 30
    assert oracle.topk_positions(oracle.rank_scores(q, k, 0, 1.0), 1)[0, 0, 0] == 3
    assert oracle.topk_positions(oracle.rank_scores(q, k, 1, 1.0), 1)[0, 0, 0] == 30


def _torch_mass(q_row, keys, sm_scale, n_cached):
    """log of the summed softmax mass of the G heads (torch softmax over all given keys) on the
    first n_cached keys.  q_row [B, Hkv, G, D], keys [B, Hkv, M, D]."""
    logits = sm_scale * torch.from_numpy(q_row) @ torch.from_numpy(keys).transpose(-1, -2)
    p = torch.softmax(logits, dim=-1)[..., :n_cached]
    return torch.log(p.sum(dim=2)).numpy()


def test_mixed_rank_fetching_everything_is_fp16_attention_mass():
    """Algorithm 3's reading with every row fetched: the rank is the attention mass of the
    16-bit keys, computed here with torch's softmax."""
    rng = np.random.default_rng(21)
    q, k = _rand_case(rng, B=2, Hkv=2, G=3, N=64, D=16)
    k16 = (k + 0.1 * rng.standard_normal(k.shape)).astype(np.float16)
    idx = np.broadcast_to(np.arange(64, dtype=np.int32), (2, 2, 64)).copy()
    for row in (0, 1):
        r = oracle.rank_scores_mixed(q, k, row, 0.3, idx=idx, k_sel=k16)
        qr = q[:, :, row, :].astype(np.float64).reshape(2, 2, 3, 16)
        want = _torch_mass(qr, k16.astype(np.float64), 0.3, 64)
        assert np.allclose(r, want, atol=1e-12)


def test_mixed_rank_replaces_fetched_rows_and_normalizes_over_visible_tail():
    """Fetched rows use their 16-bit keys; the visible tail entries (j <= R - T + t) share
    each head's softmax but are no candidates."""
    rng = np.random.default_rng(22)
    B, Hkv, G, T, N, D, R = 1, 2, 2, 2, 48, 8, 3
    q, k = _rand_case(rng, B=B, Hkv=Hkv, G=G, T=T, N=N, D=D)
    idx = np.stack([np.sort(rng.choice(N, 5, replace=False)) for _ in range(Hkv)])[None].astype(np.int32)
    k_sel = rng.standard_normal((B, Hkv, 5, D)).astype(np.float16)
    k_tail = rng.standard_normal((B, Hkv, R, D)).astype(np.float16)
    mixed = k.copy()
    for h in range(Hkv):
        mixed[0, h, idx[0, h]] = k_sel[0, h].astype(np.float64)
    for row in (0, 1):
        visible = R - T + row + 1
        keys = np.concatenate([mixed, k_tail[:, :, :visible].astype(np.float64)], axis=2)
        qr = q[:, :, row, :].astype(np.float64).reshape(B, Hkv, G, D)
        want = _torch_mass(qr, keys, 0.5, N)
        got = oracle.rank_scores_mixed(q, k, row, 0.5, idx=idx, k_sel=k_sel, k_tail=k_tail)
        assert np.allclose(got, want, atol=1e-12)
        assert np.all(np.exp(got).sum(axis=-1) < G)       # the tail holds some of the mass


def test_mixed_rank_hides_the_speculative_entry_from_the_real_row():
    B, Hkv, G, T, N, D, R = 1, 1, 1, 2, 32, 4, 2
    k = np.zeros((B, Hkv, N, D))
    q = np.zeros((B, 1, T, D), dtype=np.float16)
    q[..., 0] = 1.0
    k_tail = np.zeros((B, Hkv, R, D), dtype=np.float16)
    k_tail[0, 0, R - 1, 0] = 30.0                    # the speculative token's own key
    r0 = oracle.rank_scores_mixed(q, k, 0, 1.0, k_tail=k_tail)
    r1 = oracle.rank_scores_mixed(q, k, 1, 1.0, k_tail=k_tail)
    assert np.allclose(np.exp(r0).sum(), N / (N + 1))   # row 0 sees one tail entry, logit 0
    assert np.exp(r1).sum() < 1e-9                       # row 1 also sees the logit-30 entry


def test_mixed_rank_without_fetch_or_tail_is_the_c_prime_rank():
    rng = np.random.default_rng(23)
    q, k = _rand_case(rng, G=4)
    assert np.allclose(oracle.rank_scores_mixed(q, k, 1, 0.25), oracle.rank_scores(q, k, 1, 0.25), atol=1e-12)


def test_topk_ties_and_full_set():
    r = np.zeros((1, 2, 50))
    r[0, 1, 7] = 1.0
    assert oracle.topk_positions(r, 5)[0, 0].tolist() == [0, 1, 2, 3, 4]
    assert oracle.topk_positions(r, 3)[0, 1].tolist() == [0, 1, 7]
    assert oracle.topk_positions(r, 50)[0, 1].tolist() == list(range(50))
    assert oracle.topk_positions(r, 0).shape == (1, 2, 0)


def test_topk_brute_force_tiny():
    """Brute force: the chosen set maximizes the summed r among all k-subsets."""
    from itertools import combinations
    rng = np.random.default_rng(8)
    r = rng.standard_normal((1, 1, 10))
    idx = oracle.topk_positions(r, 3)[0, 0]
    best = max(combinations(range(10), 3), key=lambda c: sum(r[0, 0, list(c)]))
    assert sorted(best) == idx.tolist()


@pytest.mark.parametrize("bits", [1, 2])
def test_planted_peak_recalled_from_low_bit_copy(bits):
    """The synthetic planted positions (about 90% of the attention mass, as in the
    SpeCache §2 sparsity observation) are found from the low-bit copy."""
    cfg = get_config("llama8k").with_(seq_len=2048, batch=1, n_kv_heads=2, n_q_heads=8, bits=bits,
                                      top_k=64)
    K, V, Q, planted, _, _ = generate_all(cfg)
    codes, z, s = oracle.quantize_keys(K, bits)
    khat = oracle.dequantize_keys(codes, z, s)
    idx, _ = oracle.score_topk(Q, khat, 1, cfg.sm_scale, cfg.top_k)
    for h in range(2):
        recall = np.isin(planted[0, h], idx[0, h]).mean()
        assert recall >= 0.9, (h, recall)


# --------------------------------------------------------------------------
# Attention over C' ∪ C_κ
# --------------------------------------------------------------------------

def _sdpa(q16, keys, values, mask=None):
    """torch SDPA in float64 on the CPU, GQA by repeating each KV head G times."""
    B, Hq, T, D = q16.shape
    G = Hq // keys.shape[1]
    qt = torch.from_numpy(q16.astype(np.float64))
    kt = torch.from_numpy(np.asarray(keys, dtype=np.float64)).repeat_interleave(G, dim=1)
    vt = torch.from_numpy(np.asarray(values, dtype=np.float64)).repeat_interleave(G, dim=1)
    m = None if mask is None else torch.from_numpy(mask)
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m,
                                                            scale=1.0 / math.sqrt(D)).numpy()


def _small_cache(bits=1, seed=0, N=256, D=64):
    cfg = get_config("tiny").with_(seq_len=N, head_dim=D, bits=bits, seed=seed, batch=2)
    K, V, Q, _, _, _ = generate_all(cfg)
    kc, kz, ks = oracle.quantize_keys(K, bits)
    vc, vz, vs = oracle.quantize_values(V, bits)
    return cfg, K, V, Q, oracle.dequantize_keys(kc, kz, ks), oracle.dequantize_values(vc, vz, vs)


@pytest.mark.parametrize("bits", [1, 2])
def test_attention_without_fetch_is_sdpa_over_dequantized(bits):
    cfg, K, V, Q, kh, vh = _small_cache(bits)
    o = oracle.mixed_attention(Q, kh, vh, sm_scale=cfg.sm_scale)
    assert np.allclose(o, _sdpa(Q, kh, vh), rtol=0, atol=1e-12)


def test_attention_fetching_everything_is_fp16_attention():
    cfg, K, V, Q, kh, vh = _small_cache(1)
    N = K.shape[2]
    idx = np.broadcast_to(np.arange(N, dtype=np.int32), K.shape[:2] + (N,))
    ks, vs = oracle.gather_rows(K, V, idx)
    o = oracle.mixed_attention(Q, kh, vh, idx, ks, vs, sm_scale=cfg.sm_scale)
    assert np.allclose(o, _sdpa(Q, K, V), rtol=0, atol=1e-12)


def test_attention_replacement_semantics():
    """Rows of κ are replaced, not added: fetching rows equal to their dequantized
    values leaves the output unchanged; fetching true rows equals SDPA over the
    hand-mixed cache."""
    cfg, K, V, Q, kh, vh = _small_cache(2)
    rng = np.random.default_rng(9)
    N = K.shape[2]
    idx = np.stack([np.stack([np.sort(rng.choice(N, 20, replace=False)) for _ in range(2)])
                    for _ in range(2)]).astype(np.int32)
    same = oracle.mixed_attention(Q, kh, vh, idx, *oracle.gather_rows(kh, vh, idx), sm_scale=cfg.sm_scale)
    assert np.allclose(same, oracle.mixed_attention(Q, kh, vh, sm_scale=cfg.sm_scale), atol=1e-12)
    mk, mv = kh.copy(), vh.copy()
    for b in range(2):
        for h in range(2):
            mk[b, h, idx[b, h]] = K[b, h, idx[b, h]]
            mv[b, h, idx[b, h]] = V[b, h, idx[b, h]]
    o = oracle.mixed_attention(Q, kh, vh, idx, *oracle.gather_rows(K, V, idx), sm_scale=cfg.sm_scale)
    assert np.allclose(o, _sdpa(Q, mk, mv), atol=1e-12)


def test_attention_rows_sum_to_one():
    cfg, K, V, Q, kh, vh = _small_cache(1)
    p, _, _ = oracle.attention_probs(Q, kh, vh, sm_scale=cfg.sm_scale)
    assert np.all(np.abs(p.sum(-1) - 1.0) < 1e-12)


def test_attention_tail_mask():
    """MaskedSoftmax of Alg. 3: the real row does not see the speculative token's
    new entry; the speculative row sees both (checked against SDPA with a mask)."""
    cfg, K, V, Q, kh, vh = _small_cache(1)
    rng = np.random.default_rng(10)
    B, Hkv, N, D = K.shape
    kt = rng.standard_normal((B, Hkv, 2, D)).astype(np.float16)
    vt = rng.standard_normal((B, Hkv, 2, D)).astype(np.float16)
    o = oracle.mixed_attention(Q, kh, vh, k_tail=kt, v_tail=vt, sm_scale=cfg.sm_scale)
    mask = np.ones((2, N + 2), dtype=bool)
    mask[0, N + 1] = False
    want = _sdpa(Q, np.concatenate([kh, kt], 2), np.concatenate([vh, vt], 2), mask)
    assert np.allclose(o, want, atol=1e-12)
    kt2 = kt.copy()
    kt2[:, :, 1] += np.float16(3)
    o2 = oracle.mixed_attention(Q, kh, vh, k_tail=kt2, v_tail=vt, sm_scale=cfg.sm_scale)
    assert np.array_equal(o2[:, :, 0], o[:, :, 0]) and not np.allclose(o2[:, :, 1], o[:, :, 1])


def test_resident_rows_brute_force():
    """Rows of the new set whose position the previous set also holds (numpy isin as the check)."""
    rng = np.random.default_rng(31)
    for k, kp in ((5, 7), (16, 16), (9, 1), (4, 0)):
        idx = np.stack([np.sort(rng.choice(40, k, replace=False)) for _ in range(3)])[None].astype(np.int32)
        prev = np.stack([np.sort(rng.choice(40, kp, replace=False)) for _ in range(3)])[None].astype(np.int32)
        got = oracle.resident_rows(idx, prev)
        for h in range(3):
            assert got[0, h].tolist() == np.isin(idx[0, h], prev[0, h]).tolist()
    same = np.arange(8, dtype=np.int32)[None, None]
    assert oracle.resident_rows(same, same).all()


def test_gather_is_index_select():
    rng = np.random.default_rng(1)
    k = rng.standard_normal((2, 3, 40, 8)).astype(np.float16)
    v = rng.standard_normal((2, 3, 40, 8)).astype(np.float16)
    idx = rng.integers(0, 40, size=(2, 3, 5)).astype(np.int32)
    ks, vs = oracle.gather_rows(k, v, idx)
    tk = torch.from_numpy(k).flatten(0, 1)
    ti = torch.from_numpy(idx).flatten(0, 1).long()
    want = torch.stack([tk[i].index_select(0, ti[i]) for i in range(6)]).reshape(2, 3, 5, 8)
    assert np.array_equal(ks.view(np.uint16), want.numpy().view(np.uint16))
    assert vs.shape == ks.shape
