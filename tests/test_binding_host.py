"""Host checks of the Python binding's argument validation (no GPU).

The C ABI takes raw pointers, so an operand whose shape disagrees with the cache or the
index set would make a kernel read or write out of bounds.  The binding checks every
operand's dtype, shape and layout first and the device last, before anything reaches the
library: with host tensors, a wrong shape must therefore raise a shape error (and a correct
one get as far as the device check)."""
import pytest
import torch

from decode_attention_bit_kivi_amd import (
    decode_attn, decode_attn_fp16, decode_step, empty_cache, gather_fp16, gather_fp16_missing, gather_reuse,
    offload_fp16, quantize_append, quantize_pack, score_topk,
)

B, HQ, HKV, N, D, T, K = 2, 8, 2, 256, 64, 2, 16


def cache():
    return empty_cache(B, HKV, N, D, 1, device="cpu")


def h(*shape, dtype=torch.float16):
    return torch.zeros(shape, dtype=dtype)


def q():
    return h(B, HQ, T, D)


def idx(k=K, b=B, hk=HKV):
    return torch.zeros((b, hk, k), dtype=torch.int32)


def _shape_error(fn, name):
    with pytest.raises(ValueError, match=rf"{name} must have"):
        fn()


def _device_error(fn):
    with pytest.raises(ValueError, match="GPU tensor"):
        fn()


def test_well_formed_host_operands_reach_the_device_check():
    c = cache()
    _device_error(lambda: score_topk(q(), c, K))
    _device_error(lambda: decode_attn(q(), c, idx(), h(B, HKV, K, D), h(B, HKV, K, D)))
    _device_error(lambda: decode_step(q(), c, K, idx=idx(), k_sel=h(B, HKV, K, D), v_sel=h(B, HKV, K, D),
                                      k_tail=h(B, HKV, 2, D), v_tail=h(B, HKV, 2, D)))
    _device_error(lambda: gather_fp16(idx(), h(B, HKV, N, D), h(B, HKV, N, D)))
    _device_error(lambda: quantize_pack(h(B, HKV, N, D), h(B, HKV, N, D), 1))


@pytest.mark.parametrize("case", [
    "q_batch", "q_dim", "q_heads", "idx_out", "rank_key_out",
])
def test_score_topk_shape_mismatches(case):
    c = cache()
    args = dict(q16=q(), cache=c, k=K)
    name = {"q_batch": "q16", "q_dim": "q16", "q_heads": "q16", "idx_out": "idx_out",
            "rank_key_out": "rank_key_out"}[case]
    if case == "q_batch":
        args["q16"] = h(B + 1, HQ, T, D)
    elif case == "q_dim":
        args["q16"] = h(B, HQ, T, 2 * D)
    elif case == "q_heads":
        args["q16"] = h(B, 3, T, D)
        with pytest.raises(ValueError, match="multiple"):
            score_topk(**args)
        return
    elif case == "idx_out":
        args["idx_out"] = idx(K + 1)
    elif case == "rank_key_out":
        args["rank_key_out"] = h(B, HKV, N - 32, dtype=torch.float32)
    _shape_error(lambda: score_topk(**args), name)


_ATTN_CASES = ["idx_batch", "k_sel_rows", "v_sel_dim", "k_tail_dim", "v_tail_len", "out"]


@pytest.mark.parametrize("fn,case", [("decode_attn", c) for c in _ATTN_CASES] +
                         [("decode_step", c) for c in _ATTN_CASES + ["idx_next_out", "rank_key_out"]])
def test_attention_shape_mismatches(fn, case):
    c = cache()
    ops = dict(idx=idx(), k_sel=h(B, HKV, K, D), v_sel=h(B, HKV, K, D), k_tail=h(B, HKV, 3, D),
               v_tail=h(B, HKV, 3, D))
    extra = {}
    name = None
    if case == "idx_batch":
        ops["idx"], name = idx(b=B - 1), "idx"
    elif case == "k_sel_rows":
        ops["k_sel"], name = h(B, HKV, K - 1, D), "k_sel"
    elif case == "v_sel_dim":
        ops["v_sel"], name = h(B, HKV, K, D // 2), "v_sel"
    elif case == "k_tail_dim":
        ops["k_tail"], name = h(B, HKV, 3, D + 8), "k_tail"
    elif case == "v_tail_len":
        ops["v_tail"], name = h(B, HKV, 2, D), "v_tail"
    elif case == "out":
        extra["out"], name = h(B, HQ, 1, D), "out"
    elif case == "idx_next_out":
        extra["idx_next_out"], name = idx(K - 2), "idx_next_out"
    elif case == "rank_key_out":
        extra["rank_key_out"], name = h(B, HKV, N + 32, dtype=torch.float32), "rank_key_out"
    if fn == "decode_attn":
        call = lambda: decode_attn(q(), c, **ops, **extra)  # noqa: E731
    else:
        call = lambda: decode_step(q(), c, K, **ops, **extra)  # noqa: E731
    _shape_error(call, name)


@pytest.mark.parametrize("case", ["idx_heads", "v_src", "k_sel", "v_sel"])
def test_gather_shape_mismatches(case):
    src_k, src_v, i, ks, vs = h(B, HKV, N, D), h(B, HKV, N, D), idx(), None, None
    if case == "idx_heads":
        i = idx(hk=HKV + 1)
    elif case == "v_src":
        src_v = h(B, HKV, N - 32, D)
    elif case == "k_sel":
        ks = h(B, HKV, K, D + 1)
    elif case == "v_sel":
        vs = h(B, HKV, K + 1, D)
    name = {"idx_heads": "idx", "v_src": "v16_src"}.get(case, case)
    _shape_error(lambda: gather_fp16(i, src_k, src_v, k_sel=ks, v_sel=vs), name)


@pytest.mark.parametrize("case", ["idx_prev", "k_sel_prev", "v_sel_prev", "k_sel", "fetch_idx"])
def test_reuse_shape_mismatches(case):
    i, ip = idx(), idx(K + 4)
    kp, vp = h(B, HKV, K + 4, D), h(B, HKV, K + 4, D)
    kw = {}
    if case == "idx_prev":
        ip = idx(K + 4, b=B + 1)
    elif case == "k_sel_prev":
        kp = h(B, HKV, K, D)
    elif case == "v_sel_prev":
        vp = h(B, HKV, K + 4, D - 8)
    elif case == "k_sel":
        kw["k_sel"] = h(B, HKV, K + 4, D)
    elif case == "fetch_idx":
        kw["fetch_idx"] = idx(K + 1)
    _shape_error(lambda: gather_reuse(i, ip, kp, vp, N, **kw), case)


def test_missing_fetch_and_cache_update_shape_mismatches():
    src = h(B, HKV, N, D)
    _shape_error(lambda: gather_fp16_missing(idx(), src, src, h(B, HKV, K, D), h(B, HKV, K - 1, D)), "v_sel")
    _shape_error(lambda: gather_fp16_missing(idx(b=1), src, src, h(B, HKV, K, D), h(B, HKV, K, D)), "fetch_idx")
    c = cache()
    _shape_error(lambda: quantize_append(c, h(B, HKV + 1, 32, D), h(B, HKV + 1, 32, D)), "k16_new")
    _shape_error(lambda: quantize_append(c, h(B, HKV, 32, D), h(B, HKV, 64, D)), "v16_new")
    _shape_error(lambda: offload_fp16(h(B, HKV, 32, D), h(B, HKV, 32, D), src, h(B, HKV, N, 2 * D), 0), "v16_cache")
    _shape_error(lambda: offload_fp16(h(B, HKV, 32, D - 1), h(B, HKV, 32, D), src, src, 0), "k16_new")
    _shape_error(lambda: quantize_pack(h(B, HKV, N, D), h(B, HKV, N, D // 2), 1), "v16")
    _shape_error(lambda: decode_attn_fp16(h(B, HQ, T, D), src, h(B, HKV, N - 32, D)), "v16")
    _shape_error(lambda: decode_attn_fp16(h(B + 1, HQ, T, D), src, src), "q16")


def test_cache_buffers_are_checked():
    c = cache()
    c.k_codes = torch.zeros((B, HKV, N // 2, 1, D // 32), dtype=torch.int32)
    _shape_error(lambda: score_topk(q(), c, K), r"cache\.k_codes")
    c = cache()
    c.seq_len = N + 32
    with pytest.raises(ValueError, match="capacity"):
        decode_attn(q(), c)
    c = cache()
    with pytest.raises(ValueError, match="out cache"):
        quantize_pack(h(B, HKV, N, D), h(B, HKV, N, D), 2, out=c)
