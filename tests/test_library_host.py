"""Host-side checks of libspecache (no GPU): the shared object loads, exports
every function include/specache.h declares, validates arguments before any HIP
call, and sizes its buffers as documented."""
from __future__ import annotations

import ctypes
import json
import os
import re

import numpy as np
import pytest

from decode_attention_bit_kivi_amd import _lib
from decode_attention_bit_kivi_amd.api import lowbit_sizes

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "specache.h")


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def _declared_functions():
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(specache_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_function(lib):
    declared = _declared_functions()
    assert set(declared) == set(_lib.EXPORTED)
    for name in declared:
        assert hasattr(lib, name), name


def test_abi_version_and_status_strings(lib):
    assert lib.specache_abi_version() == _lib.ABI_VERSION
    for code in range(7):
        assert lib.specache_status_string(code)
    assert lib.specache_status_string(99) == b"unknown status"


def _shape(**kw):
    base = dict(batch=1, n_q_heads=8, n_kv_heads=2, head_dim=128, seq_len=1024, bits=1, group=32)
    base.update(kw)
    return _lib.Shape(**base)


@pytest.mark.parametrize("bad,status", [
    (dict(seq_len=1000), _lib.SPECACHE_ERR_INVALID),          # not a multiple of 32
    (dict(seq_capacity=992), _lib.SPECACHE_ERR_INVALID),      # capacity below seq_len
    (dict(seq_capacity=1040), _lib.SPECACHE_ERR_INVALID),     # capacity not a multiple of 32
    (dict(bits=3), _lib.SPECACHE_ERR_INVALID),
    (dict(n_q_heads=7), _lib.SPECACHE_ERR_INVALID),           # not a multiple of Hkv
    (dict(head_dim=96), _lib.SPECACHE_ERR_UNSUPPORTED),
    (dict(group=16), _lib.SPECACHE_ERR_UNSUPPORTED),
    (dict(group=64, seq_len=1056), _lib.SPECACHE_ERR_INVALID),  # not whole 64-token groups
    (dict(batch=0), _lib.SPECACHE_ERR_INVALID),
    (dict(n_q_heads=2 * 17), _lib.SPECACHE_ERR_UNSUPPORTED),  # G = 17 > 16
])
def test_shape_validation(lib, bad, status):
    s = _shape(**bad)
    lb = _lib.LowBit(1, 1, 1, 1)
    assert lib.specache_quantize_pack(ctypes.byref(s), 1, 1, ctypes.byref(lb), None) == status
    assert lib.specache_score_topk_workspace_size(ctypes.byref(s), 2, 8) == 0
    assert lib.specache_decode_attn_workspace_size(ctypes.byref(s), 2, 8, 0) == 0


def test_argument_validation(lib):
    s = _shape()
    lb = _lib.LowBit(1, 1, 1, 1)
    null_lb = _lib.LowBit(1, 0, 1, 1)
    ws = lib.specache_score_topk_workspace_size(ctypes.byref(s), 2, 16)
    assert ws > 0
    call = lambda **kw: lib.specache_score_topk(  # noqa: E731
        ctypes.byref(s), kw.get("q", 1), kw.get("T", 2), kw.get("row", 1), ctypes.byref(kw.get("lb", lb)),
        kw.get("scale", 0.1), kw.get("k", 16), kw.get("idx", 1), None, kw.get("ws", 1), kw.get("wsb", ws), None)
    assert call(k=0) == _lib.SPECACHE_ERR_INVALID
    assert call(k=1025) == _lib.SPECACHE_ERR_INVALID
    assert call(row=2) == _lib.SPECACHE_ERR_INVALID
    assert call(T=3) == _lib.SPECACHE_ERR_INVALID
    assert call(q=0) == _lib.SPECACHE_ERR_INVALID
    assert call(lb=null_lb) == _lib.SPECACHE_ERR_INVALID
    assert call(idx=0) == _lib.SPECACHE_ERR_INVALID
    assert call(scale=0.0) == _lib.SPECACHE_ERR_INVALID
    assert call(ws=0) == _lib.SPECACHE_ERR_WORKSPACE
    assert call(wsb=ws - 1) == _lib.SPECACHE_ERR_WORKSPACE

    wa = lib.specache_decode_attn_workspace_size(ctypes.byref(s), 2, 16, 2)
    assert wa > 0
    attn = lambda **kw: lib.specache_decode_attn(  # noqa: E731
        ctypes.byref(s), 1, kw.get("T", 2), ctypes.byref(lb), kw.get("idx", 1), kw.get("k", 16), 1, 1,
        kw.get("kt", 1), 1, kw.get("R", 2), 0.1, 1, kw.get("ws", 1), kw.get("wsb", wa), None)
    assert attn(k=-1) == _lib.SPECACHE_ERR_INVALID
    assert attn(k=1025) == _lib.SPECACHE_ERR_INVALID
    assert attn(idx=0) == _lib.SPECACHE_ERR_INVALID
    assert attn(R=65) == _lib.SPECACHE_ERR_INVALID
    assert attn(kt=0) == _lib.SPECACHE_ERR_INVALID
    assert attn(wsb=wa - 1) == _lib.SPECACHE_ERR_WORKSPACE
    s16 = _shape(n_q_heads=2 * 16)          # G = 16, T = 2 -> 32 rows
    assert lib.specache_decode_attn_workspace_size(ctypes.byref(s16), 2, 0, 0) == 0
    assert lib.specache_decode_attn_workspace_size(ctypes.byref(s16), 1, 0, 0) > 0

    wf = lib.specache_decode_step_workspace_size(ctypes.byref(s), 2, 16, 2, 16)
    # the fused step also holds the speculative row's logits: 4 bytes per (query head, position)
    assert wf >= wa + 4 * s.batch * s.n_q_heads * s.seq_len
    assert lib.specache_decode_step_workspace_size(ctypes.byref(s), 2, 16, 2, 0) == 0
    assert lib.specache_decode_step_workspace_size(ctypes.byref(s), 2, 16, 2, s.seq_len + 1) == 0
    assert lib.specache_decode_step_workspace_size(ctypes.byref(s16), 2, 0, 0, 8) == 0
    step = lambda **kw: lib.specache_decode_step(  # noqa: E731
        ctypes.byref(s), 1, kw.get("T", 2), kw.get("row", 1), kw.get("mixed", 0), ctypes.byref(lb), kw.get("idx", 1),
        kw.get("k", 16), 1, 1, 1, 1, 2, 0.1, 1, kw.get("kn", 16), kw.get("idx_next", 1), None,
        kw.get("ws", 1), kw.get("wsb", wf), None)
    assert step(kn=0) == _lib.SPECACHE_ERR_INVALID
    assert step(kn=s.seq_len + 1) == _lib.SPECACHE_ERR_INVALID
    assert step(row=2) == _lib.SPECACHE_ERR_INVALID
    assert step(row=-1) == _lib.SPECACHE_ERR_INVALID
    assert step(T=1, row=1) == _lib.SPECACHE_ERR_INVALID
    assert step(idx_next=0) == _lib.SPECACHE_ERR_INVALID
    assert step(mixed=2) == _lib.SPECACHE_ERR_INVALID
    assert step(idx=0) == _lib.SPECACHE_ERR_INVALID
    assert step(ws=0) == _lib.SPECACHE_ERR_WORKSPACE
    assert step(wsb=wf - 1) == _lib.SPECACHE_ERR_WORKSPACE

    reuse = lambda **kw: lib.specache_gather_reuse(  # noqa: E731
        ctypes.byref(s), kw.get("idx", 1), kw.get("k", 8), kw.get("prev", 1), kw.get("kp", 8), kw.get("kprev", 2),
        kw.get("vprev", 3), kw.get("ks", 4), kw.get("vs", 5), kw.get("fetch", 6), None)
    assert reuse(k=-1) == _lib.SPECACHE_ERR_INVALID
    assert reuse(kp=s.seq_len + 1) == _lib.SPECACHE_ERR_INVALID
    assert reuse(idx=0) == _lib.SPECACHE_ERR_INVALID
    assert reuse(fetch=0) == _lib.SPECACHE_ERR_INVALID
    assert reuse(prev=0) == _lib.SPECACHE_ERR_INVALID
    assert reuse(ks=2) == _lib.SPECACHE_ERR_INVALID          # output aliases the previous rows
    assert reuse(k=0) == _lib.SPECACHE_OK                     # nothing to do
    missing = lambda **kw: lib.specache_gather_fp16_missing(  # noqa: E731
        ctypes.byref(s), kw.get("fetch", 1), kw.get("k", 8), kw.get("src", 1), 1, 1, 1, None)
    assert missing(k=-1) == _lib.SPECACHE_ERR_INVALID
    assert missing(fetch=0) == _lib.SPECACHE_ERR_INVALID
    assert missing(k=0) == _lib.SPECACHE_OK

    assert lib.specache_gather_fp16(ctypes.byref(s), 1, -1, 1, 1, 1, 1, None) == _lib.SPECACHE_ERR_INVALID
    assert lib.specache_gather_fp16(ctypes.byref(s), 0, 4, 1, 1, 1, 1, None) == _lib.SPECACHE_ERR_INVALID
    assert lib.specache_gather_fp16(ctypes.byref(s), 1, 0, 0, 0, 0, 0, None) == _lib.SPECACHE_OK  # k = 0: no-op


@pytest.mark.parametrize("bits", [1, 2])
@pytest.mark.parametrize("D", [64, 128])
def test_lowbit_bytes_match_layout(lib, bits, D):
    s = _shape(head_dim=D, bits=bits, batch=3, n_kv_heads=2, seq_len=4096)
    out = [ctypes.c_size_t() for _ in range(4)]
    total = lib.specache_lowbit_bytes(ctypes.byref(s), *[ctypes.byref(o) for o in out])
    want = [4 * np.prod(lowbit_sizes(3, 2, 4096, D, bits)[0]), 2 * np.prod(lowbit_sizes(3, 2, 4096, D, bits)[1]),
            4 * np.prod(lowbit_sizes(3, 2, 4096, D, bits)[2]), 2 * np.prod(lowbit_sizes(3, 2, 4096, D, bits)[3])]
    assert [o.value for o in out] == want and total == sum(want)
    per_pos = total / (3 * 2 * 4096)
    assert per_pos == 2 * (bits * D / 8 + 4 * D / 32)


def test_capacity_sizes_the_buffers_and_bounds_append_and_offload(lib):
    s = _shape(seq_len=1024, seq_capacity=4096, batch=2)
    tight = _shape(seq_len=4096, batch=2)
    assert lib.specache_lowbit_bytes(ctypes.byref(s), None, None, None, None) == \
        lib.specache_lowbit_bytes(ctypes.byref(tight), None, None, None, None)
    lb = _lib.LowBit(1, 1, 1, 1)
    app = lambda n, shape=s: lib.specache_quantize_append(ctypes.byref(shape), 1, 1, n, ctypes.byref(lb), None)  # noqa: E731
    assert app(48) == _lib.SPECACHE_ERR_INVALID                 # not whole groups
    assert app(3072 + 32) == _lib.SPECACHE_ERR_INVALID          # past the capacity
    assert app(-32) == _lib.SPECACHE_ERR_INVALID
    assert app(0) == _lib.SPECACHE_OK
    assert app(32, _shape(seq_len=1024)) == _lib.SPECACHE_ERR_INVALID   # no room without a capacity
    off = lambda n, pos: lib.specache_offload_fp16(ctypes.byref(s), 1, 1, n, pos, 1, 1, None)  # noqa: E731
    assert off(1, 4096) == _lib.SPECACHE_ERR_INVALID
    assert off(2, 4095) == _lib.SPECACHE_ERR_INVALID
    assert off(1, -1) == _lib.SPECACHE_ERR_INVALID
    assert off(0, 0) == _lib.SPECACHE_OK


@pytest.mark.parametrize("group", [32, 64])
def test_group_sizes_the_metadata(lib, group):
    s = _shape(group=group, batch=2, seq_len=2048)
    out = [ctypes.c_size_t() for _ in range(4)]
    lib.specache_lowbit_bytes(ctypes.byref(s), *[ctypes.byref(o) for o in out])
    shapes = lowbit_sizes(2, 2, 2048, 128, 1, group=group)
    assert [o.value for o in out] == [4 * np.prod(shapes[0]), 2 * np.prod(shapes[1]),
                                      4 * np.prod(shapes[2]), 2 * np.prod(shapes[3])]
    # metadata: 2 float16 per key group per channel, 2 per value group per token
    assert out[1].value == 2 * 2 * (2048 // group) * 2 * 128 * 2
    assert out[3].value == 2 * 2 * 2048 * 2 * (128 // group) * 2


def test_mixed_bit_widths_size_the_value_planes(lib):
    kc, km, vc, vm = [ctypes.c_size_t() for _ in range(4)]
    s = _shape(bits=1, v_bits=2, batch=2, seq_len=2048)
    total = lib.specache_lowbit_bytes(ctypes.byref(s), ctypes.byref(kc), ctypes.byref(km), ctypes.byref(vc),
                                      ctypes.byref(vm))
    shapes = lowbit_sizes(2, 2, 2048, 128, 1, v_bits=2)
    assert [kc.value, km.value, vc.value, vm.value] == [4 * np.prod(shapes[0]), 2 * np.prod(shapes[1]),
                                                       4 * np.prod(shapes[2]), 2 * np.prod(shapes[3])]
    assert total / (2 * 2 * 2048) == (1 * 128 / 8 + 4 * 128 / 32) + (2 * 128 / 8 + 4 * 128 / 32)
    assert lib.specache_lowbit_bytes(ctypes.byref(_shape(v_bits=3)), None, None, None, None) == 0


def test_compression_ratio_matches_pages():
    """SpeCache summary, Figure 4 caption: at g = 32 and 1 bit the GPU copy is 0.13
    (Mistral, 32K) and 0.14 (LLaMA-3, 8K) of the 16-bit cache, with the §4 setup of
    64 residual and top-64 fetched 16-bit rows.  Our metadata format (float16 z and s
    per group of 32) reproduces both numbers."""
    with open(os.path.join(ROOT, "tests", "golden", "pages_figures.json")) as f:
        fig = json.load(f)["compression_ratio"]
    lib = _lib.load()
    for case in fig["cases"]:
        N = case["context"]
        s = _shape(head_dim=128, bits=1, seq_len=32 * ((N - fig["residual"]) // 32), n_kv_heads=1, batch=1)
        lowbit = lib.specache_lowbit_bytes(ctypes.byref(s), None, None, None, None)
        fp16_rows = (fig["residual"] + fig["top_k"]) * 2 * 128 * 2
        ratio = (lowbit + fp16_rows) / (N * 2 * 128 * 2)
        assert round(ratio, 2) == case["ratio"], (N, ratio)


def test_flag_argument_validation(lib):
    """Null flag or timeout words and a zero bound are refused before any launch."""
    inv = _lib.SPECACHE_ERR_INVALID
    assert lib.specache_flag_set(None, 1, None) == inv
    assert lib.specache_flag_wait(None, 1, 100, 1, None) == inv
    assert lib.specache_flag_wait(1, 1, 100, None, None) == inv
    assert lib.specache_flag_wait(1, 1, 0, 1, None) == inv


def test_noalloc_step_refuses_sizes_beyond_its_scratch_before_any_hip_call(lib):
    """The no-allocation decode step checks the scratch it would need against its static array
    on the host: too large -> SPECACHE_ERR_TOO_LARGE, bad arguments -> their own status."""
    big = _shape(batch=32, n_q_heads=32, n_kv_heads=8, seq_len=32768)
    need = lib.specache_decode_step_workspace_size(ctypes.byref(big), 2, 328, 0, 328)
    assert need > _lib.NOALLOC_SCRATCH_BYTES
    lb = _lib.LowBit(1, 1, 1, 1)
    call = lambda s, k_next=328, T=2: lib.specache_decode_step_noalloc(  # noqa: E731
        ctypes.byref(s), 1, T, 1, 0, ctypes.byref(lb), 1, 328, 1, 1, None, None, 0, 0.1, 1, k_next, 1, None, None)
    assert call(big) == _lib.SPECACHE_ERR_TOO_LARGE
    small = _shape(batch=2, n_q_heads=32, n_kv_heads=8, seq_len=4096)
    assert call(small, k_next=0) == _lib.SPECACHE_ERR_INVALID        # k_next < 1: invalid, not "too large"
    assert call(small, T=3) == _lib.SPECACHE_ERR_INVALID
    assert lib.specache_decode_step_workspace_size(ctypes.byref(small), 2, 328, 0, 328) <= _lib.NOALLOC_SCRATCH_BYTES
    # the header's example: the 32K step at batch 16 (the 32-layer workload's shape) fits
    layers32 = _shape(batch=16, n_q_heads=32, n_kv_heads=8, seq_len=32768)
    assert lib.specache_decode_step_workspace_size(ctypes.byref(layers32), 2, 328, 0, 328) <= _lib.NOALLOC_SCRATCH_BYTES
