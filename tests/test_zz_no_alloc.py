"""The no-allocation decode step (specache_decode_step_noalloc, through the C ABI) against the
workspace decode step (specache_decode_step) on the same inputs and stream: the same kernels,
so the outputs must agree bit for bit (beyond the 2e-3 attention bar) and the next selections
exactly.  Two calls in a row share the library's static scratch array; the second has a smaller
input, so any state the first left behind would show.  A problem too large for the array is
refused before anything is enqueued."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from decode_attention_bit_kivi_amd import (
    SpecacheError, decode_step, decode_step_noalloc, decode_step_workspace_size, quantize_pack,
)
from decode_attention_bit_kivi_amd import _lib
from workloads import generate_all, get_config

pytestmark = pytest.mark.gpu


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def _case(cfg, seed):
    K, V, Q, _, KT, VT = generate_all(cfg)
    cache = quantize_pack(_dev(K), _dev(V), cfg.bits)
    rng = np.random.default_rng(seed)
    B, H, N, k = cfg.batch, cfg.n_kv_heads, cfg.seq_len, cfg.top_k
    idx = np.stack([np.stack([np.sort(rng.choice(N, k, replace=False)) for _ in range(H)]) for _ in range(B)])
    idx = _dev(idx.astype(np.int32))
    ks = _dev(rng.standard_normal((B, H, k, cfg.head_dim)).astype(np.float16))
    vs = _dev(rng.standard_normal((B, H, k, cfg.head_dim)).astype(np.float16))
    kt = None if KT is None else _dev(KT)
    vt = None if VT is None else _dev(VT)
    return dict(q16=_dev(Q), cache=cache, k_next=k, idx=idx, k_sel=ks, v_sel=vs, k_tail=kt, v_tail=vt)


def _outputs(c):
    B, H, N = c["cache"].batch, c["cache"].n_kv_heads, c["cache"].seq_len
    return (torch.full_like(c["q16"], float("nan")),
            torch.full((B, H, c["k_next"]), -7, dtype=torch.int32, device="cuda"),
            torch.full((B, H, N), float("nan"), dtype=torch.float32, device="cuda"))


@pytest.mark.parametrize("mixed", [False, True])
def test_noalloc_step_equals_workspace_step_twice_in_a_row(gpu, mixed):
    big = _case(get_config("llama8k").with_(batch=2, bits=1, seed=3), 5)            # 8192 positions, 16 slices
    small = _case(get_config("tiny").with_(tail_len=2, top_k=24, seed=4), 6)        # 512 positions, D 64
    want = []
    for c in (big, small):
        o, nx, rk = _outputs(c)
        decode_step(**c, rank_mixed=mixed, out=o, idx_next_out=nx, rank_key_out=rk)
        want.append((o, nx, rk))
    got = []
    for c in (big, small):                       # back to back on one stream, the larger first
        o, nx, rk = _outputs(c)
        decode_step_noalloc(**c, rank_mixed=mixed, out=o, idx_next_out=nx, rank_key_out=rk)
        got.append((o, nx, rk))
    torch.cuda.synchronize()
    for (wo, wn, wr), (go, gn, gr) in zip(want, got):
        assert torch.equal(go.view(torch.int16), wo.view(torch.int16))
        assert torch.equal(gn, wn)
        assert torch.equal(gr.view(torch.int32), wr.view(torch.int32))
    # and once more on the larger input after the smaller one
    o, nx, rk = _outputs(big)
    decode_step_noalloc(**big, rank_mixed=mixed, out=o, idx_next_out=nx, rank_key_out=rk)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), want[0][0].view(torch.int16)) and torch.equal(nx, want[0][1])


def test_noalloc_refuses_a_problem_beyond_its_scratch(gpu):
    cfg = get_config("llama8k").with_(batch=2, bits=1, seq_len=512)
    c = _case(cfg, 1)
    # a 32K-context step at batch 32 needs more than the static array holds
    from decode_attention_bit_kivi_amd import empty_cache
    big = empty_cache(32, 8, 32768, 128, 1, device="cuda")
    assert decode_step_workspace_size(big, 32, 2, 328, 0, 328) > _lib.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((32, 32, 2, 128), dtype=torch.float16, device="cuda")
    out = torch.empty_like(q)
    nx = torch.empty((32, 8, 328), dtype=torch.int32, device="cuda")
    with pytest.raises(SpecacheError) as e:
        decode_step_noalloc(q, big, 328, out=out, idx_next_out=nx)
    assert e.value.status == _lib.SPECACHE_ERR_TOO_LARGE
    # the refusal left nothing behind: the next call still matches the workspace step
    o1, n1, _ = _outputs(c)
    o2, n2, _ = _outputs(c)
    decode_step(**c, out=o1, idx_next_out=n1)
    decode_step_noalloc(**c, out=o2, idx_next_out=n2)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(n1, n2)
