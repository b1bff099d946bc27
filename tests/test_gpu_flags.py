"""GPU checks of the device-flag ordering between two streams (specache_flag_set /
specache_flag_wait), the overlapped loop's alternative to a queue barrier: the waiting
stream's later work sees what the setting stream wrote before the set, and a wait whose flag
is never set ends at its bound and says so."""
from __future__ import annotations

import pytest
import torch

from decode_attention_bit_kivi_amd import ComputeStream, GatherStream, flag_set, flag_wait

pytestmark = pytest.mark.gpu


def test_flag_orders_the_waiting_stream_after_the_setter(gpu):
    """The consumer is enqueued first, so its stream really waits: its copy runs after the
    producer's writes, on the library's two CU-limited streams (each its own hardware queue)."""
    gs, cs = GatherStream(8), ComputeStream(8)
    try:
        n = 1 << 24
        src = torch.arange(n, dtype=torch.int32, device="cuda")
        mid = torch.zeros_like(src)
        out = torch.zeros_like(src)
        flag = torch.zeros(1, dtype=torch.int32, device="cuda")
        tmo = torch.zeros_like(flag)
        torch.cuda.synchronize()
        for seq in (1, 2):  # the same flag serves successive rounds with growing numbers
            flag_wait(flag, seq, tmo, max_wait_us=2_000_000, stream=gs)
            with torch.cuda.stream(gs.torch):
                out.copy_(mid)
            with torch.cuda.stream(cs.torch):
                for _ in range(8):
                    mid.copy_(src)
                mid.add_(seq)
            flag_set(flag, seq, stream=cs)
            torch.cuda.synchronize()
            assert tmo.item() == 0
            assert torch.equal(out, src + seq)
    finally:
        gs.close()
        cs.close()


def test_flag_wait_ends_at_its_bound(gpu):
    """Forced from the host with a short bound: a flag below the value ends the wait at the
    bound (one timeout counted); a flag at or past it (also across the 2^32 wrap) does not."""
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    tmo = torch.zeros_like(flag)
    flag_wait(flag, 7, tmo, max_wait_us=200)
    torch.cuda.synchronize()
    assert tmo.item() == 1
    flag_set(flag, 7)
    flag_wait(flag, 7, tmo, max_wait_us=200)
    flag_wait(flag, 5, tmo, max_wait_us=200)
    torch.cuda.synchronize()
    assert tmo.item() == 1 and flag.item() == 7
    flag_set(flag, 3)                                  # 3 is 5 past 2^32 - 2
    flag_wait(flag, 0xFFFFFFFE, tmo, max_wait_us=200)
    flag_wait(flag, 4, tmo, max_wait_us=200)           # not reached: a second timeout
    torch.cuda.synchronize()
    assert tmo.item() == 2


def test_pinned_tensor_freed_after_its_copy_stream_is_closed(gpu):
    """torch's pinned-host allocator records an event on every stream a pinned block was copied
    on when the block is freed; close() therefore retires a library stream without releasing
    it, so a pinned tensor copied on the stream may outlive the stream object."""
    import gc
    for cls in (GatherStream, ComputeStream):
        st = cls(16)
        pinned = torch.arange(1 << 20, dtype=torch.float32).pin_memory()
        dst = torch.empty(1 << 20, dtype=torch.float32, device="cuda")
        with torch.cuda.stream(st.torch):
            dst.copy_(pinned, non_blocking=True)
        st.close()
        assert st.handle is None
        del st, pinned
        gc.collect()
        torch.cuda.synchronize()
        assert torch.equal(dst.cpu(), torch.arange(1 << 20, dtype=torch.float32))
    # the freed pinned blocks are reused by later allocations and copies
    again = torch.ones(1 << 20, dtype=torch.float32).pin_memory()
    assert float(again.cuda().sum().item()) == float(1 << 20)
