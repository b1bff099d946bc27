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
