"""Independent reader of the C' buffer layouts documented in include/specache.h.

Test infrastructure: turns the packed device buffers (copied to numpy) back
into per-element codes and per-group float16 zero-points / scales, so they can
be compared element by element with the oracle's.  Written from the header's
prose, not from the kernels.
"""
from __future__ import annotations

import numpy as np

# bit i of a packed word <-> element 2*(i mod 16) + (i div 16)
BIT_ELEM = np.array([2 * (i % 16) + i // 16 for i in range(32)])


def _planes_to_codes(words: np.ndarray, bits_axis: int) -> np.ndarray:
    """uint32 words with a plane axis -> codes by bit position, plane axis removed, bit axis last."""
    w = words.astype(np.uint64)
    bitv = (w[..., None] >> np.arange(32, dtype=np.uint64)) & np.uint64(1)     # [..., 32]
    bitv = np.moveaxis(bitv, bits_axis, -1)                                     # plane axis last
    weights = (np.uint64(1) << np.arange(bitv.shape[-1], dtype=np.uint64))
    return (bitv * weights).sum(axis=-1).astype(np.uint8)


def unpack_keys(k_codes: np.ndarray, k_meta: np.ndarray, bits: int):
    """k_codes uint32 [B, Hkv, N, bits, W]; k_meta float16 [B, Hkv, N/32, 2, D]
    -> codes [B, Hkv, N, D] uint8, z, s [B, Hkv, N/32, D] float16."""
    B, Hkv, N, nb, W = k_codes.shape
    assert nb == bits
    by_bit = _planes_to_codes(k_codes.view(np.uint32), bits_axis=3)   # [B, Hkv, N, W, 32]
    codes = np.empty((B, Hkv, N, W * 32), dtype=np.uint8)
    for w in range(W):
        codes[..., 32 * w + BIT_ELEM] = by_bit[..., w, :]
    return codes, k_meta[:, :, :, 0, :], k_meta[:, :, :, 1, :]


def unpack_values(v_codes: np.ndarray, v_meta: np.ndarray, bits: int):
    """v_codes uint32 [B, Hkv, N/32, bits, D]; v_meta float16 [B, Hkv, N/32, 2, W, 32]
    -> codes [B, Hkv, N, D] uint8, z, s [B, Hkv, N, W] float16."""
    B, Hkv, nblk, nb, D = v_codes.shape
    assert nb == bits
    by_bit = _planes_to_codes(v_codes.view(np.uint32), bits_axis=3)   # [B, Hkv, nblk, D, 32]
    tok = np.empty((B, Hkv, nblk, 32, D), dtype=np.uint8)
    tok[:, :, :, BIT_ELEM, :] = np.moveaxis(by_bit, -1, 3)
    codes = tok.reshape(B, Hkv, nblk * 32, D)
    z = np.moveaxis(v_meta[:, :, :, 0], -1, 3).reshape(B, Hkv, nblk * 32, -1)   # [B,Hkv,nblk,32,W]
    s = np.moveaxis(v_meta[:, :, :, 1], -1, 3).reshape(B, Hkv, nblk * 32, -1)
    return codes, z, s
