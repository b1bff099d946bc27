"""Oracle quantizer: KIVI grouping with SpeCache's 1-bit zero-point and scale.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What it follows:
  * [SpeCache] §3 "original KIVI quantization": Q(X) = round((X - z_X) / s_X),
    X' = Q(X) * s_X + z_X, with z_X = min X and s_X = (max X - min X) / (2^B - 1);
    the rounding the page names is ordinary round-to-nearest, read as round half up.
  * [SpeCache] §3 "improved 1-bit quantization" (also the quick-read equation):
    at one bit, z_X = (3 min X + max X) / 4 and s_X = (max X - min X) / 2, so the
    two codes land on the midpoints of [min, mid) and (mid, max].
  * [SemKV] §2.1: KIVI quantizes keys per channel and values per token; groups
    of g = 32 consecutive elements ([SpeCache] §4 uses g = 32 and 64).

Readings where the pages are silent (all listed in the design notes):
  * z and s are stored as float16 (round-to-nearest-even), -0 stored as +0; the
    encoder uses the stored float16 values, so encoder and decoder agree.
  * z, s are computed in float32 from the float16 inputs in the order the
    equations are written: 1 bit: t = 3*min (exact), u = t + max, z = u * 0.25;
    d = max - min, s = d * 0.5.  B bits (B = 2): z = min, s = d / (2^B - 1), a
    correctly rounded division.
  * q = fl32(fl32(x - z16) / s16); code = clamp(floor(q + 1/2), 0, 2^B - 1)
    ("round half up", taken exactly); a group with s16 == 0 gets code 0.
"""
from __future__ import annotations

import numpy as np


def zero_point_scale(mn: np.ndarray, mx: np.ndarray, bits: int):
    """float16 (z, s) of groups with minimum `mn` and maximum `mx` (float16/float32)."""
    if bits not in (1, 2):
        raise ValueError("bits must be 1 or 2")
    mn = np.asarray(mn, dtype=np.float32)
    mx = np.asarray(mx, dtype=np.float32)
    if bits == 1:
        # [SpeCache] §3, improved 1-bit: z = (3 min + max) / 4, s = (max - min) / 2
        t = np.float32(3.0) * mn                      # exact: 11-bit mantissa times 3
        u = t + mx                                    # float32 RNE
        z = u * np.float32(0.25)                      # exact scaling
        s = (mx - mn) * np.float32(0.5)
    else:
        # [SpeCache] §3, original KIVI: z = min, s = (max - min) / (2^B - 1)
        z = mn
        s = (mx - mn) / np.float32((1 << bits) - 1)
    z16 = np.asarray(z, dtype=np.float32).astype(np.float16)
    s16 = np.asarray(s, dtype=np.float32).astype(np.float16)
    z16 = np.where(z16 == 0, np.float16(0), z16)      # canonical +0
    s16 = np.where(s16 == 0, np.float16(0), s16)
    return z16, s16


def _codes(x: np.ndarray, z16: np.ndarray, s16: np.ndarray, bits: int) -> np.ndarray:
    """Round-half-up codes of float16 values x against broadcastable float16 (z, s)."""
    xf = x.astype(np.float32)
    zf = np.broadcast_to(z16.astype(np.float32), xf.shape)
    sf = np.broadcast_to(s16.astype(np.float32), xf.shape)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = (xf - zf) / sf                            # two float32 RNE steps
    qmax = (1 << bits) - 1
    code = np.floor(q.astype(np.float64) + 0.5)       # exact in float64
    code = np.where(sf == 0, 0.0, code)
    code = np.clip(np.nan_to_num(code, nan=0.0), 0, qmax)
    return code.astype(np.uint8)


def quantize_keys(k16: np.ndarray, bits: int, group: int = 32):
    """Per-channel key quantization ([SemKV] §2.1): each group is `group`
    consecutive tokens of one channel.

    k16: [..., N, D] float16, N a multiple of `group`.
    Returns codes [..., N, D] uint8, z16 and s16 [..., N/group, D] float16."""
    k16 = np.asarray(k16, dtype=np.float16)
    *lead, n, d = k16.shape
    if n % group:
        raise ValueError("N must be a multiple of the group size")
    xg = k16.reshape(*lead, n // group, group, d)
    z16, s16 = zero_point_scale(xg.min(axis=-2), xg.max(axis=-2), bits)
    codes = _codes(xg, z16[..., None, :], s16[..., None, :], bits)
    return codes.reshape(*lead, n, d), z16, s16


def quantize_values(v16: np.ndarray, bits: int, group: int = 32):
    """Per-token value quantization ([SemKV] §2.1): each group is `group`
    consecutive channels of one token.

    v16: [..., N, D] float16, D a multiple of `group`.
    Returns codes [..., N, D] uint8, z16 and s16 [..., N, D/group] float16."""
    v16 = np.asarray(v16, dtype=np.float16)
    *lead, n, d = v16.shape
    if d % group:
        raise ValueError("D must be a multiple of the group size")
    xg = v16.reshape(*lead, n, d // group, group)
    z16, s16 = zero_point_scale(xg.min(axis=-1), xg.max(axis=-1), bits)
    codes = _codes(xg, z16[..., None], s16[..., None], bits)
    return codes.reshape(*lead, n, d), z16, s16


def dequantize_keys(codes: np.ndarray, z16: np.ndarray, s16: np.ndarray, group: int = 32) -> np.ndarray:
    """X' = Q(X) * s_X + z_X ([SpeCache] §3), float64 (exact)."""
    *lead, n, d = codes.shape
    c = codes.astype(np.float64).reshape(*lead, n // group, group, d)
    out = c * s16.astype(np.float64)[..., None, :] + z16.astype(np.float64)[..., None, :]
    return out.reshape(*lead, n, d)


def dequantize_values(codes: np.ndarray, z16: np.ndarray, s16: np.ndarray, group: int = 32) -> np.ndarray:
    """X' = Q(X) * s_X + z_X ([SpeCache] §3), float64 (exact)."""
    *lead, n, d = codes.shape
    c = codes.astype(np.float64).reshape(*lead, n, d // group, group)
    out = c * s16.astype(np.float64)[..., None] + z16.astype(np.float64)[..., None]
    return out.reshape(*lead, n, d)
