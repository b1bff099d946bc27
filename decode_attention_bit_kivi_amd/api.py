"""Python binding of libspecache: the C-ABI calls on torch tensors.

Argument marshalling only -- every step of the path runs in the HIP kernels
behind include/specache.h.  torch provides device memory (outputs and
workspaces are torch allocations) and the current HIP stream.
"""
from __future__ import annotations

import ctypes
import math
from dataclasses import dataclass

import torch

from . import _lib


@dataclass
class LowBitCache:
    """C' of one layer: the four device buffers written by quantize_pack, laid out for
    `capacity` positions of which the first `seq_len` are in use."""
    k_codes: torch.Tensor   # uint32 [B, Hkv, Nc, bits, D/32]   (stored as int32)
    k_meta: torch.Tensor    # float16 [B, Hkv, Nc/32, 2, D]
    v_codes: torch.Tensor   # uint32 [B, Hkv, Nc/32, bits, D]
    v_meta: torch.Tensor    # float16 [B, Hkv, Nc/32, 2, D/32, 32]
    batch: int
    n_kv_heads: int
    seq_len: int
    head_dim: int
    bits: int
    group: int = 32
    capacity: int = 0       # 0: seq_len
    v_bits: int = 0         # bits of the value codes; 0: `bits` (then bits is both)

    def c_struct(self) -> _lib.LowBit:
        return _lib.LowBit(self.k_codes.data_ptr(), self.k_meta.data_ptr(),
                           self.v_codes.data_ptr(), self.v_meta.data_ptr())

    def shape(self, n_q_heads: int | None = None) -> _lib.Shape:
        return _lib.Shape(self.batch, n_q_heads or self.n_kv_heads, self.n_kv_heads, self.head_dim,
                          self.seq_len, self.bits, self.group, self.capacity or self.seq_len, self.v_bits or self.bits)

    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in (self.k_codes, self.k_meta, self.v_codes, self.v_meta))


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    if hasattr(stream, "handle"):       # GatherStream
        return stream.handle
    return int(stream)


def _need(t: torch.Tensor, name: str, dtype, ndim: int, cuda: bool = True):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if cuda and not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")


def lowbit_sizes(batch: int, n_kv_heads: int, seq_len: int, head_dim: int, bits: int, group: int = 32,
                 v_bits: int | None = None):
    """(k_codes, k_meta, v_codes, v_meta) element shapes of C' (see include/specache.h); bits
    of the keys, v_bits (default bits) of the values, quantization group 32 or 64."""
    nblk = seq_len // 32
    vb = v_bits or bits
    return ((batch, n_kv_heads, seq_len, bits, head_dim // 32), (batch, n_kv_heads, seq_len // group, 2, head_dim),
            (batch, n_kv_heads, nblk, vb, head_dim), (batch, n_kv_heads, nblk, 2, head_dim // group, 32))


def empty_cache(batch, n_kv_heads, seq_len, head_dim, bits, device="cuda", capacity: int | None = None,
                v_bits: int | None = None, group: int = 32) -> LowBitCache:
    cap = capacity or seq_len
    kc, km, vc, vm = lowbit_sizes(batch, n_kv_heads, cap, head_dim, bits, group=group, v_bits=v_bits)
    return LowBitCache(torch.empty(kc, dtype=torch.int32, device=device),
                       torch.empty(km, dtype=torch.float16, device=device),
                       torch.empty(vc, dtype=torch.int32, device=device),
                       torch.empty(vm, dtype=torch.float16, device=device),
                       batch, n_kv_heads, seq_len, head_dim, bits, group=group, capacity=cap,
                       v_bits=v_bits or bits)


def quantize_pack(k16: torch.Tensor, v16: torch.Tensor, bits: int, out: LowBitCache | None = None,
                  seq_len: int | None = None, stream=None, v_bits: int | None = None,
                  group: int = 32) -> LowBitCache:
    """specache_quantize_pack: K, V [B, Hkv, Nc, D] float16 (device) -> C' laid out for Nc
    positions, of which the first seq_len (default Nc) are quantized; keys with `bits`, values
    with `v_bits` (default `bits`), in groups of `group` (32 or 64) tokens / channels."""
    _need(k16, "k16", torch.float16, 4)
    _need(v16, "v16", torch.float16, 4)
    if k16.shape != v16.shape:
        raise ValueError("k16 and v16 must have the same shape")
    B, Hkv, Nc, D = k16.shape
    N = Nc if seq_len is None else int(seq_len)
    cache = out if out is not None else empty_cache(B, Hkv, N, D, bits, k16.device, capacity=Nc, v_bits=v_bits,
                                                    group=group)
    lib = _lib.load()
    if out is not None:
        cache.seq_len = N
    shape = cache.shape()
    if (cache.batch, cache.n_kv_heads, cache.capacity or cache.seq_len, cache.head_dim, cache.bits) != \
            (B, Hkv, Nc, D, bits):
        raise ValueError("out cache shape does not match the inputs")
    _lib.check(lib.specache_quantize_pack(ctypes.byref(shape), k16.data_ptr(), v16.data_ptr(),
                                          ctypes.byref(cache.c_struct()), _stream(stream)),
               "specache_quantize_pack")
    return cache


def quantize_append(cache: LowBitCache, k16_new: torch.Tensor, v16_new: torch.Tensor, stream=None) -> LowBitCache:
    """specache_quantize_append: quantize K, V [B, Hkv, n_new, D] (n_new a multiple of 32) into
    positions [seq_len, seq_len + n_new) of the cache; cache.seq_len grows by n_new."""
    _need(k16_new, "k16_new", torch.float16, 4)
    _need(v16_new, "v16_new", torch.float16, 4)
    if k16_new.shape != v16_new.shape:
        raise ValueError("k16_new and v16_new must have the same shape")
    n_new = k16_new.shape[2]
    _lib.check(_lib.load().specache_quantize_append(ctypes.byref(cache.shape()), k16_new.data_ptr(),
                                                    v16_new.data_ptr(), n_new, ctypes.byref(cache.c_struct()),
                                                    _stream(stream)),
               "specache_quantize_append")
    cache.seq_len += n_new
    return cache


def offload_fp16(k16_new: torch.Tensor, v16_new: torch.Tensor, k16_cache: torch.Tensor, v16_cache: torch.Tensor,
                 pos0: int, stream=None):
    """specache_offload_fp16: rows [B, Hkv, n_new, D] (device) -> positions pos0.. of the 16-bit
    cache [B, Hkv, Nc, D] (pinned host or device)."""
    _need(k16_new, "k16_new", torch.float16, 4)
    _need(v16_new, "v16_new", torch.float16, 4)
    _need(k16_cache, "k16_cache", torch.float16, 4, cuda=False)
    _need(v16_cache, "v16_cache", torch.float16, 4, cuda=False)
    B, Hkv, Nc, D = k16_cache.shape
    n_new = k16_new.shape[2]
    shape = _lib.Shape(B, Hkv, Hkv, D, Nc, 1, 32, Nc)   # only the layout (Nc) matters here
    _lib.check(_lib.load().specache_offload_fp16(ctypes.byref(shape), k16_new.data_ptr(), v16_new.data_ptr(), n_new,
                                                 pos0, k16_cache.data_ptr(), v16_cache.data_ptr(), _stream(stream)),
               "specache_offload_fp16")


def score_topk_workspace_size(cache: LowBitCache, n_q_heads: int, n_tokens: int, k: int) -> int:
    shape = cache.shape(n_q_heads)
    return int(_lib.load().specache_score_topk_workspace_size(ctypes.byref(shape), n_tokens, k))


def score_topk(q16: torch.Tensor, cache: LowBitCache, k: int, rank_row: int = 1, sm_scale: float | None = None,
               idx_out: torch.Tensor | None = None, rank_key_out: torch.Tensor | None = None,
               workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """specache_score_topk: idx [B, Hkv, k] int32 (ascending) of the top-k positions
    by the rank row's attention over C'.  rank_key_out, if given ([B, Hkv, N]
    float32), receives r(p)."""
    _need(q16, "q16", torch.float16, 4)
    B, Hq, T, D = q16.shape
    sm_scale = 1.0 / math.sqrt(D) if sm_scale is None else float(sm_scale)
    lib = _lib.load()
    shape = cache.shape(Hq)
    need = lib.specache_score_topk_workspace_size(ctypes.byref(shape), T, k)
    if need == 0:
        raise ValueError("invalid score_topk arguments (shape, n_tokens or k)")
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q16.device)
    if idx_out is None:
        idx_out = torch.empty((B, cache.n_kv_heads, k), dtype=torch.int32, device=q16.device)
    _need(idx_out, "idx_out", torch.int32, 3)
    rk = 0
    if rank_key_out is not None:
        _need(rank_key_out, "rank_key_out", torch.float32, 3)
        rk = rank_key_out.data_ptr()
    _lib.check(lib.specache_score_topk(ctypes.byref(shape), q16.data_ptr(), T, rank_row,
                                       ctypes.byref(cache.c_struct()), sm_scale, k, idx_out.data_ptr(), rk,
                                       workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                       _stream(stream)),
               "specache_score_topk")
    return idx_out


def gather_fp16(idx: torch.Tensor, k16_src: torch.Tensor, v16_src: torch.Tensor, bits: int = 1,
                k_sel: torch.Tensor | None = None, v_sel: torch.Tensor | None = None, stream=None,
                seq_len: int | None = None):
    """specache_gather_fp16: rows idx of the 16-bit cache (pinned host or device,
    [B, Hkv, Nc, D], positions [0, seq_len) in use) -> (k_sel, v_sel) [B, Hkv, k, D]."""
    _need(idx, "idx", torch.int32, 3)
    _need(k16_src, "k16_src", torch.float16, 4, cuda=False)
    _need(v16_src, "v16_src", torch.float16, 4, cuda=False)
    for name, t in (("k16_src", k16_src), ("v16_src", v16_src)):
        if not (t.is_cuda or t.is_pinned()):
            raise ValueError(f"{name} must be a GPU tensor or pinned host memory")
    B, Hkv, Nc, D = k16_src.shape
    k = idx.shape[2]
    dev = idx.device
    if k_sel is None:
        k_sel = torch.empty((B, Hkv, k, D), dtype=torch.float16, device=dev)
    if v_sel is None:
        v_sel = torch.empty((B, Hkv, k, D), dtype=torch.float16, device=dev)
    shape = _lib.Shape(B, Hkv, Hkv, D, Nc if seq_len is None else seq_len, bits, 32, Nc)
    _lib.check(_lib.load().specache_gather_fp16(ctypes.byref(shape), idx.data_ptr(), k, k16_src.data_ptr(),
                                                v16_src.data_ptr(), k_sel.data_ptr(), v_sel.data_ptr(),
                                                _stream(stream)),
               "specache_gather_fp16")
    return k_sel, v_sel


def gather_reuse(idx: torch.Tensor, idx_prev: torch.Tensor, k_sel_prev: torch.Tensor, v_sel_prev: torch.Tensor,
                 seq_len: int, k_sel: torch.Tensor | None = None, v_sel: torch.Tensor | None = None,
                 fetch_idx: torch.Tensor | None = None, stream=None):
    """specache_gather_reuse: rows of idx also in idx_prev are copied from the previous
    rows; returns (k_sel, v_sel, fetch_idx) with fetch_idx = -1 for the copied rows."""
    _need(idx, "idx", torch.int32, 3)
    _need(idx_prev, "idx_prev", torch.int32, 3)
    _need(k_sel_prev, "k_sel_prev", torch.float16, 4)
    _need(v_sel_prev, "v_sel_prev", torch.float16, 4)
    B, Hkv, k = idx.shape
    k_prev = idx_prev.shape[2]
    D = k_sel_prev.shape[3]
    dev = idx.device
    if k_sel is None:
        k_sel = torch.empty((B, Hkv, k, D), dtype=torch.float16, device=dev)
    if v_sel is None:
        v_sel = torch.empty((B, Hkv, k, D), dtype=torch.float16, device=dev)
    if fetch_idx is None:
        fetch_idx = torch.empty_like(idx)
    shape = _lib.Shape(B, Hkv, Hkv, D, seq_len, 1, 32)
    _lib.check(_lib.load().specache_gather_reuse(ctypes.byref(shape), idx.data_ptr(), k, idx_prev.data_ptr(), k_prev,
                                                 k_sel_prev.data_ptr(), v_sel_prev.data_ptr(), k_sel.data_ptr(),
                                                 v_sel.data_ptr(), fetch_idx.data_ptr(), _stream(stream)),
               "specache_gather_reuse")
    return k_sel, v_sel, fetch_idx


def gather_fp16_missing(fetch_idx: torch.Tensor, k16_src: torch.Tensor, v16_src: torch.Tensor,
                        k_sel: torch.Tensor, v_sel: torch.Tensor, bits: int = 1, stream=None,
                        seq_len: int | None = None):
    """specache_gather_fp16_missing: fetch the rows fetch_idx marks (>= 0) into k_sel / v_sel."""
    _need(fetch_idx, "fetch_idx", torch.int32, 3)
    _need(k16_src, "k16_src", torch.float16, 4, cuda=False)
    _need(v16_src, "v16_src", torch.float16, 4, cuda=False)
    _need(k_sel, "k_sel", torch.float16, 4)
    _need(v_sel, "v_sel", torch.float16, 4)
    for name, t in (("k16_src", k16_src), ("v16_src", v16_src)):
        if not (t.is_cuda or t.is_pinned()):
            raise ValueError(f"{name} must be a GPU tensor or pinned host memory")
    B, Hkv, Nc, D = k16_src.shape
    k = fetch_idx.shape[2]
    shape = _lib.Shape(B, Hkv, Hkv, D, Nc if seq_len is None else seq_len, bits, 32, Nc)
    _lib.check(_lib.load().specache_gather_fp16_missing(ctypes.byref(shape), fetch_idx.data_ptr(), k,
                                                        k16_src.data_ptr(), v16_src.data_ptr(), k_sel.data_ptr(),
                                                        v_sel.data_ptr(), _stream(stream)),
               "specache_gather_fp16_missing")
    return k_sel, v_sel


class CUStream:
    """A HIP stream limited to a set of compute units (created by the library,
    released by close()).  `.torch` is a torch stream view of it."""

    _create = None

    def __init__(self, n_cus: int = 8):
        handle = ctypes.c_void_p()
        _lib.check(getattr(_lib.load(), self._create)(n_cus, ctypes.byref(handle)), self._create)
        self.handle = handle.value
        self.n_cus = n_cus
        self.torch = torch.cuda.ExternalStream(self.handle)

    def close(self):
        if self.handle:
            torch.cuda.synchronize()
            _lib.check(_lib.load().specache_stream_destroy(self.handle), "specache_stream_destroy")
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class GatherStream(CUStream):
    """specache_gather_stream_create: compute units [0, n_cus), for gather_fp16."""
    _create = "specache_gather_stream_create"


class ComputeStream(CUStream):
    """specache_compute_stream_create: every compute unit but the n_cus of a GatherStream(n_cus)."""
    _create = "specache_compute_stream_create"


def _flag_word(t: torch.Tensor, name: str):
    if not (t.is_cuda and t.dtype in (torch.int32, torch.uint32) and t.numel() >= 1 and t.is_contiguous()):
        raise ValueError(f"{name} must be a contiguous int32 or uint32 CUDA tensor (its first element is used)")
    return t.data_ptr()


def flag_set(flag: torch.Tensor, value: int, stream=None) -> None:
    """specache_flag_set: once the stream's earlier work is done, store `value` (uint32) into
    flag[0] with device-scope release ordering."""
    _lib.check(_lib.load().specache_flag_set(_flag_word(flag, "flag"), value & 0xFFFFFFFF, _stream(stream)),
               "specache_flag_set")


def flag_wait(flag: torch.Tensor, value: int, timeouts: torch.Tensor, max_wait_us: int = 2_000_000,
              stream=None) -> None:
    """specache_flag_wait: hold the stream until flag[0] has reached `value` (bounded by
    max_wait_us; a wait that ends on the bound adds 1 to timeouts[0])."""
    _lib.check(_lib.load().specache_flag_wait(_flag_word(flag, "flag"), value & 0xFFFFFFFF, max_wait_us,
                                              _flag_word(timeouts, "timeouts"), _stream(stream)),
               "specache_flag_wait")


def decode_attn_workspace_size(cache: LowBitCache, n_q_heads: int, n_tokens: int, k: int, tail_len: int = 0) -> int:
    shape = cache.shape(n_q_heads)
    return int(_lib.load().specache_decode_attn_workspace_size(ctypes.byref(shape), n_tokens, k, tail_len))


def _attn_operands(q16, idx, k_sel, v_sel, k_tail, v_tail):
    _need(q16, "q16", torch.float16, 4)
    k = 0
    ip = kp = vp = 0
    if idx is not None:
        _need(idx, "idx", torch.int32, 3)
        k = idx.shape[2]
        if k > 0:
            _need(k_sel, "k_sel", torch.float16, 4)
            _need(v_sel, "v_sel", torch.float16, 4)
            ip, kp, vp = idx.data_ptr(), k_sel.data_ptr(), v_sel.data_ptr()
    R = 0
    ktp = vtp = 0
    if k_tail is not None:
        _need(k_tail, "k_tail", torch.float16, 4)
        _need(v_tail, "v_tail", torch.float16, 4)
        R = k_tail.shape[2]
        ktp, vtp = k_tail.data_ptr(), v_tail.data_ptr()
    return k, ip, kp, vp, R, ktp, vtp


def decode_attn(q16: torch.Tensor, cache: LowBitCache, idx: torch.Tensor | None = None,
                k_sel: torch.Tensor | None = None, v_sel: torch.Tensor | None = None,
                k_tail: torch.Tensor | None = None, v_tail: torch.Tensor | None = None,
                sm_scale: float | None = None, out: torch.Tensor | None = None,
                workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """specache_decode_attn: O [B, Hq, T, D] float16 = Attn(q, C' with rows idx replaced by
    k_sel / v_sel, then the optional tail)."""
    k, ip, kp, vp, R, ktp, vtp = _attn_operands(q16, idx, k_sel, v_sel, k_tail, v_tail)
    B, Hq, T, D = q16.shape
    sm_scale = 1.0 / math.sqrt(D) if sm_scale is None else float(sm_scale)
    lib = _lib.load()
    shape = cache.shape(Hq)
    need = lib.specache_decode_attn_workspace_size(ctypes.byref(shape), T, k, R)
    if need == 0:
        raise ValueError("invalid decode_attn arguments (shape, n_tokens, k or tail length)")
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q16.device)
    if out is None:
        out = torch.empty_like(q16)
    _lib.check(lib.specache_decode_attn(ctypes.byref(shape), q16.data_ptr(), T, ctypes.byref(cache.c_struct()),
                                        ip, k, kp, vp, ktp, vtp, R, sm_scale, out.data_ptr(),
                                        workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                        _stream(stream)),
               "specache_decode_attn")
    return out


def decode_attn_fp16(q16: torch.Tensor, k16: torch.Tensor, v16: torch.Tensor, seq_len: int | None = None,
                     k_tail: torch.Tensor | None = None, v_tail: torch.Tensor | None = None,
                     sm_scale: float | None = None, out: torch.Tensor | None = None,
                     workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """specache_decode_attn_fp16: the 16-bit comparator, attention over the full float16 cache
    k16 / v16 [B, Hkv, Nc, D] (positions [0, seq_len) used) and the optional tail."""
    _need(q16, "q16", torch.float16, 4)
    _need(k16, "k16", torch.float16, 4, cuda=False)
    _need(v16, "v16", torch.float16, 4, cuda=False)
    B, Hq, T, D = q16.shape
    _, Hkv, Nc, _ = k16.shape
    N = Nc if seq_len is None else int(seq_len)
    sm_scale = 1.0 / math.sqrt(D) if sm_scale is None else float(sm_scale)
    R = 0
    ktp = vtp = 0
    if k_tail is not None:
        _need(k_tail, "k_tail", torch.float16, 4)
        _need(v_tail, "v_tail", torch.float16, 4)
        R = k_tail.shape[2]
        ktp, vtp = k_tail.data_ptr(), v_tail.data_ptr()
    lib = _lib.load()
    shape = _lib.Shape(B, Hq, Hkv, D, N, 1, 32, Nc)
    need = lib.specache_decode_attn_fp16_workspace_size(ctypes.byref(shape), T, R)
    if need == 0:
        raise ValueError("invalid decode_attn_fp16 arguments (shape, n_tokens or tail length)")
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q16.device)
    if out is None:
        out = torch.empty_like(q16)
    _lib.check(lib.specache_decode_attn_fp16(ctypes.byref(shape), q16.data_ptr(), T, k16.data_ptr(), v16.data_ptr(),
                                             ktp, vtp, R, sm_scale, out.data_ptr(), workspace.data_ptr(),
                                             workspace.numel() * workspace.element_size(), _stream(stream)),
               "specache_decode_attn_fp16")
    return out


def decode_step_workspace_size(cache: LowBitCache, n_q_heads: int, n_tokens: int, k: int, tail_len: int,
                               k_next: int) -> int:
    shape = cache.shape(n_q_heads)
    return int(_lib.load().specache_decode_step_workspace_size(ctypes.byref(shape), n_tokens, k, tail_len,
                                                                k_next))


def decode_step(q16: torch.Tensor, cache: LowBitCache, k_next: int, rank_row: int = 1,
                rank_mixed: bool = False, idx: torch.Tensor | None = None, k_sel: torch.Tensor | None = None,
                v_sel: torch.Tensor | None = None, k_tail: torch.Tensor | None = None,
                v_tail: torch.Tensor | None = None, sm_scale: float | None = None,
                out: torch.Tensor | None = None, idx_next_out: torch.Tensor | None = None,
                rank_key_out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                stream=None):
    """specache_decode_step: (O, idx_next) -- decode_attn's output and the next selection
    for row rank_row from one pass over C': ranked against C' (score_topk's ranking), or
    with rank_mixed by that row of the attention itself (fetched rows and tail included)."""
    k, ip, kp, vp, R, ktp, vtp = _attn_operands(q16, idx, k_sel, v_sel, k_tail, v_tail)
    B, Hq, T, D = q16.shape
    sm_scale = 1.0 / math.sqrt(D) if sm_scale is None else float(sm_scale)
    lib = _lib.load()
    shape = cache.shape(Hq)
    need = lib.specache_decode_step_workspace_size(ctypes.byref(shape), T, k, R, k_next)
    if need == 0:
        raise ValueError("invalid decode_step arguments (shape, n_tokens, k, tail length or k_next)")
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q16.device)
    if out is None:
        out = torch.empty_like(q16)
    if idx_next_out is None:
        idx_next_out = torch.empty((B, cache.n_kv_heads, k_next), dtype=torch.int32, device=q16.device)
    _need(idx_next_out, "idx_next_out", torch.int32, 3)
    rk = 0
    if rank_key_out is not None:
        _need(rank_key_out, "rank_key_out", torch.float32, 3)
        rk = rank_key_out.data_ptr()
    _lib.check(lib.specache_decode_step(ctypes.byref(shape), q16.data_ptr(), T, rank_row, int(bool(rank_mixed)),
                                        ctypes.byref(cache.c_struct()), ip, k, kp, vp, ktp, vtp, R, sm_scale,
                                        out.data_ptr(), k_next, idx_next_out.data_ptr(), rk,
                                        workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                        _stream(stream)),
               "specache_decode_step")
    return out, idx_next_out
