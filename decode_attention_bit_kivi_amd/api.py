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

    def check(self) -> None:
        """The four buffers have the shapes, types and layout the C ABI assumes for this
        cache's dimensions (raises ValueError / TypeError before any kernel sees them)."""
        cap = self.capacity or self.seq_len
        if self.seq_len <= 0 or self.seq_len > cap:
            raise ValueError(f"cache seq_len {self.seq_len} outside (0, capacity {cap}]")
        sizes = lowbit_sizes(self.batch, self.n_kv_heads, cap, self.head_dim, self.bits, group=self.group,
                             v_bits=self.v_bits or self.bits)
        for name, t, dt, shp in (("k_codes", self.k_codes, torch.int32, sizes[0]),
                                 ("k_meta", self.k_meta, torch.float16, sizes[1]),
                                 ("v_codes", self.v_codes, torch.int32, sizes[2]),
                                 ("v_meta", self.v_meta, torch.float16, sizes[3])):
            _need(t, f"cache.{name}", dt, shp)


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    if hasattr(stream, "handle"):       # GatherStream
        return stream.handle
    return int(stream)


def _need(t: torch.Tensor, name: str, dtype, shape):
    """t is a contiguous tensor of `dtype` whose shape matches `shape` (a tuple whose None
    entries match any size, or an int: only the number of dimensions is fixed).  The device is
    checked separately (_on_gpu), after every shape: a mismatch never reaches the library, whose
    kernels take raw pointers and would read or write out of bounds."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    ndim = shape if isinstance(shape, int) else len(shape)
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if not isinstance(shape, int):
        for got, want in zip(t.shape, shape):
            if want is not None and got != want:
                raise ValueError(f"{name} must have shape {tuple('*' if w is None else w for w in shape)}, "
                                 f"got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _on_gpu(**tensors):
    """Every named tensor (None entries skipped) is on one GPU."""
    dev = None
    for name, t in tensors.items():
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device}, the other operands on {dev}")


def _host_readable(t: torch.Tensor, name: str):
    """A gather / offload endpoint: device memory or pinned host memory."""
    if not (t.is_cuda or t.is_pinned()):
        raise ValueError(f"{name} must be a GPU tensor or pinned host memory")


def _workspace(ws, need: int, device):
    """The caller's workspace (any dtype, contiguous, at least `need` bytes, on the operands'
    GPU), or a new one."""
    if ws is None:
        return torch.empty(need, dtype=torch.uint8, device=device)
    if not isinstance(ws, torch.Tensor) or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor")
    if ws.numel() * ws.element_size() < need:
        raise ValueError(f"workspace holds {ws.numel() * ws.element_size()} bytes, {need} needed")
    return ws


def _nbytes(t: torch.Tensor) -> int:
    return t.numel() * t.element_size()


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
    B, Hkv, Nc, D = k16.shape
    _need(v16, "v16", torch.float16, (B, Hkv, Nc, D))
    N = Nc if seq_len is None else int(seq_len)
    if out is not None:
        out.check()
        if (out.batch, out.n_kv_heads, out.capacity or out.seq_len, out.head_dim, out.bits, out.group) != \
                (B, Hkv, Nc, D, bits, group) or (v_bits is not None and (out.v_bits or out.bits) != v_bits):
            raise ValueError("out cache shape does not match the inputs")
        _on_gpu(k16=k16, v16=v16, k_codes=out.k_codes, k_meta=out.k_meta, v_codes=out.v_codes, v_meta=out.v_meta)
    else:
        _on_gpu(k16=k16, v16=v16)
    cache = out if out is not None else empty_cache(B, Hkv, N, D, bits, k16.device, capacity=Nc, v_bits=v_bits,
                                                    group=group)
    cache.seq_len = N
    _lib.check(_lib.load().specache_quantize_pack(ctypes.byref(cache.shape()), k16.data_ptr(), v16.data_ptr(),
                                                  ctypes.byref(cache.c_struct()), _stream(stream)),
               "specache_quantize_pack")
    return cache


def _cache_on_gpu(cache: LowBitCache, **others):
    _on_gpu(k_codes=cache.k_codes, k_meta=cache.k_meta, v_codes=cache.v_codes, v_meta=cache.v_meta, **others)


def quantize_append(cache: LowBitCache, k16_new: torch.Tensor, v16_new: torch.Tensor, stream=None) -> LowBitCache:
    """specache_quantize_append: quantize K, V [B, Hkv, n_new, D] (n_new a multiple of 32) into
    positions [seq_len, seq_len + n_new) of the cache; cache.seq_len grows by n_new."""
    cache.check()
    _need(k16_new, "k16_new", torch.float16, (cache.batch, cache.n_kv_heads, None, cache.head_dim))
    _need(v16_new, "v16_new", torch.float16, tuple(k16_new.shape))
    _cache_on_gpu(cache, k16_new=k16_new, v16_new=v16_new)
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
    _need(k16_cache, "k16_cache", torch.float16, 4)
    B, Hkv, Nc, D = k16_cache.shape
    _need(v16_cache, "v16_cache", torch.float16, (B, Hkv, Nc, D))
    _need(k16_new, "k16_new", torch.float16, (B, Hkv, None, D))
    _need(v16_new, "v16_new", torch.float16, tuple(k16_new.shape))
    _on_gpu(k16_new=k16_new, v16_new=v16_new)
    _host_readable(k16_cache, "k16_cache")
    _host_readable(v16_cache, "v16_cache")
    n_new = k16_new.shape[2]
    shape = _lib.Shape(B, Hkv, Hkv, D, Nc, 1, 32, Nc)   # only the layout (Nc) matters here
    _lib.check(_lib.load().specache_offload_fp16(ctypes.byref(shape), k16_new.data_ptr(), v16_new.data_ptr(), n_new,
                                                 pos0, k16_cache.data_ptr(), v16_cache.data_ptr(), _stream(stream)),
               "specache_offload_fp16")


def score_topk_workspace_size(cache: LowBitCache, n_q_heads: int, n_tokens: int, k: int) -> int:
    shape = cache.shape(n_q_heads)
    return int(_lib.load().specache_score_topk_workspace_size(ctypes.byref(shape), n_tokens, k))


def _queries(q16: torch.Tensor, cache: LowBitCache):
    """q16 [B, Hq, T, D] for this cache: (B, Hq, T, D)."""
    cache.check()
    _need(q16, "q16", torch.float16, (cache.batch, None, None, cache.head_dim))
    B, Hq, T, D = q16.shape
    if Hq % cache.n_kv_heads:
        raise ValueError(f"q16 has {Hq} heads, not a multiple of the cache's {cache.n_kv_heads} KV heads")
    return B, Hq, T, D


def score_topk(q16: torch.Tensor, cache: LowBitCache, k: int, rank_row: int = 1, sm_scale: float | None = None,
               idx_out: torch.Tensor | None = None, rank_key_out: torch.Tensor | None = None,
               workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """specache_score_topk: idx [B, Hkv, k] int32 (ascending) of the top-k positions
    by the rank row's attention over C'.  rank_key_out, if given ([B, Hkv, N]
    float32), receives r(p)."""
    B, Hq, T, D = _queries(q16, cache)
    Hkv, N = cache.n_kv_heads, cache.seq_len
    if idx_out is not None:
        _need(idx_out, "idx_out", torch.int32, (B, Hkv, k))
    if rank_key_out is not None:
        _need(rank_key_out, "rank_key_out", torch.float32, (B, Hkv, N))
    sm_scale = 1.0 / math.sqrt(D) if sm_scale is None else float(sm_scale)
    lib = _lib.load()
    shape = cache.shape(Hq)
    need = lib.specache_score_topk_workspace_size(ctypes.byref(shape), T, k)
    if need == 0:
        raise ValueError("invalid score_topk arguments (shape, n_tokens or k)")
    _cache_on_gpu(cache, q16=q16, idx_out=idx_out, rank_key_out=rank_key_out, workspace=workspace)
    workspace = _workspace(workspace, need, q16.device)
    if idx_out is None:
        idx_out = torch.empty((B, Hkv, k), dtype=torch.int32, device=q16.device)
    rk = 0 if rank_key_out is None else rank_key_out.data_ptr()
    _lib.check(lib.specache_score_topk(ctypes.byref(shape), q16.data_ptr(), T, rank_row,
                                       ctypes.byref(cache.c_struct()), sm_scale, k, idx_out.data_ptr(), rk,
                                       workspace.data_ptr(), _nbytes(workspace), _stream(stream)),
               "specache_score_topk")
    return idx_out


def _rows_out(t, name, shape, device):
    """A caller's row buffer of `shape` (float16, GPU), or a new one."""
    if t is None:
        return torch.empty(shape, dtype=torch.float16, device=device)
    _need(t, name, torch.float16, shape)
    return t


def gather_fp16(idx: torch.Tensor, k16_src: torch.Tensor, v16_src: torch.Tensor, bits: int = 1,
                k_sel: torch.Tensor | None = None, v_sel: torch.Tensor | None = None, stream=None,
                seq_len: int | None = None):
    """specache_gather_fp16: rows idx of the 16-bit cache (pinned host or device,
    [B, Hkv, Nc, D], positions [0, seq_len) in use) -> (k_sel, v_sel) [B, Hkv, k, D]."""
    _need(k16_src, "k16_src", torch.float16, 4)
    B, Hkv, Nc, D = k16_src.shape
    _need(v16_src, "v16_src", torch.float16, (B, Hkv, Nc, D))
    _need(idx, "idx", torch.int32, (B, Hkv, None))
    k = idx.shape[2]
    for name, t in (("k_sel", k_sel), ("v_sel", v_sel)):
        if t is not None:
            _need(t, name, torch.float16, (B, Hkv, k, D))
    _on_gpu(idx=idx, k_sel=k_sel, v_sel=v_sel)
    _host_readable(k16_src, "k16_src")
    _host_readable(v16_src, "v16_src")
    k_sel = _rows_out(k_sel, "k_sel", (B, Hkv, k, D), idx.device)
    v_sel = _rows_out(v_sel, "v_sel", (B, Hkv, k, D), idx.device)
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
    B, Hkv, k = idx.shape
    _need(idx_prev, "idx_prev", torch.int32, (B, Hkv, None))
    k_prev = idx_prev.shape[2]
    _need(k_sel_prev, "k_sel_prev", torch.float16, (B, Hkv, k_prev, None))
    D = k_sel_prev.shape[3]
    _need(v_sel_prev, "v_sel_prev", torch.float16, (B, Hkv, k_prev, D))
    for name, t in (("k_sel", k_sel), ("v_sel", v_sel)):
        if t is not None:
            _need(t, name, torch.float16, (B, Hkv, k, D))
    if fetch_idx is not None:
        _need(fetch_idx, "fetch_idx", torch.int32, (B, Hkv, k))
    _on_gpu(idx=idx, idx_prev=idx_prev, k_sel_prev=k_sel_prev, v_sel_prev=v_sel_prev, k_sel=k_sel, v_sel=v_sel,
            fetch_idx=fetch_idx)
    k_sel = _rows_out(k_sel, "k_sel", (B, Hkv, k, D), idx.device)
    v_sel = _rows_out(v_sel, "v_sel", (B, Hkv, k, D), idx.device)
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
    _need(k16_src, "k16_src", torch.float16, 4)
    B, Hkv, Nc, D = k16_src.shape
    _need(v16_src, "v16_src", torch.float16, (B, Hkv, Nc, D))
    _need(fetch_idx, "fetch_idx", torch.int32, (B, Hkv, None))
    k = fetch_idx.shape[2]
    _need(k_sel, "k_sel", torch.float16, (B, Hkv, k, D))
    _need(v_sel, "v_sel", torch.float16, (B, Hkv, k, D))
    _on_gpu(fetch_idx=fetch_idx, k_sel=k_sel, v_sel=v_sel)
    _host_readable(k16_src, "k16_src")
    _host_readable(v16_src, "v16_src")
    shape = _lib.Shape(B, Hkv, Hkv, D, Nc if seq_len is None else seq_len, bits, 32, Nc)
    _lib.check(_lib.load().specache_gather_fp16_missing(ctypes.byref(shape), fetch_idx.data_ptr(), k,
                                                        k16_src.data_ptr(), v16_src.data_ptr(), k_sel.data_ptr(),
                                                        v_sel.data_ptr(), _stream(stream)),
               "specache_gather_fp16_missing")
    return k_sel, v_sel


# Library streams that close() has retired.  torch's pinned-host allocator records an event on
# every stream a pinned block was copied on when that block is freed, which may happen long after
# the stream's last use (a pinned tensor that outlives the stream object); a destroyed stream
# there crashes the process.  So a closed stream keeps its HIP handle until the process ends.
_RETIRED_STREAMS: list = []


class CUStream:
    """A HIP stream limited to a set of compute units (created by the library).  `.torch` is a
    torch stream view of it.  close() waits for the stream's work and retires it: no work may be
    enqueued on it afterwards, but the HIP stream itself is released only when the process ends
    (see _RETIRED_STREAMS), so that freeing a pinned tensor that was copied on it stays safe."""

    _create = None

    def __init__(self, n_cus: int = 8):
        handle = ctypes.c_void_p()
        _lib.check(getattr(_lib.load(), self._create)(n_cus, ctypes.byref(handle)), self._create)
        self.handle = handle.value
        self.n_cus = n_cus
        self.torch = torch.cuda.ExternalStream(self.handle)

    def close(self):
        if self.handle:
            self.torch.synchronize()
            _RETIRED_STREAMS.append((self.handle, self.torch))
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


def _attn_operands(q16, cache, idx, k_sel, v_sel, k_tail, v_tail, out):
    """Shapes of the attention operands against q16 [B, Hq, T, D] and the cache:
    idx [B, Hkv, k], k_sel / v_sel [B, Hkv, k, D], k_tail / v_tail [B, Hkv, R, D], out like q16."""
    B, Hq, T, D = _queries(q16, cache)
    Hkv = cache.n_kv_heads
    k = 0
    if idx is not None:
        _need(idx, "idx", torch.int32, (B, Hkv, None))
        k = idx.shape[2]
        if k > 0:
            _need(k_sel, "k_sel", torch.float16, (B, Hkv, k, D))
            _need(v_sel, "v_sel", torch.float16, (B, Hkv, k, D))
    R = 0
    if k_tail is not None:
        _need(k_tail, "k_tail", torch.float16, (B, Hkv, None, D))
        _need(v_tail, "v_tail", torch.float16, tuple(k_tail.shape))
        R = k_tail.shape[2]
    elif v_tail is not None:
        raise ValueError("v_tail given without k_tail")
    if out is not None:
        _need(out, "out", torch.float16, (B, Hq, T, D))
    return k, R


def _ptrs(k, idx, k_sel, v_sel, R, k_tail, v_tail):
    ip, kp, vp = (idx.data_ptr(), k_sel.data_ptr(), v_sel.data_ptr()) if k > 0 else (0, 0, 0)
    ktp, vtp = (k_tail.data_ptr(), v_tail.data_ptr()) if R > 0 else (0, 0)
    return ip, kp, vp, ktp, vtp


def decode_attn(q16: torch.Tensor, cache: LowBitCache, idx: torch.Tensor | None = None,
                k_sel: torch.Tensor | None = None, v_sel: torch.Tensor | None = None,
                k_tail: torch.Tensor | None = None, v_tail: torch.Tensor | None = None,
                sm_scale: float | None = None, out: torch.Tensor | None = None,
                workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """specache_decode_attn: O [B, Hq, T, D] float16 = Attn(q, C' with rows idx replaced by
    k_sel / v_sel, then the optional tail)."""
    k, R = _attn_operands(q16, cache, idx, k_sel, v_sel, k_tail, v_tail, out)
    B, Hq, T, D = q16.shape
    sm_scale = 1.0 / math.sqrt(D) if sm_scale is None else float(sm_scale)
    lib = _lib.load()
    shape = cache.shape(Hq)
    need = lib.specache_decode_attn_workspace_size(ctypes.byref(shape), T, k, R)
    if need == 0:
        raise ValueError("invalid decode_attn arguments (shape, n_tokens, k or tail length)")
    _cache_on_gpu(cache, q16=q16, idx=idx if k else None, k_sel=k_sel if k else None, v_sel=v_sel if k else None,
                  k_tail=k_tail, v_tail=v_tail, out=out, workspace=workspace)
    workspace = _workspace(workspace, need, q16.device)
    if out is None:
        out = torch.empty_like(q16)
    ip, kp, vp, ktp, vtp = _ptrs(k, idx, k_sel, v_sel, R, k_tail, v_tail)
    _lib.check(lib.specache_decode_attn(ctypes.byref(shape), q16.data_ptr(), T, ctypes.byref(cache.c_struct()),
                                        ip, k, kp, vp, ktp, vtp, R, sm_scale, out.data_ptr(),
                                        workspace.data_ptr(), _nbytes(workspace), _stream(stream)),
               "specache_decode_attn")
    return out


def decode_attn_fp16(q16: torch.Tensor, k16: torch.Tensor, v16: torch.Tensor, seq_len: int | None = None,
                     k_tail: torch.Tensor | None = None, v_tail: torch.Tensor | None = None,
                     sm_scale: float | None = None, out: torch.Tensor | None = None,
                     workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """specache_decode_attn_fp16: the 16-bit comparator, attention over the full float16 cache
    k16 / v16 [B, Hkv, Nc, D] (positions [0, seq_len) used) and the optional tail."""
    _need(k16, "k16", torch.float16, 4)
    B, Hkv, Nc, D = k16.shape
    _need(v16, "v16", torch.float16, (B, Hkv, Nc, D))
    _need(q16, "q16", torch.float16, (B, None, None, D))
    _, Hq, T, _ = q16.shape
    if Hq % Hkv:
        raise ValueError(f"q16 has {Hq} heads, not a multiple of the cache's {Hkv} KV heads")
    N = Nc if seq_len is None else int(seq_len)
    sm_scale = 1.0 / math.sqrt(D) if sm_scale is None else float(sm_scale)
    R = 0
    if k_tail is not None:
        _need(k_tail, "k_tail", torch.float16, (B, Hkv, None, D))
        _need(v_tail, "v_tail", torch.float16, tuple(k_tail.shape))
        R = k_tail.shape[2]
    if out is not None:
        _need(out, "out", torch.float16, (B, Hq, T, D))
    lib = _lib.load()
    shape = _lib.Shape(B, Hq, Hkv, D, N, 1, 32, Nc)
    need = lib.specache_decode_attn_fp16_workspace_size(ctypes.byref(shape), T, R)
    if need == 0:
        raise ValueError("invalid decode_attn_fp16 arguments (shape, n_tokens or tail length)")
    _on_gpu(q16=q16, k_tail=k_tail, v_tail=v_tail, out=out, workspace=workspace)
    _host_readable(k16, "k16")
    _host_readable(v16, "v16")
    workspace = _workspace(workspace, need, q16.device)
    if out is None:
        out = torch.empty_like(q16)
    ktp, vtp = (k_tail.data_ptr(), v_tail.data_ptr()) if R > 0 else (0, 0)
    _lib.check(lib.specache_decode_attn_fp16(ctypes.byref(shape), q16.data_ptr(), T, k16.data_ptr(), v16.data_ptr(),
                                             ktp, vtp, R, sm_scale, out.data_ptr(), workspace.data_ptr(),
                                             _nbytes(workspace), _stream(stream)),
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
    k, R = _attn_operands(q16, cache, idx, k_sel, v_sel, k_tail, v_tail, out)
    B, Hq, T, D = q16.shape
    Hkv, N = cache.n_kv_heads, cache.seq_len
    if idx_next_out is not None:
        _need(idx_next_out, "idx_next_out", torch.int32, (B, Hkv, k_next))
    if rank_key_out is not None:
        _need(rank_key_out, "rank_key_out", torch.float32, (B, Hkv, N))
    sm_scale = 1.0 / math.sqrt(D) if sm_scale is None else float(sm_scale)
    lib = _lib.load()
    shape = cache.shape(Hq)
    need = lib.specache_decode_step_workspace_size(ctypes.byref(shape), T, k, R, k_next)
    if need == 0:
        raise ValueError("invalid decode_step arguments (shape, n_tokens, k, tail length or k_next)")
    _cache_on_gpu(cache, q16=q16, idx=idx if k else None, k_sel=k_sel if k else None, v_sel=v_sel if k else None,
                  k_tail=k_tail, v_tail=v_tail, out=out, idx_next_out=idx_next_out, rank_key_out=rank_key_out,
                  workspace=workspace)
    workspace = _workspace(workspace, need, q16.device)
    if out is None:
        out = torch.empty_like(q16)
    if idx_next_out is None:
        idx_next_out = torch.empty((B, Hkv, k_next), dtype=torch.int32, device=q16.device)
    rk = 0 if rank_key_out is None else rank_key_out.data_ptr()
    ip, kp, vp, ktp, vtp = _ptrs(k, idx, k_sel, v_sel, R, k_tail, v_tail)
    _lib.check(lib.specache_decode_step(ctypes.byref(shape), q16.data_ptr(), T, rank_row, int(bool(rank_mixed)),
                                        ctypes.byref(cache.c_struct()), ip, k, kp, vp, ktp, vtp, R, sm_scale,
                                        out.data_ptr(), k_next, idx_next_out.data_ptr(), rk,
                                        workspace.data_ptr(), _nbytes(workspace), _stream(stream)),
               "specache_decode_step")
    return out, idx_next_out


def decode_step_noalloc(q16: torch.Tensor, cache: LowBitCache, k_next: int, rank_row: int = 1,
                        rank_mixed: bool = False, idx: torch.Tensor | None = None, k_sel: torch.Tensor | None = None,
                        v_sel: torch.Tensor | None = None, k_tail: torch.Tensor | None = None,
                        v_tail: torch.Tensor | None = None, sm_scale: float | None = None,
                        out: torch.Tensor = None, idx_next_out: torch.Tensor = None,
                        rank_key_out: torch.Tensor | None = None, stream=None):
    """specache_decode_step_noalloc: decode_step with its scratch in the library's static device
    array (no workspace; out and idx_next_out are the caller's, so nothing is allocated here
    either).  Calls that overlap on one GPU race on the array."""
    k, R = _attn_operands(q16, cache, idx, k_sel, v_sel, k_tail, v_tail, out)
    B, Hq, T, D = q16.shape
    Hkv, N = cache.n_kv_heads, cache.seq_len
    if out is None or idx_next_out is None:
        raise ValueError("decode_step_noalloc allocates nothing: pass out and idx_next_out")
    _need(idx_next_out, "idx_next_out", torch.int32, (B, Hkv, k_next))
    if rank_key_out is not None:
        _need(rank_key_out, "rank_key_out", torch.float32, (B, Hkv, N))
    sm_scale = 1.0 / math.sqrt(D) if sm_scale is None else float(sm_scale)
    _cache_on_gpu(cache, q16=q16, idx=idx if k else None, k_sel=k_sel if k else None, v_sel=v_sel if k else None,
                  k_tail=k_tail, v_tail=v_tail, out=out, idx_next_out=idx_next_out, rank_key_out=rank_key_out)
    rk = 0 if rank_key_out is None else rank_key_out.data_ptr()
    ip, kp, vp, ktp, vtp = _ptrs(k, idx, k_sel, v_sel, R, k_tail, v_tail)
    _lib.check(_lib.load().specache_decode_step_noalloc(
        ctypes.byref(cache.shape(Hq)), q16.data_ptr(), T, rank_row, int(bool(rank_mixed)),
        ctypes.byref(cache.c_struct()), ip, k, kp, vp, ktp, vtp, R, sm_scale, out.data_ptr(), k_next,
        idx_next_out.data_ptr(), rk, _stream(stream)),
        "specache_decode_step_noalloc")
    return out, idx_next_out
