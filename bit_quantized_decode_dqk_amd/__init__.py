"""Python binding of libdqk (the C ABI in include/dqk.h), argument marshalling only.

Every step of the decode path runs in the HIP kernels of libdqk.so; this module
turns torch tensors into device pointers and a HIP stream, calls the C entry
point of the same name, and raises on a non-OK status.  There is no fallback:
if libdqk.so is missing or cannot be loaded, every call raises.
PyTorch provides device memory and streams only.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional, Sequence

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdqk.so")

DQK_F32, DQK_BF16 = 0, 1
GROUP = 32


class DqkError(RuntimeError):
    pass


class _Cache(C.Structure):
    _fields_ = [("batch", C.c_int32), ("num_kv_heads", C.c_int32), ("head_dim", C.c_int32),
                ("capacity", C.c_int32), ("k_codes", C.c_void_p), ("k_scales", C.c_void_p),
                ("k_ch0", C.c_void_p), ("k_tail", C.c_void_p), ("v_codes", C.c_void_p),
                ("v_scales", C.c_void_p), ("lengths", C.c_void_p)]


_lib = None
EXPORTS = ("dqk_status_str", "dqk_keep_count", "dqk_cache_plane_bytes", "dqk_transform_quantize_append",
           "dqk_select_channels", "dqk_append_select", "dqk_decode_workspace_bytes",
           "dqk_decode_attention", "dqk_select_channels_shared", "dqk_decode_attention_shared",
           "dqk_decode_attention_noalloc", "dqk_cache_grow", "dqk_stream_read_config",
           "dqk_dequant_reference", "dqk_bf16_decode_workspace_bytes",
           "dqk_bf16_decode_attention", "dqk_debug_f16_from_f32", "dqk_stream_read")


def lib():
    """Load libdqk.so (built in-tree by build.py); raises if it is absent."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise DqkError(f"{LIB_PATH} is missing: build it with "
                           "`python -m bit_quantized_decode_dqk_amd.build` (no fallback exists)")
        L = C.CDLL(LIB_PATH)
        P, I, S = C.c_void_p, C.c_int32, C.c_size_t
        L.dqk_status_str.restype = C.c_char_p
        L.dqk_status_str.argtypes = [C.c_int]
        for name, args in {
            "dqk_keep_count": [I, I, P],
            "dqk_cache_plane_bytes": [I, I, I, I, P],
            "dqk_transform_quantize_append": [C.POINTER(_Cache), P, P, C.c_int, P, P, I, P],
            "dqk_select_channels": [P, C.c_int, P, I, I, I, I, I, P, P, P],
            "dqk_append_select": [C.POINTER(_Cache), P, P, P, P, I, P, P, I, I, C.c_int, P, P, P],
            "dqk_decode_workspace_bytes": [C.POINTER(_Cache), I, I, P],
            "dqk_decode_attention": [C.POINTER(_Cache), P, P, I, I, C.c_float, I, P, P, S, P],
            "dqk_select_channels_shared": [P, C.c_int, P, I, I, I, I, I, P, P, P],
            "dqk_decode_attention_noalloc": [C.POINTER(_Cache), P, P, I, I, C.c_float, I, P, P],
            "dqk_decode_attention_shared": [C.POINTER(_Cache), P, P, I, I, C.c_float, I, P, P, S,
                                            P],
            "dqk_dequant_reference": [C.POINTER(_Cache), P, P, P],
            "dqk_cache_grow": [C.POINTER(_Cache), C.POINTER(_Cache), P],
            "dqk_bf16_decode_workspace_bytes": [I, I, I, I, I, I, P],
            "dqk_bf16_decode_attention": [P, P, P, P, I, I, I, I, I, C.c_float, I, P, P, S, P],
            "dqk_debug_f16_from_f32": [P, P, S, P],
            "dqk_stream_read": [P, S, P, P],
            "dqk_stream_read_config": [P, S, P, I, I, P],
        }.items():
            fn = getattr(L, name)
            fn.restype = C.c_int
            fn.argtypes = args
        _lib = L
    return _lib


def _check(status: int, what: str):
    if status != 0:
        msg = lib().dqk_status_str(status).decode()
        raise DqkError(f"{what}: {msg} (status {status})")


def _torch():
    import torch
    return torch


def _stream(stream) -> C.c_void_p:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream)


def _ptr(t) -> C.c_void_p:
    if t is None:
        return C.c_void_p(0)
    if not t.is_cuda:
        raise DqkError("tensor must be on the GPU")
    if not t.is_contiguous():
        raise DqkError("tensor must be contiguous")
    return C.c_void_p(t.data_ptr())


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return DQK_F32
    if t.dtype == torch.bfloat16:
        return DQK_BF16
    raise DqkError(f"unsupported dtype {t.dtype}")


def keep_for_sparsity(head_dim: int, sparsity_pct: int) -> int:
    """Channels kept per query head at a query-channel sparsity in percent, as the
    library defines it (dqk_keep_count)."""
    out = C.c_int32(0)
    _check(lib().dqk_keep_count(int(head_dim), int(sparsity_pct), C.byref(out)), "dqk_keep_count")
    return int(out.value)


def cache_plane_bytes(batch: int, hkv: int, d: int, cap: int):
    """Bytes of each of the cache's seven planes (k_codes, k_scales, k_ch0, k_tail,
    v_codes, v_scales, lengths) for this shape; a host query, no GPU needed."""
    out = (C.c_size_t * 7)()
    _check(lib().dqk_cache_plane_bytes(batch, hkv, d, cap, out), "dqk_cache_plane_bytes")
    return list(out)


PLANES = ("k_codes", "k_scales", "k_ch0", "k_tail", "v_codes", "v_scales", "lengths")


class Cache:
    """Device planes of a 2-bit cache (torch tensors, zero-filled)."""

    def __init__(self, batch: int, hkv: int, d: int, cap: int, device="cuda"):
        torch = _torch()
        self.batch, self.hkv, self.d, self.cap = batch, hkv, d, cap
        sizes = cache_plane_bytes(batch, hkv, d, cap)
        shapes = {
            "k_codes": ((batch, hkv, d, cap // 4), torch.uint8),
            "k_scales": ((batch, hkv, d, cap // GROUP), torch.int16),   # fp16 bits
            "k_ch0": ((batch, hkv, cap), torch.int16),                   # fp16 bits
            "k_tail": ((batch, hkv, GROUP, d), torch.float32),
            "v_codes": ((batch, hkv, cap // 16, d), torch.int32),        # 32-bit code words
            "v_scales": ((batch, hkv, cap, d // GROUP), torch.int16),    # fp16 bits
            "lengths": ((2 * batch,), torch.int32),   # lengths, then arrival counters
        }
        for (name, (shape, dt)), nbytes in zip(shapes.items(), sizes):
            t = torch.zeros(shape, dtype=dt, device=device)
            assert t.numel() * t.element_size() == nbytes, name
            setattr(self, name, t)

    def struct(self) -> _Cache:
        return _Cache(self.batch, self.hkv, self.d, self.cap, *(_ptr(getattr(self, n)).value
                                                                for n in PLANES))

    def planes(self):
        return {n: getattr(self, n) for n in PLANES}

    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in self.planes().values())


def transform_quantize_append(cache: Cache, k_new, v_new, bmat, n_new, stream=None):
    """k_new/v_new [batch][hkv][max_new][d] (fp32 or bf16), bmat [hkv][d][d] fp32,
    n_new [batch] int32 on the device."""
    if k_new.dtype != v_new.dtype or k_new.shape != v_new.shape:
        raise DqkError("k_new and v_new must match in dtype and shape")
    max_new = int(k_new.shape[2])
    s = cache.struct()
    _check(lib().dqk_transform_quantize_append(C.byref(s), _ptr(k_new), _ptr(v_new),
                                               _dtype_code(k_new), _ptr(bmat), _ptr(n_new),
                                               max_new, _stream(stream)),
           "dqk_transform_quantize_append")


def select_channels(q, amat, hkv: int, keep: int, q_prime=None, sel_idx=None, stream=None):
    """q [batch][hq][d] (fp32 or bf16), amat [hkv][d][d] fp32 -> (q' fp32, idx int32)."""
    torch = _torch()
    batch, hq, d = q.shape
    if q_prime is None:
        q_prime = torch.empty((batch, hq, d), dtype=torch.float32, device=q.device)
    if sel_idx is None:
        sel_idx = torch.empty((batch, hq, keep), dtype=torch.int32, device=q.device)
    _check(lib().dqk_select_channels(_ptr(q), _dtype_code(q), _ptr(amat), batch, hq, hkv, d, keep,
                                     _ptr(q_prime), _ptr(sel_idx), _stream(stream)),
           "dqk_select_channels")
    return q_prime, sel_idx


def append_select(cache: Cache, k_new, v_new, bmat, n_new, q, amat, keep: int, q_prime=None,
                  sel_idx=None, stream=None):
    """transform_quantize_append and select_channels of one step in one launch (q, k_new
    and v_new of one dtype; the selection uses the cache's batch and KV heads)."""
    torch = _torch()
    if k_new.dtype != v_new.dtype or k_new.shape != v_new.shape or q.dtype != k_new.dtype:
        raise DqkError("q, k_new and v_new must share a dtype; k_new and v_new a shape")
    batch, hq, d = q.shape
    if q_prime is None:
        q_prime = torch.empty((batch, hq, d), dtype=torch.float32, device=q.device)
    if sel_idx is None:
        sel_idx = torch.empty((batch, hq, keep), dtype=torch.int32, device=q.device)
    s = cache.struct()
    _check(lib().dqk_append_select(C.byref(s), _ptr(k_new), _ptr(v_new), _ptr(bmat), _ptr(n_new),
                                   int(k_new.shape[2]), _ptr(q), _ptr(amat), hq, keep,
                                   _dtype_code(q), _ptr(q_prime), _ptr(sel_idx), _stream(stream)),
           "dqk_append_select")
    return q_prime, sel_idx


def decode_workspace_bytes(cache: Cache, hq: int, split_tokens: int = 0) -> int:
    """Bytes of device workspace dqk_decode_attention needs for this cache shape, hq
    query heads and split length (0: the library's choice), as dqk.h defines it."""
    out = C.c_size_t(0)
    s = cache.struct()
    _check(lib().dqk_decode_workspace_bytes(C.byref(s), hq, split_tokens, C.byref(out)),
           "dqk_decode_workspace_bytes")
    return int(out.value)


def decode_attention(cache: Cache, q_prime, sel_idx, sm_scale: float, split_tokens: int = 0,
                     out=None, workspace=None, stream=None):
    """Pruned 2-bit decode attention (dqk_decode_attention): q_prime [batch][hq][d] fp32
    and sel_idx [batch][hq][keep] int32 as dqk_select_channels leaves them; returns out
    [batch][hq][d] fp32 (allocated when not given).  The workspace, if given, holds at
    least decode_workspace_bytes(...) bytes and needs no initialization."""
    torch = _torch()
    batch, hq, d = q_prime.shape
    keep = int(sel_idx.shape[-1])
    if out is None:
        out = torch.empty((batch, hq, d), dtype=torch.float32, device=q_prime.device)
    if workspace is None:
        nb = decode_workspace_bytes(cache, hq, split_tokens)
        workspace = torch.empty(max(nb, 16), dtype=torch.uint8, device=q_prime.device)
    s = cache.struct()
    _check(lib().dqk_decode_attention(C.byref(s), _ptr(q_prime), _ptr(sel_idx), hq, keep,
                                      float(sm_scale), split_tokens, _ptr(out), _ptr(workspace),
                                      workspace.numel() * workspace.element_size(),
                                      _stream(stream)),
           "dqk_decode_attention")
    return out


DECODE_SCRATCH_BYTES = 16 << 20


def decode_attention_noalloc(cache: Cache, q_prime, sel_idx, sm_scale: float,
                             split_tokens: int = 0, out=None, stream=None):
    """dqk_decode_attention_noalloc: the per-head decode with the split partials in
    the library's device scratch (no workspace; the library allocates nothing).
    Pass `out` to keep the whole call free of allocation.  Calls that overlap on
    one GPU race on the scratch."""
    torch = _torch()
    batch, hq, d = q_prime.shape
    keep = int(sel_idx.shape[-1])
    if out is None:
        out = torch.empty((batch, hq, d), dtype=torch.float32, device=q_prime.device)
    s = cache.struct()
    _check(lib().dqk_decode_attention_noalloc(C.byref(s), _ptr(q_prime), _ptr(sel_idx), hq, keep,
                                              float(sm_scale), split_tokens, _ptr(out),
                                              _stream(stream)),
           "dqk_decode_attention_noalloc")
    return out


def select_channels_shared(q, amat, hkv: int, keep: int, q_prime=None, sel_idx=None,
                           stream=None):
    """Group-shared selection (dqk_select_channels_shared): q [batch][hq][d] (fp32 or
    bf16), amat [hkv][d][d] fp32 -> (q' [batch][hq][d] fp32, idx [batch][hkv][keep])."""
    torch = _torch()
    batch, hq, d = q.shape
    if q_prime is None:
        q_prime = torch.empty((batch, hq, d), dtype=torch.float32, device=q.device)
    if sel_idx is None:
        sel_idx = torch.empty((batch, hkv, keep), dtype=torch.int32, device=q.device)
    _check(lib().dqk_select_channels_shared(_ptr(q), _dtype_code(q), _ptr(amat), batch, hq, hkv,
                                            d, keep, _ptr(q_prime), _ptr(sel_idx),
                                            _stream(stream)),
           "dqk_select_channels_shared")
    return q_prime, sel_idx


def decode_attention_shared(cache: Cache, q_prime, sel_idx, sm_scale: float,
                            split_tokens: int = 0, out=None, workspace=None, stream=None):
    """Decode with group-shared kept sets (dqk_decode_attention_shared): q_prime
    [batch][hq][d] fp32, sel_idx [batch][hkv][keep] int32; returns out [batch][hq][d]."""
    torch = _torch()
    batch, hq, d = q_prime.shape
    keep = int(sel_idx.shape[-1])
    if out is None:
        out = torch.empty((batch, hq, d), dtype=torch.float32, device=q_prime.device)
    if workspace is None:
        nb = decode_workspace_bytes(cache, hq, split_tokens)
        workspace = torch.empty(max(nb, 16), dtype=torch.uint8, device=q_prime.device)
    s = cache.struct()
    _check(lib().dqk_decode_attention_shared(C.byref(s), _ptr(q_prime), _ptr(sel_idx), hq, keep,
                                             float(sm_scale), split_tokens, _ptr(out),
                                             _ptr(workspace),
                                             workspace.numel() * workspace.element_size(),
                                             _stream(stream)),
           "dqk_decode_attention_shared")
    return out


def cache_grow(cache: Cache, capacity: int, out: Optional[Cache] = None, stream=None) -> Cache:
    """A cache of a larger capacity holding the same contents (dqk_cache_grow copies
    every plane of `cache` into it): `out` if given (zero-filled by the caller),
    else a new zero-filled cache."""
    if capacity < cache.cap:
        raise DqkError("a grown cache needs at least the old capacity")
    new = out if out is not None else Cache(cache.batch, cache.hkv, cache.d, capacity,
                                            device=cache.k_codes.device)
    if (new.batch, new.hkv, new.d, new.cap) != (cache.batch, cache.hkv, cache.d, capacity):
        raise DqkError("the destination cache has another shape")
    src, dst = cache.struct(), new.struct()
    _check(lib().dqk_cache_grow(C.byref(src), C.byref(dst), _stream(stream)), "dqk_cache_grow")
    return new


def dequant_reference(cache: Cache, stream=None):
    """Dense dequantized keys and values [batch][hkv][capacity][d] fp32 (zero past each
    row's length): a checking and inspection aid, not on the decode path."""
    torch = _torch()
    shape = (cache.batch, cache.hkv, cache.cap, cache.d)
    k = torch.empty(shape, dtype=torch.float32, device=cache.k_codes.device)
    v = torch.empty_like(k)
    s = cache.struct()
    _check(lib().dqk_dequant_reference(C.byref(s), _ptr(k), _ptr(v), _stream(stream)),
           "dqk_dequant_reference")
    return k, v


def bf16_decode_workspace_bytes(batch, hq, hkv, d, ld_t, split_tokens=0) -> int:
    """Workspace bytes of the unpruned bf16 comparator for this shape and split."""
    out = C.c_size_t(0)
    _check(lib().dqk_bf16_decode_workspace_bytes(batch, hq, hkv, d, ld_t, split_tokens,
                                                 C.byref(out)), "dqk_bf16_decode_workspace_bytes")
    return int(out.value)


def bf16_decode_attention(q, k, v, lengths, sm_scale: float, split_tokens: int = 0, out=None,
                          workspace=None, stream=None):
    """The unpruned bf16 comparator: plain decode attention over raw keys and values.
    q [batch][hq][d] bf16; k/v [batch][hkv][ld_t][d] bf16; lengths [batch] int32;
    returns out [batch][hq][d] fp32."""
    torch = _torch()
    batch, hq, d = q.shape
    hkv, ld_t = int(k.shape[1]), int(k.shape[2])
    if out is None:
        out = torch.empty((batch, hq, d), dtype=torch.float32, device=q.device)
    if workspace is None:
        nb = bf16_decode_workspace_bytes(batch, hq, hkv, d, ld_t, split_tokens)
        workspace = torch.empty(max(nb, 16), dtype=torch.uint8, device=q.device)
    for t in (q, k, v):
        if t.dtype != torch.bfloat16:
            raise DqkError("bf16 decode takes bfloat16 q, k, v")
    _check(lib().dqk_bf16_decode_attention(_ptr(q), _ptr(k), _ptr(v), _ptr(lengths), batch, hq,
                                           hkv, d, ld_t, float(sm_scale), split_tokens, _ptr(out),
                                           _ptr(workspace),
                                           workspace.numel() * workspace.element_size(),
                                           _stream(stream)),
           "dqk_bf16_decode_attention")
    return out


def debug_f16_from_f32(x, stream=None):
    """The device's fp32 -> fp16 conversion (the one every stored scale and channel-0
    key uses), element-wise; returns the fp16 bit patterns as int16."""
    torch = _torch()
    out = torch.empty(x.shape, dtype=torch.int16, device=x.device)   # fp16 bits
    _check(lib().dqk_debug_f16_from_f32(_ptr(x), _ptr(out), x.numel(), _stream(stream)),
           "dqk_debug_f16_from_f32")
    return out


STREAM_READ_SINK_WORDS = 8192


def stream_read(buf, sink=None, stream=None):
    """Read every byte of the device tensor `buf` once (a plain streaming kernel;
    a measurement aid).  Returns the sink [8192] int32 tensor, whose XOR is the XOR
    of the buffer's 32-bit words."""
    torch = _torch()
    if sink is None:
        sink = torch.empty(STREAM_READ_SINK_WORDS, dtype=torch.int32, device=buf.device)
    _check(lib().dqk_stream_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink),
                                 _stream(stream)), "dqk_stream_read")
    return sink


def stream_read_config(buf, workgroups: int, loads_in_flight: int, sink=None, stream=None):
    """The read probe with its launch shape given (dqk_stream_read_config)."""
    torch = _torch()
    if sink is None:
        sink = torch.empty(STREAM_READ_SINK_WORDS, dtype=torch.int32, device=buf.device)
    _check(lib().dqk_stream_read_config(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink),
                                        int(workgroups), int(loads_in_flight), _stream(stream)),
           "dqk_stream_read_config")
    return sink
