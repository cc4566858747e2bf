"""Python access to the plain CPU oracle (``dqk_oracle.c``).

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` use this module to check and time the GPU
library; the GPU library never imports it.  Arrays are numpy, on the host.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "dqk_oracle.c")
LIB = os.path.join(HERE, "libdqk_oracle.so")

CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
          "-fno-fast-math", "-Wall", "-Wextra"]


def build(verbose: bool = False) -> str:
    """Compile the oracle with gcc (always rebuilds)."""
    tmp = LIB + ".tmp"
    cmd = ["gcc", *CFLAGS, SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build()
        _lib = C.CDLL(LIB)
        _declare(_lib)
    return _lib


class _Cache(C.Structure):
    _fields_ = [("batch", C.c_int32), ("hkv", C.c_int32), ("d", C.c_int32), ("cap", C.c_int32),
                ("k_codes", C.c_void_p), ("k_scales", C.c_void_p), ("k_ch0", C.c_void_p),
                ("k_tail", C.c_void_p), ("v_codes", C.c_void_p), ("v_scales", C.c_void_p),
                ("lengths", C.c_void_p)]


P = C.c_void_p


def _declare(L):
    L.dqko_f16_from_f32.restype = C.c_uint16
    L.dqko_f16_from_f32.argtypes = [C.c_float]
    L.dqko_f32_from_f16.restype = C.c_float
    L.dqko_f32_from_f16.argtypes = [C.c_uint16]
    L.dqko_f16_from_f32_n.argtypes = [P, C.c_size_t, P]
    L.dqko_f32_from_f16_n.argtypes = [P, C.c_size_t, P]
    L.dqko_transform.argtypes = [P, P, C.c_int, P]
    L.dqko_quantize32.argtypes = [P, C.c_ssize_t, P, P]
    L.dqko_keep_count.restype = C.c_int
    L.dqko_keep_count.argtypes = [C.c_int, C.c_int]
    L.dqko_select.argtypes = [P, C.c_int, C.c_int, P]
    L.dqko_queries.argtypes = [P, P, C.c_int, C.c_int, C.c_int, C.c_int, C.c_int, P, P]
    L.dqko_select_shared.argtypes = [P, C.c_int, C.c_int, C.c_int, P]
    L.dqko_queries_shared.argtypes = [P, P, C.c_int, C.c_int, C.c_int, C.c_int, C.c_int, P, P]
    L.dqko_append.argtypes = [C.POINTER(_Cache), P, P, P, P, C.c_int32]
    L.dqko_dequant.argtypes = [C.POINTER(_Cache), P, P]
    L.dqko_cache_grow.argtypes = [C.POINTER(_Cache), C.POINTER(_Cache)]
    L.dqko_attend_dense.argtypes = [P, P, C.c_int, P, P, C.c_int, C.c_int, C.c_ssize_t,
                                    C.c_double, P]
    L.dqko_decode.argtypes = [C.POINTER(_Cache), P, P, C.c_int, C.c_int, C.c_double, P, P,
                              C.c_int]
    L.dqko_plain_attention.argtypes = [P, P, P, P, C.c_int, C.c_int, C.c_int, C.c_int,
                                       C.c_int, C.c_double, P]
    L.dqko_decode_bytes.argtypes = [C.POINTER(_Cache), P, C.c_int, C.c_int, P]


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(C.c_void_p)


def _f32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32)


# ----------------------------------------------------------------------------- scalar pieces

def f16_from_f32(x) -> np.ndarray:
    x = _f32(x)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().dqko_f16_from_f32_n(_p(x), x.size, _p(out))
    return out


def f32_from_f16(h) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.empty(h.shape, dtype=np.float32)
    lib().dqko_f32_from_f16_n(_p(h), h.size, _p(out))
    return out


def transform(x, m) -> np.ndarray:
    """y = x M for one row vector x[d]."""
    x, m = _f32(x), _f32(m)
    d = x.shape[-1]
    y = np.empty(d, dtype=np.float32)
    lib().dqko_transform(_p(x), _p(m), d, _p(y))
    return y


def quantize32(x):
    """Returns (sigma bits uint16, codes uint8[32])."""
    x = _f32(x)
    assert x.shape == (32,)
    s = np.zeros(1, dtype=np.uint16)
    u = np.zeros(32, dtype=np.uint8)
    lib().dqko_quantize32(_p(x), 1, _p(s), _p(u))
    return int(s[0]), u


def keep_count(d: int, sparsity_pct: int) -> int:
    return int(lib().dqko_keep_count(d, sparsity_pct))


def select(qp, keep: int) -> np.ndarray:
    qp = _f32(qp)
    idx = np.zeros(keep, dtype=np.int32)
    lib().dqko_select(_p(qp), qp.shape[-1], keep, _p(idx))
    return idx


def queries(q, a, hkv: int, keep: int):
    """q [batch][hq][d], a [hkv][d][d] -> (q' [batch][hq][d], idx [batch][hq][keep])."""
    q, a = _f32(q), _f32(a)
    batch, hq, d = q.shape
    qp = np.zeros_like(q)
    idx = np.zeros((batch, hq, keep), dtype=np.int32)
    lib().dqko_queries(_p(q), _p(a), batch, hq, hkv, d, keep, _p(qp), _p(idx))
    return qp, idx


def select_shared(qp_group, keep: int) -> np.ndarray:
    """One kept set for a group of query heads: qp_group [grp][d]."""
    qp_group = _f32(qp_group)
    grp, d = qp_group.shape
    idx = np.zeros(keep, dtype=np.int32)
    lib().dqko_select_shared(_p(qp_group), grp, d, keep, _p(idx))
    return idx


def queries_shared(q, a, hkv: int, keep: int):
    """q [batch][hq][d], a [hkv][d][d] -> (q' [batch][hq][d], idx [batch][hkv][keep])
    with one group-shared kept set per (batch row, KV head)."""
    q, a = _f32(q), _f32(a)
    batch, hq, d = q.shape
    qp = np.zeros_like(q)
    idx = np.zeros((batch, hkv, keep), dtype=np.int32)
    lib().dqko_queries_shared(_p(q), _p(a), batch, hq, hkv, d, keep, _p(qp), _p(idx))
    return qp, idx


def per_head(idx_shared, group: int) -> np.ndarray:
    """Group-shared kept sets [batch][hkv][keep] laid out per query head
    [batch][hkv*group][keep] (every head of a group keeps its group's set), the
    form the oracle's decode takes."""
    return np.ascontiguousarray(np.repeat(np.asarray(idx_shared, dtype=np.int32), group, axis=1))


# ----------------------------------------------------------------------------- cache

class Cache:
    """Host-side stored cache in the packed layout (all planes zeroed)."""

    def __init__(self, batch: int, hkv: int, d: int, cap: int):
        assert cap % 32 == 0 and d % 32 == 0
        self.batch, self.hkv, self.d, self.cap = batch, hkv, d, cap
        u = batch * hkv
        self.k_codes = np.zeros((batch, hkv, d, cap // 4), dtype=np.uint8)
        self.k_scales = np.zeros((batch, hkv, d, cap // 32), dtype=np.uint16)
        self.k_ch0 = np.zeros((batch, hkv, cap), dtype=np.uint16)
        self.k_tail = np.zeros((batch, hkv, 32, d), dtype=np.float32)
        self.v_codes = np.zeros((batch, hkv, cap // 16, d), dtype=np.uint32)
        self.v_scales = np.zeros((batch, hkv, cap, d // 32), dtype=np.uint16)
        self.lengths = np.zeros(batch, dtype=np.int32)
        del u

    def _struct(self) -> _Cache:
        return _Cache(self.batch, self.hkv, self.d, self.cap, _p(self.k_codes).value,
                      _p(self.k_scales).value, _p(self.k_ch0).value, _p(self.k_tail).value,
                      _p(self.v_codes).value, _p(self.v_scales).value, _p(self.lengths).value)

    def append(self, k_new, v_new, bm, n_new: Sequence[int]):
        """k_new/v_new: [batch][hkv][max_new][d] fp32 (bf16 inputs widened exactly)."""
        k_new, v_new, bm = _f32(k_new), _f32(v_new), _f32(bm)
        max_new = k_new.shape[2]
        n = np.ascontiguousarray(n_new, dtype=np.int32)
        s = self._struct()
        lib().dqko_append(C.byref(s), _p(k_new), _p(v_new), _p(bm), _p(n), max_new)

    def grow(self, cap: int) -> "Cache":
        """A cache of capacity `cap` (>= this one's) holding the same contents."""
        assert cap >= self.cap and cap % 32 == 0
        out = Cache(self.batch, self.hkv, self.d, cap)
        s, t = self._struct(), out._struct()
        lib().dqko_cache_grow(C.byref(s), C.byref(t))
        return out

    def dequant(self):
        k = np.zeros((self.batch, self.hkv, self.cap, self.d), dtype=np.float32)
        v = np.zeros_like(k)
        s = self._struct()
        lib().dqko_dequant(C.byref(s), _p(k), _p(v))
        return k, v

    def decode(self, qp, idx, sm: float, heads_mask: Optional[np.ndarray] = None,
               nthreads: int = 0) -> np.ndarray:
        qp = _f32(qp)
        idx = np.ascontiguousarray(idx, dtype=np.int32)
        batch, hq, d = qp.shape
        keep = idx.shape[-1]
        out = np.zeros((batch, hq, d), dtype=np.float32)
        mask = None if heads_mask is None else np.ascontiguousarray(heads_mask, dtype=np.uint8)
        s = self._struct()
        lib().dqko_decode(C.byref(s), _p(qp), _p(idx), hq, keep, float(sm), _p(out),
                          None if mask is None else _p(mask), nthreads)
        return out

    def decode_bytes(self, idx) -> np.ndarray:
        idx = np.ascontiguousarray(idx, dtype=np.int32)
        hq, keep = idx.shape[1], idx.shape[2]
        out = np.zeros(7, dtype=np.uint64)
        s = self._struct()
        lib().dqko_decode_bytes(C.byref(s), _p(idx), hq, keep, _p(out))
        return out

    def planes(self):
        return dict(k_codes=self.k_codes, k_scales=self.k_scales, k_ch0=self.k_ch0,
                    k_tail=self.k_tail, v_codes=self.v_codes, v_scales=self.v_scales,
                    lengths=self.lengths)


def attend_dense(qp, idx, k, v, sm: float) -> np.ndarray:
    """One head: qp[d], idx[keep], k/v [t][d] dense."""
    qp, k, v = _f32(qp), _f32(k), _f32(v)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    t, d = k.shape
    out = np.zeros(d, dtype=np.float32)
    lib().dqko_attend_dense(_p(qp), _p(idx), idx.size, _p(k), _p(v), t, d, d, float(sm), _p(out))
    return out


def plain_attention(q, k, v, lengths, sm: float) -> np.ndarray:
    """q [batch][hq][d]; k/v [batch][hkv][ld_t][d]; fp64 softmax(sm q K^T) V."""
    q, k, v = _f32(q), _f32(k), _f32(v)
    lengths = np.ascontiguousarray(lengths, dtype=np.int32)
    batch, hq, d = q.shape
    hkv, ld_t = k.shape[1], k.shape[2]
    out = np.zeros_like(q)
    lib().dqko_plain_attention(_p(q), _p(k), _p(v), _p(lengths), batch, hq, hkv, d, ld_t,
                               float(sm), _p(out))
    return out
