"""Helpers for the GPU parity tests: moving seeded inputs to the device, reading
cache planes back, and the error metric.  No arithmetic of the method lives here."""
from __future__ import annotations

import sys

import numpy as np

import workloads as W

REL_TOL = 2e-3   # max over heads of ||o - o_ref||_inf / ||o_ref||_inf


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def torch():
    import torch as T
    return T


def dev_f32(x):
    T = torch()
    return T.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def dev_i32(x):
    T = torch()
    return T.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).cuda()


def dev_input(x, dtype: str):
    """fp32 values (exact bf16 numbers when dtype is bf16) -> device tensor."""
    T = torch()
    if dtype == "bf16":
        bits = W.bf16_bits(x)
        return T.from_numpy(bits.view(np.int16)).cuda().view(T.bfloat16)
    return dev_f32(x)


def planes_np(cache):
    """Device cache planes as numpy arrays with the oracle's dtypes."""
    out = {}
    for name, t in cache.planes().items():
        a = t.cpu().numpy()
        if name in ("k_scales", "k_ch0", "v_scales"):
            a = a.view(np.uint16)
        elif name == "v_codes":
            a = a.view(np.uint32)
        out[name] = a
    return out


def assert_same_cache(gpu, orc_cache, unit_map=None):
    """Byte-equal planes.  unit_map: list of ((gpu b, g), (oracle b, g)); default all.
    Tail rows are compared where defined (row < len mod 32)."""
    o = orc_cache.planes()
    if unit_map is None:
        unit_map = [((b, g), (b, g)) for b in range(orc_cache.batch) for g in range(orc_cache.hkv)]
    for (gb, gg), (ob, og) in unit_map:
        assert gpu["lengths"][gb] == o["lengths"][ob], "lengths"
        for name in ("k_codes", "k_scales", "k_ch0", "v_codes", "v_scales"):
            a, b = gpu[name][gb, gg], o[name][ob, og]
            if not np.array_equal(a, b):
                bad = np.argwhere(a != b)
                raise AssertionError(f"{name} differs at unit ({gb},{gg}) first {bad[:5].tolist()} "
                                     f"gpu {a[tuple(bad[0])]} oracle {b[tuple(bad[0])]}")
        r = int(o["lengths"][ob]) % 32
        assert np.array_equal(gpu["k_tail"][gb, gg, :r], o["k_tail"][ob, og, :r]), "k_tail"


def rel_err(out, ref):
    """Per (b, h) ||out - ref||_inf / ||ref||_inf, max over heads (0/0 -> 0)."""
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = np.abs(out - ref).max(axis=-1)
    den = np.abs(ref).max(axis=-1)
    r = np.where(den > 0, num / np.where(den > 0, den, 1), np.where(num > 0, np.inf, 0.0))
    return float(r.max()) if r.size else 0.0
