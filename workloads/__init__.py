"""Seeded synthetic inputs for the Dual-QK decode path.

This module only draws random numbers and lays them out.  It holds none of the
method's arithmetic: no transform is applied, nothing is quantized, nothing is
selected.  The paired transforms A and B are inputs here because building them
from calibrated statistics (Dual-QK abstract, "partial key whitening with a
query-aligned basis") needs trained-model activations that are not available.
Both the CPU oracle and the GPU path take their inputs from here.

Workload shapes follow the five decode configurations the build is measured on
(tiny fp32 sanity case, GQA 32/8 at 8K, a 64-step append+decode loop at 32K,
128K context with a sparsity sweep, and a ragged batch of 16 at up to 64K).

Seeding: every stream is ``np.random.default_rng(SeedSequence([seed, cid, kind, ...]))``.
K and V come from one stream per (batch row, KV head), so any unit can be
regenerated on its own without drawing the whole cache.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Tuple

import numpy as np

# Stream kinds inside one workload.
_GLOBAL, _KEYS, _VALUES, _QUERIES, _LENGTHS = 0, 1, 2, 3, 4


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    cid: int                 # workload id used in the seed
    batch: int
    hq: int
    hkv: int
    d: int
    ctx: Tuple[int, ...]     # prefilled context length per batch row
    cap: int                 # cache capacity per sequence (multiple of 32)
    steps: int               # append+decode steps after the prefill
    sparsity: Tuple[int, ...]  # query-channel sparsity sweep, percent
    dtype: str               # "f32" or "bf16" for q/k/v
    seed: int = 0
    student_t_queries: bool = False
    random_outlier_channels: int = 0   # extra x10 key channels (tiny case)
    log_uniform_key_scales: bool = False

    @property
    def group(self) -> int:
        return self.hq // self.hkv

    def describe(self) -> str:
        lens = (f"{min(self.ctx)}..{max(self.ctx)}" if len(set(self.ctx)) > 1
                else str(self.ctx[0]))
        return (f"{self.name}: batch {self.batch}, heads {self.hq}/{self.hkv}, "
                f"head_dim {self.d}, ctx {lens}, cap {self.cap}, {self.dtype}, "
                f"sparsity {list(self.sparsity)}%, steps {self.steps}")


def _cap_for(n: int) -> int:
    return (n + 31) // 32 * 32


def _ragged_lengths(seed: int, cid: int, batch: int, lo: int, hi: int) -> Tuple[int, ...]:
    rng = np.random.default_rng(np.random.SeedSequence([seed, cid, _LENGTHS]))
    return tuple(int(x) for x in rng.integers(lo, hi, size=batch, endpoint=True))


def workload(name: str, *, batch: Optional[int] = None, ctx: Optional[int] = None,
             steps: Optional[int] = None) -> Workload:
    """Named workloads.  ``batch``/``ctx``/``steps`` shrink a workload for fast tests
    (same distributions, smaller shapes)."""
    if name == "tiny":      # 1 seq, 1/1 heads, D 64, 1024 tokens, fp32, 40%
        b = batch or 1
        t = ctx or 1024
        return Workload("tiny", 1, b, 1, 1, 64, (t,) * b, _cap_for(t + (steps or 0)),
                        steps or 0, (40,), "f32", random_outlier_channels=3)
    if name == "gqa8k":     # batch 4, 32/8 heads, D 128, 8K, bf16, 40%
        b = batch or 4
        t = ctx or 8192
        return Workload("gqa8k", 2, b, 32, 8, 128, (t,) * b, _cap_for(t + (steps or 0)),
                        steps or 0, (40,), "bf16", log_uniform_key_scales=True)
    if name == "append32k":  # batch 8, 32/8, 32K prefill + 64 single-token steps
        b = batch or 8
        t = ctx or 32768
        s = 64 if steps is None else steps
        return Workload("append32k", 3, b, 32, 8, 128, (t,) * b, _cap_for(t + s), s,
                        (40,), "bf16", log_uniform_key_scales=True)
    if name == "ctx128k":   # batch 1, 32/8, 128K, sparsity sweep 0/40/60
        b = batch or 1
        t = ctx or 131072
        return Workload("ctx128k", 4, b, 32, 8, 128, (t,) * b, _cap_for(t + (steps or 0)),
                        steps or 0, (0, 40, 60), "bf16", log_uniform_key_scales=True)
    if name == "ragged64k":  # batch 16, 64/8, ragged 16K..64K, Student-t queries
        b = batch or 16
        hi = ctx or 65536
        lo = max(1, hi // 4)
        lens = _ragged_lengths(0, 5, b, lo, hi)
        return Workload("ragged64k", 5, b, 64, 8, 128, lens, _cap_for(hi + (steps or 0)),
                        steps or 0, (40,), "bf16", student_t_queries=True,
                        log_uniform_key_scales=True)
    raise KeyError(name)


WORKLOADS = ("tiny", "gqa8k", "append32k", "ctx128k", "ragged64k")


def custom(name: str, cid: int, batch: int, hq: int, hkv: int, d: int,
           ctx: List[int], cap: int, dtype: str = "bf16", steps: int = 0,
           sparsity=(40,), **kw) -> Workload:
    """A workload with explicit shapes (edge-case tests)."""
    assert cap % 32 == 0 and hq % hkv == 0
    return Workload(name, cid, batch, hq, hkv, d, tuple(int(x) for x in ctx), cap, steps,
                    tuple(sparsity), dtype, **kw)


# ----------------------------------------------------------------------------- rounding

def round_bf16(x: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Round fp32 values to bf16 (round to nearest even).  Returns (fp32 values that
    are exactly bf16, uint16 bit patterns).  Inputs are finite draws."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    u32 = u.astype(np.uint32)
    return u32.view(np.float32), (u32 >> 16).astype(np.uint16)


def _finish(x: np.ndarray, dtype: str) -> np.ndarray:
    x = x.astype(np.float32)
    if dtype == "bf16":
        x, _ = round_bf16(x)
    return x


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Bit patterns of fp32 values that are already exact bf16 numbers."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    lo = x.view(np.uint32) & 0xFFFF
    assert not lo.any(), "value is not an exact bf16 number"
    return (x.view(np.uint32) >> 16).astype(np.uint16)


# ----------------------------------------------------------------------------- draws

def _global_rng(wl: Workload) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([wl.seed, wl.cid, _GLOBAL]))


def _global_draws(wl: Workload):
    """Transforms, per-channel key scales and outlier channels, in that order."""
    rng = _global_rng(wl)
    d = wl.d
    a64 = np.eye(d)[None] + 0.1 * rng.standard_normal((wl.hkv, d, d))
    a32 = a64.astype(np.float32)
    if wl.log_uniform_key_scales:
        kscale = np.exp(rng.uniform(np.log(0.5), np.log(20.0), size=(wl.hkv, d)))
    else:
        kscale = np.ones((wl.hkv, d))
    kscale[:, 0] *= 8.0
    if wl.random_outlier_channels:
        for g in range(wl.hkv):
            ch = rng.choice(np.arange(1, d), size=wl.random_outlier_channels, replace=False)
            kscale[g, ch] *= 10.0
    return a32, kscale.astype(np.float32)


def transforms(wl: Workload) -> Tuple[np.ndarray, np.ndarray]:
    """Per-KV-head paired transforms: A = I + 0.1*N(0,1) (rounded to fp32) and
    B = inverse(A)^T evaluated in fp64 from the fp32 A, rounded to fp32.
    Shapes [hkv][d][d], row-major; q' = q A and k' = k B act on row vectors."""
    a32, _ = _global_draws(wl)
    b = np.stack([np.linalg.inv(a32[g].astype(np.float64)).T for g in range(wl.hkv)])
    return np.ascontiguousarray(a32), np.ascontiguousarray(b.astype(np.float32))


def key_scales(wl: Workload) -> np.ndarray:
    return _global_draws(wl)[1]


def final_lengths(wl: Workload) -> np.ndarray:
    return np.array(wl.ctx, dtype=np.int64) + wl.steps


def unit_kv(wl: Workload, b: int, g: int, t0: int = 0, n: Optional[int] = None,
            kscale: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Keys and values of one (batch row, KV head) for token positions [t0, t0+n).
    Positions past the prefill are the tokens appended by the decode steps.
    Returns fp32 arrays [n][d] (values exactly bf16 when the workload is bf16)."""
    ctx = int(wl.ctx[b])
    total = ctx + wl.steps
    if n is None:
        n = total - t0
    assert 0 <= t0 and t0 + n <= total
    if kscale is None:
        kscale = key_scales(wl)

    def draw(kind: int, part: int, rows: int, lo: int, hi: int) -> np.ndarray:
        if hi <= lo:
            return np.zeros((0, wl.d), dtype=np.float32)
        r = np.random.default_rng(np.random.SeedSequence([wl.seed, wl.cid, kind, b, g, part]))
        return r.standard_normal((rows, wl.d), dtype=np.float32)[lo:hi]

    # The prefill and the appended decode-step tokens come from separate streams,
    # each drawn whole so any slice is the same numbers.
    p_lo, p_hi = min(t0, ctx), min(t0 + n, ctx)
    s_lo, s_hi = max(t0, ctx) - ctx, max(t0 + n, ctx) - ctx
    k = np.concatenate([draw(_KEYS, 0, ctx, p_lo, p_hi), draw(_KEYS, 1, wl.steps, s_lo, s_hi)])
    v = np.concatenate([draw(_VALUES, 0, ctx, p_lo, p_hi),
                        draw(_VALUES, 1, wl.steps, s_lo, s_hi)])
    k = k * kscale[g][None, :]
    v = v.copy()
    v[:, 0] *= 8.0
    return _finish(k, wl.dtype), _finish(v, wl.dtype)


def queries(wl: Workload, step: int = 0) -> np.ndarray:
    """Decode queries for one step: [batch][hq][d] fp32 (exact bf16 when bf16)."""
    rng = np.random.default_rng(np.random.SeedSequence([wl.seed, wl.cid, _QUERIES, step]))
    shape = (wl.batch, wl.hq, wl.d)
    if wl.student_t_queries:
        q = rng.standard_t(3.0, size=shape)
    else:
        q = rng.standard_normal(shape)
    q = q.astype(np.float32)
    q[:, :, 0] *= 8.0
    return _finish(q, wl.dtype)


def prefill_kv(wl: Workload, units=None):
    """Prefill keys/values for all (or the listed) units as dense arrays
    [batch][hkv][cap][d] (zero past each row's prefill length)."""
    kscale = key_scales(wl)
    k = np.zeros((wl.batch, wl.hkv, wl.cap, wl.d), dtype=np.float32)
    v = np.zeros_like(k)
    for b in range(wl.batch):
        for g in range(wl.hkv):
            if units is not None and (b, g) not in units:
                continue
            kk, vv = unit_kv(wl, b, g, 0, int(wl.ctx[b]), kscale)
            k[b, g, :kk.shape[0]] = kk
            v[b, g, :vv.shape[0]] = vv
    return k, v


def step_kv(wl: Workload, step: int) -> Tuple[np.ndarray, np.ndarray]:
    """The single token each batch row appends at decode step ``step``:
    [batch][hkv][1][d]."""
    kscale = key_scales(wl)
    k = np.zeros((wl.batch, wl.hkv, 1, wl.d), dtype=np.float32)
    v = np.zeros_like(k)
    for b in range(wl.batch):
        for g in range(wl.hkv):
            kk, vv = unit_kv(wl, b, g, int(wl.ctx[b]) + step, 1, kscale)
            k[b, g] = kk
            v[b, g] = vv
    return k, v


def default_sm_scale(d: int) -> float:
    return float(np.float32(1.0 / np.sqrt(d)))
