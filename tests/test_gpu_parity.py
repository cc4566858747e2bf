"""GPU parity: the HIP library through its C ABI against the CPU oracle.

Bit-exact: cache planes (codes, scales, channel 0, tail), q', selected channel
sets, the dense dequantized cache, the fp16 conversion.  Within 2e-3 (max over
heads of ||o - o_ref||_inf / ||o_ref||_inf): attention outputs.  Inputs are the
seeded synthetic workloads, at sizes the oracle finishes in seconds that still
span several splits and a ragged tail.
"""
import os

import numpy as np
import pytest
import torch

import bit_quantized_decode_dqk_amd as M
import workloads as W
from gpu_util import (REL_TOL, assert_same_cache, dev_f32, dev_i32, dev_input, planes_np,
                      rel_err, say)

pytestmark = pytest.mark.gpu


def _env_int(name: str, default: int) -> int:
    """Case count or seed of the seeded random sweeps below (environment override, for
    longer runs than the default suite's)."""
    return int(os.environ.get(name, default))


def _counts(wl, pos, n):
    return np.clip(np.array(wl.ctx) - pos, 0, n).astype(np.int32)


def build_gpu(wl, chunks=None, kv=None):
    a, b = W.transforms(wl)
    k, v = kv if kv is not None else W.prefill_kv(wl)
    cache = M.Cache(wl.batch, wl.hkv, wl.d, wl.cap)
    bm = dev_f32(b)
    chunks = chunks or [max(wl.ctx)]
    pos = 0
    for n in chunks:
        n = min(n, wl.cap - pos, max(wl.ctx) - pos)
        if n <= 0:
            break
        M.transform_quantize_append(cache, dev_input(k[:, :, pos:pos + n], wl.dtype),
                                    dev_input(v[:, :, pos:pos + n], wl.dtype), bm,
                                    dev_i32(_counts(wl, pos, n)))
        pos += n
    return cache, a, b, k, v


def build_oracle(orc, wl, k, v, b):
    c = orc.Cache(wl.batch, wl.hkv, wl.d, wl.cap)
    n = max(wl.ctx)
    c.append(k[:, :, :n], v[:, :, :n], b, list(wl.ctx))
    return c


def gpu_queries(wl, q, a, keep):
    qp, idx = M.select_channels(dev_input(q, wl.dtype), dev_f32(a), wl.hkv, keep)
    return qp, idx


# ----------------------------------------------------------------------------- conversion

def test_f16_conversion_matches_oracle(orc):
    """Every positive pattern with biased exponent 100..143, both signs of a
    stride through it, zeros/infinities, and random patterns."""
    say("f16 conversion: exponents 100..143")
    lo, hi = 100 << 23, 144 << 23
    step = 1 << 26
    for start in range(lo, hi, step):
        bits = np.arange(start, min(start + step, hi), dtype=np.uint32)
        x = bits.view(np.float32)
        got = M.debug_f16_from_f32(dev_f32(x)).cpu().numpy().view(np.uint16)
        assert np.array_equal(got, orc.f16_from_f32(x)), hex(start)
    rnd = np.random.default_rng(5).integers(0, 1 << 32, size=1 << 22, dtype=np.uint64).astype(np.uint32)
    x = rnd.view(np.float32)
    x = x[~np.isnan(x)]
    neg = np.arange(lo, hi, 997, dtype=np.uint32) | np.uint32(0x80000000)
    x = np.concatenate([x, neg.view(np.float32),
                        np.array([0.0, -0.0, np.inf, -np.inf], dtype=np.float32)])
    got = M.debug_f16_from_f32(dev_f32(x)).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, orc.f16_from_f32(x))


# ----------------------------------------------------------------------------- append

def test_append_tiny_bulk_single_and_mixed(orc):
    wl = W.workload("tiny")
    say("append tiny bulk")
    g_bulk, a, b, k, v = build_gpu(wl)
    ref = build_oracle(orc, wl, k, v, b)
    assert_same_cache(planes_np(g_bulk), ref)
    say("append tiny single-token x1024")
    g_one, *_ = build_gpu(wl, [1] * 1024, kv=(k, v))
    assert_same_cache(planes_np(g_one), ref)
    say("append tiny mixed chunks")
    g_mix, *_ = build_gpu(wl, [31, 1, 33, 2, 100, 64, 17, 16, 760], kv=(k, v))
    assert_same_cache(planes_np(g_mix), ref)


@pytest.mark.parametrize("chunks", [[1000], [500, 500], [31, 200, 769], [1] * 70 + [930]])
def test_append_gqa_ragged(orc, chunks):
    wl = W.custom("ragged-append", 21, 3, 32, 8, 128, [1000, 33, 31], 1024, "bf16",
                  log_uniform_key_scales=True)
    say("append ragged", chunks[:3])
    g, a, b, k, v = build_gpu(wl, chunks)
    ref = build_oracle(orc, wl, k, v, b)
    assert_same_cache(planes_np(g), ref)


def _random_append_cases(n: int, seed: int):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        d = int(rng.choice([64, 128]))
        hkv = int(rng.integers(1, 4))
        batch = int(rng.integers(1, 4))
        cap = int(rng.integers(2, 40)) * 32
        lens = [int(x) for x in rng.integers(0, cap + 40, size=batch)]   # some past capacity
        chunks = []
        while sum(chunks) < max(lens) + 8:
            chunks.append(int(rng.choice([1, 1, 2, 3, 5, 31, 32, 33, 64, 200])))
        dtype = "bf16" if rng.random() < 0.6 else "f32"
        out.append((i, d, hkv, batch, cap, lens, chunks, dtype))
    return out


@pytest.mark.parametrize("case", _random_append_cases(_env_int("DQK_RANDOM_APPEND_CASES", 12),
                                                    _env_int("DQK_RANDOM_SEED", 77)),
                         ids=lambda c: f"a{c[0]}")
def test_append_random_chunks(orc, case):
    """Random chunk sequences (one-token, small and bulk appends, so both the
    held-column and the bulk forms run) with ragged per-row counts, some rows
    filled to the capacity: every plane byte-equal to the oracle's one-call
    append of the same tokens."""
    i, d, hkv, batch, cap, lens, chunks, dtype = case
    ctx = [min(n, cap) for n in lens]
    wl = W.custom(f"rapp{i}", 90 + i, batch, hkv, hkv, d, ctx, cap, dtype,
                  log_uniform_key_scales=(dtype == "bf16"))
    say("append random", i, "d", d, "hkv", hkv, "cap", cap, "lens", ctx, "chunks", chunks[:6], dtype)
    g, a, b, k, v = build_gpu(wl, chunks)
    assert_same_cache(planes_np(g), build_oracle(orc, wl, k, v, b))


@pytest.mark.parametrize("d", [64, 128])
def test_append_bulk_with_unaligned_transform(orc, d):
    """A bulk append whose B is not 16-byte aligned (one float into a buffer) takes
    the per-channel streaming form instead of the blocked one: the same planes."""
    wl = W.custom(f"unaligned-b{d}", 26, 2, 8, 2, d, [300, 77], 320, "bf16", log_uniform_key_scales=True)
    a, b = W.transforms(wl)
    k, v = W.prefill_kv(wl)
    buf = torch.zeros(b.size + 1, dtype=torch.float32, device="cuda")
    buf[1:] = dev_f32(b).reshape(-1)
    b_off = buf[1:].view(b.shape)   # 4 bytes past a 16-byte boundary
    assert b_off.data_ptr() % 16 == 4
    g = M.Cache(wl.batch, wl.hkv, wl.d, wl.cap)
    n = max(wl.ctx)
    M.transform_quantize_append(g, dev_input(k[:, :, :n], wl.dtype), dev_input(v[:, :, :n], wl.dtype),
                                b_off, dev_i32(list(wl.ctx)))
    assert_same_cache(planes_np(g), build_oracle(orc, wl, k, v, b))


def test_append_head_dim_64_and_capacity_clamp(orc):
    wl = W.custom("d64", 22, 2, 4, 2, 64, [96, 64], 96, "f32", random_outlier_channels=3)
    g, a, b, k, v = build_gpu(wl)
    ref = build_oracle(orc, wl, k, v, b)
    assert_same_cache(planes_np(g), ref)
    # appending past capacity is clamped on both sides
    extra = np.random.default_rng(1).standard_normal((2, 2, 40, 64)).astype(np.float32)
    M.transform_quantize_append(g, dev_f32(extra), dev_f32(extra), dev_f32(b), dev_i32([40, 40]))
    ref.append(extra, extra, b, [40, 40])
    assert list(ref.lengths) == [96, 96]
    assert_same_cache(planes_np(g), ref)


def test_dequant_matches_oracle(orc):
    wl = W.custom("dq", 23, 2, 8, 2, 128, [300, 77], 320, "bf16", log_uniform_key_scales=True)
    g, a, b, k, v = build_gpu(wl)
    ref = build_oracle(orc, wl, k, v, b)
    kg, vg = M.dequant_reference(g)
    ko, vo = ref.dequant()
    assert np.array_equal(kg.cpu().numpy(), ko)
    assert np.array_equal(vg.cpu().numpy(), vo)


# ----------------------------------------------------------------------------- select

@pytest.mark.parametrize("name", W.WORKLOADS)
def test_select_matches_oracle(orc, name):
    wl = W.workload(name)
    a, _ = W.transforms(wl)
    q = W.queries(wl)
    for keep in sorted({1, 2, orc.keep_count(wl.d, 60), orc.keep_count(wl.d, 40), wl.d - 1, wl.d}):
        qp, idx = gpu_queries(wl, q, a, keep)
        qpo, idxo = orc.queries(q, a, wl.hkv, keep)
        assert np.array_equal(qp.cpu().numpy().view(np.uint32), qpo.view(np.uint32)), keep
        assert np.array_equal(idx.cpu().numpy(), idxo), keep


@pytest.mark.parametrize("name,steps", [("tiny", (1, 1, 33)), ("gqa8k", (1, 40)), ("ragged64k", (1,))])
def test_fused_append_select_matches_separate_calls(orc, name, steps):
    """dqk_append_select against dqk_transform_quantize_append then
    dqk_select_channels on a twin cache: planes, q' and indices bitwise equal,
    for single-token and multi-token appends (a group flush and a straddle)."""
    kw = dict(batch=2, ctx=700 if name == "gqa8k" else 900) if name != "tiny" else {}
    wl = W.workload(name, steps=64, **kw)   # room for the appended tokens
    g1, a, b, k, v = build_gpu(wl)
    g2, _, _, _, _ = build_gpu(wl, kv=(k, v))
    a_d, b_d = dev_f32(a), dev_f32(b)
    keep = orc.keep_count(wl.d, 40)
    rng = np.random.default_rng(9)
    for st, n in enumerate(steps):
        say(f"fused append+select {name}: {n} token(s)")
        x = rng.standard_normal((wl.batch, wl.hkv, n, wl.d)).astype(np.float32)
        kx = dev_f32(x) if wl.dtype == "f32" else torch.from_numpy(x).to(torch.bfloat16).cuda()
        q = dev_input(W.queries(wl, 2 + st), wl.dtype)
        counts = dev_i32(np.full(wl.batch, n, dtype=np.int32))
        qp1, idx1 = M.append_select(g1, kx, kx, b_d, counts, q, a_d, keep)
        M.transform_quantize_append(g2, kx, kx, b_d, counts)
        qp2, idx2 = M.select_channels(q, a_d, wl.hkv, keep)
        torch.cuda.synchronize()
        p1, p2 = planes_np(g1), planes_np(g2)
        for nm in p1:
            assert np.array_equal(p1[nm], p2[nm]), (n, nm)
        assert not p1["lengths"][wl.batch:].any()   # arrival counters back at zero
        assert np.array_equal(qp1.cpu().numpy().view(np.uint32), qp2.cpu().numpy().view(np.uint32))
        assert np.array_equal(idx1.cpu().numpy(), idx2.cpu().numpy())


@pytest.mark.parametrize("d,hq,hkv,dtype", [(64, 2, 1, "f32"), (64, 8, 2, "bf16"), (64, 16, 2, "f32"),
                                              (128, 2, 1, "bf16"), (128, 16, 2, "f32")])
def test_select_and_fused_step_group_shapes(orc, d, hq, hkv, dtype):
    """Selection workgroups serve one query head (two at head_dim 64, where the
    second thread group takes the second head): every group size at both head
    dims, alone and in the fused append + select launch, against the oracle."""
    wl = W.custom(f"shape_d{d}_g{hq // hkv}", 40 + d + hq, 3, hq, hkv, d, [100, 37, 64], 192,
                  dtype=dtype)
    say("select/fused shapes", wl.describe())
    a, b = W.transforms(wl)
    q = W.queries(wl)
    for keep in sorted({1, 2, orc.keep_count(d, 40), d - 1, d}):
        qp, idx = gpu_queries(wl, q, a, keep)
        qpo, idxo = orc.queries(q, a, hkv, keep)
        assert np.array_equal(qp.cpu().numpy().view(np.uint32), qpo.view(np.uint32)), keep
        assert np.array_equal(idx.cpu().numpy(), idxo), keep
    g1, _, _, k, v = build_gpu(wl)
    g2, _, _, _, _ = build_gpu(wl, kv=(k, v))
    a_d, b_d = dev_f32(a), dev_f32(b)
    keep = orc.keep_count(d, 40)
    x = np.random.default_rng(11).standard_normal((wl.batch, hkv, 1, d)).astype(np.float32)
    kx = dev_input(W.round_bf16(x)[0] if dtype == "bf16" else x, dtype)
    qd = dev_input(W.queries(wl, 1), dtype)
    counts = dev_i32(np.ones(wl.batch, dtype=np.int32))
    qp1, idx1 = M.append_select(g1, kx, kx, b_d, counts, qd, a_d, keep)
    M.transform_quantize_append(g2, kx, kx, b_d, counts)
    qp2, idx2 = M.select_channels(qd, a_d, hkv, keep)
    torch.cuda.synchronize()
    p1, p2 = planes_np(g1), planes_np(g2)
    for nm in p1:
        assert np.array_equal(p1[nm], p2[nm]), nm
    assert np.array_equal(qp1.cpu().numpy().view(np.uint32), qp2.cpu().numpy().view(np.uint32))
    assert np.array_equal(idx1.cpu().numpy(), idx2.cpu().numpy())


def test_select_forced_ties(orc):
    """Duplicated, negated and signed-zero query channels: ties go to lower index."""
    d, hq = 128, 8
    rng = np.random.default_rng(30)
    q = rng.choice(np.array([0.0, -0.0, 1.0, -1.0, 2.5, -2.5], dtype=np.float32), (2, hq, d))
    eye = np.stack([np.eye(d, dtype=np.float32)] * 2)
    for keep in (1, 20, 77, 128):
        qp, idx = M.select_channels(dev_f32(q), dev_f32(eye), 2, keep)
        qpo, idxo = orc.queries(q, eye, 2, keep)
        assert np.array_equal(idx.cpu().numpy(), idxo)
        assert np.array_equal(qp.cpu().numpy().view(np.uint32), qpo.view(np.uint32))


# ----------------------------------------------------------------------------- decode

def decode_case(orc, wl, sparsity=40, sm_mult=1.0, splits=(0,), step=0):
    say("decode", wl.describe(), "s", sparsity, "sm x", sm_mult, "splits", splits)
    g, a, b, k, v = build_gpu(wl)
    ref = build_oracle(orc, wl, k, v, b)
    keep = orc.keep_count(wl.d, sparsity)
    q = W.queries(wl, step)
    qp, idx = gpu_queries(wl, q, a, keep)
    qpo, idxo = orc.queries(q, a, wl.hkv, keep)
    assert np.array_equal(idx.cpu().numpy(), idxo)
    sm = W.default_sm_scale(wl.d) * sm_mult
    o_ref = ref.decode(qpo, idxo, sm)
    outs = []
    for sp in splits:
        out = M.decode_attention(g, qp, idx, sm, split_tokens=sp).cpu().numpy()
        err = rel_err(out, o_ref)
        say(f"  split {sp}: max rel err {err:.3e}")
        assert err <= REL_TOL, (sp, err)
        outs.append(out)
    return g, outs, o_ref


def test_decode_tiny_full(orc):
    decode_case(orc, W.workload("tiny"), splits=(0, 32, 256, 1024))
    decode_case(orc, W.workload("tiny"), sm_mult=0.05, splits=(0, 96))


def test_decode_gqa_reduced(orc):
    wl = W.workload("gqa8k", batch=2, ctx=2500)
    decode_case(orc, wl, splits=(0, 64, 1024, 2048))
    decode_case(orc, wl, sm_mult=0.01, splits=(0, 352))
    decode_case(orc, wl, sparsity=0)
    decode_case(orc, wl, sparsity=60, sm_mult=0.02)


def test_decode_ragged_edges(orc):
    """Lengths 0, 1, 31, 32, 33, 64 and 95 in one batch (empty rows give zeros)."""
    wl = W.custom("edges", 24, 7, 16, 8, 128, [0, 1, 31, 32, 33, 64, 95], 96, "bf16",
                  log_uniform_key_scales=True)
    g, outs, o_ref = decode_case(orc, wl, splits=(0, 32, 64))
    for out in outs:
        assert not out[0].any()


@pytest.mark.parametrize("hq", [32, 64])
def test_decode_group4_empty_and_short_rows(orc, hq):
    """Rows of 0, 1, 31, 33 and 700 tokens on the matrix-core kernel (groups of
    four and eight, capacity a multiple of 64): an empty row gives zeros, the
    others match the oracle, for the default split and fixed ones."""
    wl = W.custom(f"g4-edges{hq}", 33, 5, hq, 8, 128, [0, 700, 1, 31, 33], 768, "bf16",
                  log_uniform_key_scales=True, student_t_queries=(hq == 64))
    g, outs, o_ref = decode_case(orc, wl, splits=(0, 64, 256, 768))
    for out in outs:
        assert not out[0].any()
    decode_case(orc, wl, sparsity=0, sm_mult=0.02, splits=(0,))


@pytest.mark.parametrize("hq", [4, 8])
def test_decode4_many_splits_one_dimensional_grid(orc, hq):
    """65538 splits of a row (32-token splits over a 2M-token capacity) do not fit
    the (KV head, row, split) grid of the matrix-core decodes (four and eight
    heads per workgroup): their work items are then numbered on a one-dimensional
    grid.  Most splits are empty; the result must match the oracle as for the
    default split and a 4096-token one."""
    cap = 2097216   # a multiple of 64; ceil(cap / 32) = 65538 splits
    wl = W.custom(f"many-splits{hq}", 61, 1, hq, 1, 64, [5000], cap, "bf16", log_uniform_key_scales=True)
    decode_case(orc, wl, splits=(32, 0, 4096))


def _random_cases(n: int, seed: int):
    """Seeded random shapes for the sweep below: head dimension, group size,
    capacity (a multiple of 64 or only of 32), ragged lengths with empty rows,
    keep, split and input type."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        d = int(rng.choice([64, 128]))
        g = int(rng.choice([1, 2, 4, 8]))
        hkv = int(rng.integers(1, 4))
        batch = int(rng.integers(1, 4))
        cap = int(rng.integers(2, 60)) * (64 if rng.random() < 0.6 else 32)
        lens = [int(x) for x in rng.integers(0, cap + 1, size=batch)]
        if rng.random() < 0.3:
            lens[int(rng.integers(0, batch))] = 0
        keep = int(rng.integers(1, d + 1))
        split = int(rng.choice([0, 0, 32 * int(rng.integers(1, 40)), 256 * int(rng.integers(1, 8))]))
        dtype = "bf16" if rng.random() < 0.7 else "f32"
        out.append((i, d, g, hkv, batch, cap, lens, keep, split, dtype))
    return out


@pytest.mark.parametrize("case", _random_cases(_env_int("DQK_RANDOM_CASES", 24), _env_int("DQK_RANDOM_SEED", 2024)),
                         ids=lambda c: f"r{c[0]}")
def test_decode_random_shapes(orc, case):
    """A seeded sweep of random shapes through append, select and decode against the
    oracle: planes bit-exact, q' and kept sets bit-exact, outputs within 2e-3 (an
    empty row gives zeros); the no-allocation decode bitwise equal to the workspace
    one; the group-shared selection and decode against the oracle's."""
    i, d, g, hkv, batch, cap, lens, keep, split, dtype = case
    wl = W.custom(f"rand{i}", 70 + i, batch, g * hkv, hkv, d, lens, cap, dtype,
                  log_uniform_key_scales=(dtype == "bf16"), student_t_queries=(g == 8))
    say("random", i, "d", d, "G", g, "hkv", hkv, "batch", batch, "cap", cap, "lens", lens,
        "keep", keep, "split", split, dtype)
    gc, a, b, k, v = build_gpu(wl)
    ref = build_oracle(orc, wl, k, v, b)
    assert_same_cache(planes_np(gc), ref)
    q = W.queries(wl)
    qp, idx = gpu_queries(wl, q, a, keep)
    qpo, idxo = orc.queries(q, a, wl.hkv, keep)
    assert np.array_equal(qp.cpu().numpy().view(np.uint32), qpo.view(np.uint32))
    assert np.array_equal(idx.cpu().numpy(), idxo)
    sm = W.default_sm_scale(d)
    o_ref = ref.decode(qpo, idxo, sm)
    out = M.decode_attention(gc, qp, idx, sm, split_tokens=split).cpu().numpy()
    err = rel_err(out, o_ref)
    say(f"  max rel err {err:.3e}")
    assert err <= REL_TOL, err
    for bb, n in enumerate(lens):
        if n == 0:
            assert not out[bb].any()
    # the entry point that allocates nothing: the same kernels and splits, bitwise
    if M.decode_workspace_bytes(gc, wl.hq, split) <= M.DECODE_SCRATCH_BYTES:
        na = M.decode_attention_noalloc(gc, qp, idx, sm, split_tokens=split).cpu().numpy()
        assert np.array_equal(na.view(np.uint32), out.view(np.uint32))
    # group-shared kept sets on the same cache
    qps, idxs = M.select_channels_shared(dev_input(q, wl.dtype), dev_f32(a), wl.hkv, keep)
    qpso, idxso = orc.queries_shared(q, a, wl.hkv, keep)
    assert np.array_equal(qps.cpu().numpy().view(np.uint32), qpso.view(np.uint32))
    assert np.array_equal(idxs.cpu().numpy(), idxso)
    o_sh = ref.decode(qpso, orc.per_head(idxso, wl.group), sm)
    sh = M.decode_attention_shared(gc, qps, idxs, sm, split_tokens=split).cpu().numpy()
    err = rel_err(sh, o_sh)
    say(f"  shared: max rel err {err:.3e}")
    assert err <= REL_TOL, err


@pytest.mark.parametrize("hq,hkv,d,cap", [(1, 1, 64, 1344), (2, 1, 64, 1344), (8, 1, 64, 1344),
                                          (4, 2, 128, 1344), (16, 2, 128, 1344),
                                          (64, 8, 128, 1344), (4, 1, 64, 1344), (8, 2, 64, 1376),
                                          (4, 1, 128, 1376), (8, 2, 128, 1344)])
def test_decode_group_sizes(orc, hq, hkv, d, cap):
    """Every GQA group size and head dimension; groups of four run the dedicated
    kernel, with capacities that are and are not multiples of 64 tokens."""
    wl = W.custom(f"g{hq}-{hkv}-{d}", 25, 2, hq, hkv, d, [700, min(1333, cap - 11)], cap, "bf16",
                  log_uniform_key_scales=True, student_t_queries=(hq == 64))
    decode_case(orc, wl, splits=(0, 128))
    decode_case(orc, wl, sm_mult=0.02, splits=(0,))


@pytest.mark.parametrize("d,lens,cap", [(128, [5000, 2049, 257], 5056), (64, [3000, 1, 700], 3008),
                                         (128, [4096, 4095, 31], 4096)])
def test_decode_group4_many_blocks(orc, d, lens, cap):
    """Groups of four with capacities that are multiples of 64 (the dedicated
    kernel): several 256-token blocks per workgroup, an odd block count, ragged
    rows, the exact tail, a row shorter than one key group, and split counts from
    one to more than the blocks."""
    wl = W.custom(f"g4-{d}", 27, len(lens), 32, 8, d, lens, cap, "bf16",
                  log_uniform_key_scales=True)
    decode_case(orc, wl, splits=(0, 64, 512, 1024, cap))
    decode_case(orc, wl, sparsity=0, sm_mult=0.02, splits=(0, 256))
    decode_case(orc, wl, sparsity=60, sm_mult=0.05, splits=(0,))


def test_decode_group4_chunk_sizes(orc):
    """Chunks of the dedicated kernel hold up to ten 256-token blocks, and a share
    of eleven runs as one chunk with an extra block: rows of 2304, 2200 (ragged,
    with its tail), 4300 and 5400 tokens, whole-block splits of 9, 10 and 11
    blocks, one split per row (21 blocks: 10 + 11), and the default."""
    wl = W.custom("g4-chunks", 31, 4, 32, 8, 128, [2304, 2200, 4300, 5400], 5440, "bf16",
                  log_uniform_key_scales=True)
    decode_case(orc, wl, splits=(2304, 2560, 2816, 5440, 0))


@pytest.mark.parametrize("hq,hkv,lens", [(4, 1, [3000, 1200, 64]), (12, 3, [2500]),
                                          (20, 5, [1800, 4000]), (8, 1, [3000, 1200, 64]),
                                          (24, 3, [2500]), (40, 5, [1800, 4000])])
def test_decode_group4_unit_counts(orc, hq, hkv, lens):
    """Groups of four and of eight with (row, KV head) counts that are not
    multiples of eight: the splits of one row and KV head run on different parts
    of the chip, and the combine joins the partials; groups of eight also with
    group-shared kept sets (the eight-head kernel's compact slots)."""
    wl = W.custom(f"g4-u{hkv}", 30 + hkv, len(lens), hq, hkv, 128, lens, 4032, "bf16",
                  log_uniform_key_scales=True)
    decode_case(orc, wl, splits=(0, 64, 256, 1024))
    if hq == 8 * hkv:
        decode_shared_case(orc, wl, splits=(0, 64, 1024))


def test_decode_workspace_reuse(orc):
    """One caller-provided workspace serves calls with different split counts
    and then a smaller cache: each output is bitwise the one a fresh workspace
    gives (nothing carries over between calls)."""
    wl = W.custom("g4-reuse", 28, 3, 32, 8, 128, [5000, 2049, 257], 5056, "bf16",
                  log_uniform_key_scales=True)
    g, a, b, k, v = build_gpu(wl)
    qp, idx = gpu_queries(wl, W.queries(wl), a, 77)
    sm = W.default_sm_scale(wl.d)
    splits = (0, 64, 512, 1024, 5056, 64, 0)
    nb = max(M.decode_workspace_bytes(g, wl.hq, sp) for sp in splits)
    ws = torch.full((nb,), 0xFF, dtype=torch.uint8, device="cuda")   # NaN bit patterns
    for sp in splits:
        say("workspace reuse, split", sp)
        fresh = M.decode_attention(g, qp, idx, sm, split_tokens=sp).cpu().numpy()
        out = torch.empty((wl.batch, wl.hq, wl.d), dtype=torch.float32, device="cuda")
        M.decode_attention(g, qp, idx, sm, sp, out, ws)
        assert np.array_equal(fresh.view(np.uint32), out.cpu().numpy().view(np.uint32)), sp
    wl1 = W.custom("g4-reuse1", 29, 1, 32, 8, 128, [3000], 5056, "bf16")
    g1, a1, _, _, _ = build_gpu(wl1)
    qp1, idx1 = gpu_queries(wl1, W.queries(wl1), a1, 77)
    fresh = M.decode_attention(g1, qp1, idx1, sm).cpu().numpy()
    out = torch.empty((1, wl1.hq, wl1.d), dtype=torch.float32, device="cuda")
    M.decode_attention(g1, qp1, idx1, sm, 0, out, ws)
    assert np.array_equal(fresh.view(np.uint32), out.cpu().numpy().view(np.uint32))


@pytest.mark.parametrize("ctx,sparsity,shared", [(131072, 40, False), (80000, 40, False),
                                                 (131072, 0, False), (131072, 60, False),
                                                 (131072, 40, True)])
def test_decode_ctx128k_sampled(orc, ctx, sparsity, shared):
    """The benchmark's workload at full size (batch 1, 32/8 heads, head_dim 128,
    131072 tokens, 40% sparsity, and the sweep's 0% and 60%) in its launch configuration (the default
    split: 512 workgroups, two per compute unit, the first-dispatched ones taking
    9/8 of the average share), at exactly 128K tokens, one past (one more block)
    and 33 past (a full key group and a tail token in the last block); and the
    same shape at 80000 tokens (about five blocks per split).  KV heads 0 and 5
    are checked: the oracle decodes each from a one-KV-head cache of that head's
    keys and values (the units are independent), built by the same appends."""
    wl = W.workload("ctx128k", ctx=ctx, steps=256)
    ctx, sm = int(wl.ctx[0]), W.default_sm_scale(wl.d)
    extras = (0, 1, 33)
    n_all = ctx + extras[-1]
    a, b = W.transforms(wl)
    kscale = W.key_scales(wl)
    say(f"ctx128k sampled ({ctx}): generating", n_all, "tokens x", wl.hkv, "KV heads")
    kb = np.zeros((1, wl.hkv, n_all, wl.d), dtype=np.uint16)
    vb = np.zeros_like(kb)
    sampled = {0: None, 5: None}
    for g in range(wl.hkv):
        kk, vv = W.unit_kv(wl, 0, g, 0, n_all, kscale)
        kb[0, g], vb[0, g] = W.bf16_bits(kk), W.bf16_bits(vv)
        if g in sampled:
            sampled[g] = (kk, vv)

    def to_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)

    cache = M.Cache(1, wl.hkv, wl.d, wl.cap)
    bm = dev_f32(b)
    ocs = {g: orc.Cache(1, 1, wl.d, wl.cap) for g in sampled}
    keep = orc.keep_count(wl.d, sparsity)
    q = W.queries(wl)
    if shared:   # one kept set per KV head, checked, then laid out per head for the oracle
        qp, idx = M.select_channels_shared(dev_input(q, wl.dtype), dev_f32(a), wl.hkv, keep)
        _, idxo_all = orc.queries_shared(q, a, wl.hkv, keep)
        assert np.array_equal(idx.cpu().numpy(), idxo_all)
        idx_np = orc.per_head(idxo_all, wl.group)
    else:
        qp, idx = gpu_queries(wl, q, a, keep)
        idx_np = idx.cpu().numpy()
    decode = M.decode_attention_shared if shared else M.decode_attention
    pos = 0
    for extra in extras:
        n = ctx + extra - pos
        say(f"  append {n} tokens (length {ctx + extra})")
        M.transform_quantize_append(cache, to_dev(kb[:, :, pos:pos + n]), to_dev(vb[:, :, pos:pos + n]),
                                    bm, dev_i32(np.array([n], dtype=np.int32)))
        for g, (kk, vv) in sampled.items():
            ocs[g].append(kk[None, None, pos:pos + n], vv[None, None, pos:pos + n], b[g:g + 1], [n])
        pos += n
        out = decode(cache, qp, idx, sm).cpu().numpy()
        for g in sampled:
            hs = slice(4 * g, 4 * g + 4)
            qpo, idxo = orc.queries(q[:, hs], a[g:g + 1], 1, keep)
            if shared:
                idxo = idx_np[:, hs]
            assert np.array_equal(idx_np[:, hs], idxo), g
            err = rel_err(out[:, hs], ocs[g].decode(qpo, idxo, sm))
            say(f"  length {ctx + extra}, s {sparsity}%, KV head {g}: max rel err {err:.3e}")
            assert err <= REL_TOL, (extra, g, err)


def test_decode_gqa8k_full_sampled(orc):
    """The GQA 32/8 workload at full size (batch 4, head_dim 128, 8192 tokens,
    40% sparsity, bf16) in its launch configuration (the default split): the
    whole cache is built from the workload's own keys and values, and three
    (row, KV head) units are checked against the oracle, which decodes each from
    a one-KV-head cache of that unit (the units are independent)."""
    wl = W.workload("gqa8k")
    sm = W.default_sm_scale(wl.d)
    g, a, b, k, v = build_gpu(wl)
    keep = orc.keep_count(wl.d, 40)
    q = W.queries(wl)
    qp, idx = gpu_queries(wl, q, a, keep)
    idx_np = idx.cpu().numpy()
    out = M.decode_attention(g, qp, idx, sm).cpu().numpy()
    for bb, gg in ((0, 0), (3, 7), (2, 4)):
        say(f"gqa8k full: oracle for row {bb}, KV head {gg}")
        oc = orc.Cache(1, 1, wl.d, wl.cap)
        n = int(wl.ctx[bb])
        oc.append(k[bb:bb + 1, gg:gg + 1, :n], v[bb:bb + 1, gg:gg + 1, :n], b[gg:gg + 1], [n])
        hs = slice(wl.group * gg, wl.group * (gg + 1))
        qpo, idxo = orc.queries(q[bb:bb + 1, hs], a[gg:gg + 1], 1, keep)
        assert np.array_equal(idx_np[bb:bb + 1, hs], idxo)
        err = rel_err(out[bb:bb + 1, hs], oc.decode(qpo, idxo, sm))
        say(f"  max rel err {err:.3e}")
        assert err <= REL_TOL, (bb, gg, err)


def test_append32k_fused_steps_sampled(orc):
    """The 32K append loop at full size (batch 8, 32/8 heads, head_dim 128, 32768
    prefilled tokens, then 64 steps of the fused append-one-token + select launch
    followed by the decode, 40% sparsity) as the benchmark runs it.  Two (row, KV
    head) units hold the workload's own keys and values, prefill and appended
    tokens; the others hold draws of the same channel scales.  After steps 0, 31
    (the step that closes a 32-token key group) and 63 the sampled units' outputs
    and kept sets are checked against the oracle, which replays the same appends
    on a one-KV-head cache per unit, and their cache planes must be byte-equal."""
    wl = W.workload("append32k")
    ctx, sm = int(wl.ctx[0]), W.default_sm_scale(wl.d)
    a, b = W.transforms(wl)
    kscale = W.key_scales(wl)
    units = [(0, 0), (5, 3)]
    say("append32k: drawing the sampled units' tokens")
    kv = {u: W.unit_kv(wl, u[0], u[1], 0, ctx + wl.steps, kscale) for u in units}
    cache = M.Cache(wl.batch, wl.hkv, wl.d, wl.cap)
    bm, ks_d = dev_f32(b), dev_f32(kscale)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(13)
    chunk = 8192
    for pos in range(0, ctx, chunk):
        k = torch.randn((wl.batch, wl.hkv, chunk, wl.d), generator=gen, device="cuda")
        k = (k * ks_d[None, :, None, :]).to(torch.bfloat16)
        v = torch.randn((wl.batch, wl.hkv, chunk, wl.d), generator=gen, device="cuda").to(torch.bfloat16)
        for (bb, gg), (kk, vv) in kv.items():
            k[bb, gg] = torch.from_numpy(kk[pos:pos + chunk]).cuda().to(torch.bfloat16)
            v[bb, gg] = torch.from_numpy(vv[pos:pos + chunk]).cuda().to(torch.bfloat16)
        M.transform_quantize_append(cache, k, v, bm, dev_i32(np.full(wl.batch, chunk)))
    ocs = {}
    for (bb, gg), (kk, vv) in kv.items():
        say(f"  oracle prefill: row {bb}, KV head {gg}")
        oc = orc.Cache(1, 1, wl.d, wl.cap)
        oc.append(kk[None, None, :ctx], vv[None, None, :ctx], b[gg:gg + 1], [ctx])
        ocs[(bb, gg)] = oc
    keep = orc.keep_count(wl.d, 40)
    a_d = dev_f32(a)
    ones = dev_i32(np.ones(wl.batch))
    qp = torch.empty((wl.batch, wl.hq, wl.d), dtype=torch.float32, device="cuda")
    idx = torch.empty((wl.batch, wl.hq, keep), dtype=torch.int32, device="cuda")
    out = torch.empty((wl.batch, wl.hq, wl.d), dtype=torch.float32, device="cuda")
    ws = torch.empty(M.decode_workspace_bytes(cache, wl.hq), dtype=torch.uint8, device="cuda")
    for step in range(wl.steps):
        x = torch.randn((2, wl.batch, wl.hkv, 1, wl.d), generator=gen, device="cuda")
        x[0] *= ks_d[None, :, None, :]
        for (bb, gg), (kk, vv) in kv.items():
            x[0, bb, gg, 0] = torch.from_numpy(kk[ctx + step]).cuda()
            x[1, bb, gg, 0] = torch.from_numpy(vv[ctx + step]).cuda()
        x = x.to(torch.bfloat16)
        q = W.queries(wl, step)
        M.append_select(cache, x[0].contiguous(), x[1].contiguous(), bm, ones,
                        dev_input(q, wl.dtype), a_d, keep, qp, idx)
        M.decode_attention(cache, qp, idx, sm, 0, out, ws)
        for (bb, gg), (kk, vv) in kv.items():
            ocs[(bb, gg)].append(kk[None, None, ctx + step:ctx + step + 1],
                                 vv[None, None, ctx + step:ctx + step + 1], b[gg:gg + 1], [1])
        if step not in (0, 31, 63):
            continue
        o = out.cpu().numpy()
        idx_np = idx.cpu().numpy()
        planes = planes_np(cache)
        for (bb, gg), oc in ocs.items():
            assert int(planes["lengths"][bb]) == ctx + step + 1
            assert_same_cache(planes, oc, unit_map=[((bb, gg), (0, 0))])
            hs = slice(wl.group * gg, wl.group * (gg + 1))
            qpo, idxo = orc.queries(q[bb:bb + 1, hs], a[gg:gg + 1], 1, keep)
            assert np.array_equal(idx_np[bb:bb + 1, hs], idxo), (step, bb, gg)
            err = rel_err(o[bb:bb + 1, hs], oc.decode(qpo, idxo, sm))
            say(f"  step {step}, row {bb}, KV head {gg}: max rel err {err:.3e}")
            assert err <= REL_TOL, (step, bb, gg, err)


def test_decode_ragged64k_sampled(orc):
    """The ragged group-of-eight workload at full size (batch 16, 64/8 heads,
    head_dim 128, rows of 20K..62K tokens in a 64K capacity, 40% sparsity,
    Student-t queries) in its launch configuration: the default split, here
    whole-block splits of 31 blocks of 128 tokens (chunks of 10, 10 and 10 + 1)
    with one eight-head workgroup per split (and other whole-block and
    equal-share splits for comparison).  Three (row, KV head) units are checked
    against the oracle: the longest row, the shortest and a middle one.  They hold
    the workload's own keys and values; the other units hold normal draws of the
    same channel scales (the units are independent)."""
    wl = W.workload("ragged64k")
    lens = np.array(wl.ctx)
    sm = W.default_sm_scale(wl.d)
    a, b = W.transforms(wl)
    kscale = W.key_scales(wl)
    order = np.argsort(lens, kind="stable")
    units = [(int(order[-1]), 0), (int(order[0]), 7), (int(order[len(order) // 2]), 3)]
    say("ragged64k sampled: lengths", int(lens.min()), "..", int(lens.max()), "units", units)
    kv = {u: W.unit_kv(wl, u[0], u[1], 0, int(lens[u[0]]), kscale) for u in units}
    cache = M.Cache(wl.batch, wl.hkv, wl.d, wl.cap)
    bm, ks_d = dev_f32(b), dev_f32(kscale)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(11)
    chunk = 8192
    for pos in range(0, int(lens.max()), chunk):
        nn = np.clip(lens - pos, 0, chunk).astype(np.int32)
        k = torch.randn((wl.batch, wl.hkv, chunk, wl.d), generator=gen, device="cuda")
        k = (k * ks_d[None, :, None, :]).to(torch.bfloat16)
        v = torch.randn((wl.batch, wl.hkv, chunk, wl.d), generator=gen, device="cuda").to(torch.bfloat16)
        for (bb, g), (kk, vv) in kv.items():
            m = int(nn[bb])
            if m > 0:   # exact bf16 values: the conversion is exact
                k[bb, g, :m] = torch.from_numpy(kk[pos:pos + m]).cuda().to(torch.bfloat16)
                v[bb, g, :m] = torch.from_numpy(vv[pos:pos + m]).cuda().to(torch.bfloat16)
        M.transform_quantize_append(cache, k, v, bm, dev_i32(nn))
    keep = orc.keep_count(wl.d, 40)
    q = W.queries(wl)
    qp, idx = gpu_queries(wl, q, a, keep)
    idx_np = idx.cpu().numpy()
    refs = {}
    for (bb, g), (kk, vv) in kv.items():
        say(f"  oracle: row {bb} ({int(lens[bb])} tokens), KV head {g}")
        oc = orc.Cache(1, 1, wl.d, wl.cap)
        oc.append(kk[None, None], vv[None, None], b[g:g + 1], [int(lens[bb])])
        hs = slice(8 * g, 8 * g + 8)
        qpo, idxo = orc.queries(q[bb:bb + 1, hs], a[g:g + 1], 1, keep)
        assert np.array_equal(idx_np[bb:bb + 1, hs], idxo), (bb, g)
        refs[(bb, g)] = oc.decode(qpo, idxo, sm)
    outs = {}
    for sp in (0, 3968, 5376, 4096, 8224):
        outs[sp] = out = M.decode_attention(cache, qp, idx, sm, split_tokens=sp).cpu().numpy()
        for (bb, g), ref in refs.items():
            err = rel_err(out[bb:bb + 1, 8 * g:8 * g + 8], ref)
            say(f"  split {sp}, row {bb}, KV head {g}: max rel err {err:.3e}")
            assert err <= REL_TOL, (sp, bb, g, err)
    # the default is whole-block splits of 3968 tokens here (31 blocks of 128 for
    # the eight-head decode): the same launch
    assert np.array_equal(outs[0].view(np.uint32), outs[3968].view(np.uint32))


def test_step_graph_replay_matches_eager(orc):
    """The decode step (append one token, select, decode) captured as a HIP graph:
    three replays, each followed by the same step run eagerly on a twin cache, with
    synchronisations between; every replay's cache planes, q', indices and output
    are bitwise those of the eager step.  No launch on the path records a memset."""
    wl = W.workload("gqa8k", batch=2, ctx=2600)
    ga, a, b, k, v = build_gpu(wl)
    gb, _, _, _, _ = build_gpu(wl, kv=(k, v))
    a_d, b_d = dev_f32(a), dev_f32(b)
    keep = orc.keep_count(wl.d, 40)
    sm = W.default_sm_scale(wl.d)
    rng = np.random.default_rng(5)
    kx = torch.from_numpy(rng.standard_normal((wl.batch, wl.hkv, 1, wl.d)).astype(np.float32)).to(
        torch.bfloat16).cuda()
    q = dev_input(W.queries(wl, 1), wl.dtype)
    ones = torch.ones((wl.batch,), dtype=torch.int32, device="cuda")
    qp = torch.empty((wl.batch, wl.hq, wl.d), dtype=torch.float32, device="cuda")
    idx = torch.empty((wl.batch, wl.hq, keep), dtype=torch.int32, device="cuda")
    out = torch.empty((wl.batch, wl.hq, wl.d), dtype=torch.float32, device="cuda")
    ws = torch.empty(M.decode_workspace_bytes(ga, wl.hq, 0), dtype=torch.uint8, device="cuda")

    def step(c, qp_, idx_, out_, ws_):
        M.transform_quantize_append(c, kx, kx, b_d, ones)
        M.select_channels(q, a_d, wl.hkv, keep, qp_, idx_)
        M.decode_attention(c, qp_, idx_, sm, 0, out_, ws_)

    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        step(ga, qp, idx, out, ws)
    torch.cuda.synchronize()
    for r in range(3):
        say("graph replay", r)
        graph.replay()
        torch.cuda.synchronize()
        qp_e, idx_e = torch.empty_like(qp), torch.empty_like(idx)
        out_e, ws_e = torch.empty_like(out), torch.empty_like(ws)
        step(gb, qp_e, idx_e, out_e, ws_e)
        torch.cuda.synchronize()
        pa, pb = planes_np(ga), planes_np(gb)
        for name in pa:
            assert np.array_equal(pa[name], pb[name]), (r, name)
        assert np.array_equal(qp.cpu().numpy().view(np.uint32), qp_e.cpu().numpy().view(np.uint32))
        assert np.array_equal(idx.cpu().numpy(), idx_e.cpu().numpy())
        assert np.array_equal(out.cpu().numpy().view(np.uint32), out_e.cpu().numpy().view(np.uint32)), r


@pytest.mark.parametrize("hq,cap", [(32, 1504), (32, 1536), (64, 1536)])
def test_decode_poisoned_dropped_channels(orc, hq, cap):
    """Codes and scales of channels no head of the group keeps are overwritten
    with 0xFF / fp16 NaN: the output is bitwise unchanged, so their contents are
    never used (the general kernel, capacity 1504, does not read them; the
    matrix-core kernel, capacity 1536, groups of 4 and 8, reads them only in a
    workgroup's first block and gives them zero weight)."""
    wl = W.custom(f"poison{hq}-{cap}", 2, 2, hq, 8, 128, [1500, 1500], cap, "bf16",
                  log_uniform_key_scales=True)
    g, a, b, k, v = build_gpu(wl)
    keep = orc.keep_count(wl.d, 60)
    qp, idx = gpu_queries(wl, W.queries(wl), a, keep)
    sm = W.default_sm_scale(wl.d) * 0.02
    base = M.decode_attention(g, qp, idx, sm).cpu().numpy()
    idx_np = idx.cpu().numpy()
    poisoned = 0
    for bb in range(wl.batch):
        for gg in range(wl.hkv):
            kept = set(idx_np[bb, gg * wl.group:(gg + 1) * wl.group].ravel().tolist())
            drop = [c for c in range(1, wl.d) if c not in kept]
            poisoned += len(drop)
            if drop:
                g.k_codes[bb, gg, drop] = 0xFF
                g.k_scales[bb, gg, drop] = 0x7E00     # fp16 NaN bits
    assert poisoned > 0
    again = M.decode_attention(g, qp, idx, sm).cpu().numpy()
    assert np.array_equal(base.view(np.uint32), again.view(np.uint32))


def test_decode_deterministic(orc):
    wl = W.workload("gqa8k", batch=1, ctx=3000)
    g, a, b, k, v = build_gpu(wl)
    qp, idx = gpu_queries(wl, W.queries(wl), a, 77)
    o1 = M.decode_attention(g, qp, idx, 0.01).cpu().numpy()
    o2 = M.decode_attention(g, qp, idx, 0.01).cpu().numpy()
    assert np.array_equal(o1.view(np.uint32), o2.view(np.uint32))


# ----------------------------------------------------------------------------- bf16 comparator


@pytest.mark.parametrize("nbytes", [0, 16, 4096 + 48, (64 << 20) + 16 * 777])
def test_stream_read_folds_every_word(nbytes):
    """The read probe reads each 16-byte element exactly once: the XOR of its
    sink equals the XOR of the buffer's 32-bit words (sizes below one load per
    thread, two iterations of the unrolled loop and a ragged tail, and empty)."""
    rng = np.random.default_rng(nbytes)
    words = rng.integers(0, 1 << 32, size=nbytes // 4, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(words.view(np.int32)).cuda() if nbytes else torch.empty(0, dtype=torch.int32, device="cuda")
    sink = torch.full((M.STREAM_READ_SINK_WORDS,), -1, dtype=torch.int32, device="cuda")
    M.stream_read(buf, sink)
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    want = np.bitwise_xor.reduce(words) if nbytes else np.uint32(0)
    assert got == want, (nbytes, hex(int(got)), hex(int(want)))


@pytest.mark.parametrize("wg,lif", [(1, 1), (256, 16), (1000, 8), (2048, 2)])
def test_stream_read_config_folds_every_word(wg, lif):
    """The probe with a given launch shape reads each 16-byte element once: the
    XOR of the sink words it writes equals the XOR of the buffer's words."""
    nbytes = (8 << 20) + 16 * 333
    words = np.random.default_rng(wg + lif).integers(0, 1 << 32, size=nbytes // 4,
                                                     dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(words.view(np.int32)).cuda()
    sink = torch.zeros((M.STREAM_READ_SINK_WORDS,), dtype=torch.int32, device="cuda")
    M.stream_read_config(buf, wg, lif, sink)
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32)[:4 * wg])
    assert got == np.bitwise_xor.reduce(words), (wg, lif)


@pytest.mark.parametrize("lens,sm_mult", [([4096], 1.0), ([4096], 0.02), ([1000, 1, 0, 2049], 0.05)])
def test_bf16_decode_matches_plain_attention(orc, lens, sm_mult):
    wl = W.custom("bf16cmp", 26, len(lens), 32, 8, 128, lens, 4096 + 64, "bf16",
                  log_uniform_key_scales=True)
    say("bf16 decode", lens)
    k, v = W.prefill_kv(wl)
    q = W.queries(wl)
    sm = W.default_sm_scale(wl.d) * sm_mult
    ref = orc.plain_attention(q, k, v, list(wl.ctx), sm)
    for sp in (0, 64, 2048):
        out = M.bf16_decode_attention(dev_input(q, "bf16"), dev_input(k, "bf16"),
                                      dev_input(v, "bf16"), dev_i32(wl.ctx), sm,
                                      split_tokens=sp).cpu().numpy()
        err = rel_err(out, ref)
        say(f"  split {sp}: {err:.3e}")
        assert err <= REL_TOL


@pytest.mark.parametrize("hq,hkv,d,lens", [(8, 8, 64, [700, 33]), (16, 8, 128, [1500]),
                                          (16, 4, 64, [2000, 1]), (64, 8, 128, [900, 0]),
                                          (32, 4, 64, [1200, 95])])
def test_bf16_decode_group_sizes(orc, hq, hkv, d, lens):
    """The comparator for every group size (1, 2, 4, 8) and head dimension, with
    ragged, one-token and empty rows and tiles cut by the split end."""
    cap = (max(lens) + 63) // 64 * 64 + 64
    wl = W.custom(f"bf16g{hq}-{hkv}-{d}", 27, len(lens), hq, hkv, d, lens, cap, "bf16",
                  log_uniform_key_scales=True, student_t_queries=(hq == 8 * hkv))
    say("bf16 decode", hq, hkv, d, lens)
    k, v = W.prefill_kv(wl)
    q = W.queries(wl)
    sm = W.default_sm_scale(wl.d) * 0.05
    ref = orc.plain_attention(q, k, v, list(wl.ctx), sm)
    for sp in (0, 32, 96, 1024):
        out = M.bf16_decode_attention(dev_input(q, "bf16"), dev_input(k, "bf16"),
                                      dev_input(v, "bf16"), dev_i32(wl.ctx), sm,
                                      split_tokens=sp).cpu().numpy()
        err = rel_err(out, ref)
        say(f"  split {sp}: {err:.3e}")
        assert err <= REL_TOL
        for bb, n in enumerate(lens):
            if n == 0:
                assert not out[bb].any()


def test_bf16_decode_ctx128k_full(orc):
    """The comparator at the bench's context length (131072 tokens, GQA 8/2 heads, bf16
    inputs with the 128K workload's key scales) against the oracle's plain fp64 attention,
    every output, at the default split and a split that cuts the last tile."""
    wl = W.custom("bf16-128k", 29, 1, 8, 2, 128, [131072], 131072, "bf16",
                  log_uniform_key_scales=True)
    k, v = W.prefill_kv(wl)
    q = W.queries(wl)
    sm = W.default_sm_scale(wl.d)
    ref = orc.plain_attention(q, k, v, list(wl.ctx), sm)
    kd, vd = dev_input(k, "bf16"), dev_input(v, "bf16")
    for sp in (0, 3040):
        out = M.bf16_decode_attention(dev_input(q, "bf16"), kd, vd, dev_i32(wl.ctx), sm,
                                      split_tokens=sp).cpu().numpy()
        err = rel_err(out, ref)
        say(f"bf16 decode 128K split {sp}: max rel err {err:.3e}")
        assert err <= REL_TOL


# ----------------------------------------------------------------------------- group-shared selection

@pytest.mark.parametrize("name", W.WORKLOADS)
def test_select_shared_matches_oracle(orc, name):
    """Group-shared kept sets (one per row and KV head, scored by the fp32 sum of
    |q'| over the group's heads in ascending order) and q' bit for bit."""
    wl = W.workload(name)
    a, _ = W.transforms(wl)
    q = W.queries(wl)
    for keep in sorted({1, 2, orc.keep_count(wl.d, 60), orc.keep_count(wl.d, 40), wl.d - 1, wl.d}):
        qp, idx = M.select_channels_shared(dev_input(q, wl.dtype), dev_f32(a), wl.hkv, keep)
        qpo, idxo = orc.queries_shared(q, a, wl.hkv, keep)
        assert np.array_equal(qp.cpu().numpy().view(np.uint32), qpo.view(np.uint32)), keep
        assert np.array_equal(idx.cpu().numpy(), idxo), keep


@pytest.mark.parametrize("d,hq,hkv,dtype", [(64, 2, 2, "f32"), (64, 8, 2, "bf16"), (64, 16, 2, "f32"),
                                              (128, 4, 2, "bf16"), (128, 16, 2, "f32"),
                                              (128, 8, 8, "bf16")])
def test_select_shared_group_shapes_and_ties(orc, d, hq, hkv, dtype):
    """Every group size at both head dims, and forced ties: duplicated, negated
    and signed-zero query values under an identity transform."""
    wl = W.custom(f"sh_d{d}_g{hq // hkv}", 60 + d + hq, 3, hq, hkv, d, [64, 64, 64], 64, dtype=dtype)
    a, _ = W.transforms(wl)
    q = W.queries(wl)
    for keep in sorted({1, 2, orc.keep_count(d, 40), d - 1, d}):
        qp, idx = M.select_channels_shared(dev_input(q, dtype), dev_f32(a), hkv, keep)
        qpo, idxo = orc.queries_shared(q, a, hkv, keep)
        assert np.array_equal(qp.cpu().numpy().view(np.uint32), qpo.view(np.uint32)), keep
        assert np.array_equal(idx.cpu().numpy(), idxo), keep
    rng = np.random.default_rng(61)
    qt = rng.choice(np.array([0.0, -0.0, 1.0, -1.0, 2.5, -2.5], dtype=np.float32), (3, hq, d))
    eye = np.stack([np.eye(d, dtype=np.float32)] * hkv)
    for keep in (1, 20, d // 2, d):
        qp, idx = M.select_channels_shared(dev_f32(qt), dev_f32(eye), hkv, keep)
        qpo, idxo = orc.queries_shared(qt, eye, hkv, keep)
        assert np.array_equal(idx.cpu().numpy(), idxo), keep
        assert np.array_equal(qp.cpu().numpy().view(np.uint32), qpo.view(np.uint32))


def decode_shared_case(orc, wl, sparsity=40, sm_mult=1.0, splits=(0,)):
    say("decode shared", wl.describe(), "s", sparsity, "splits", splits)
    g, a, b, k, v = build_gpu(wl)
    ref = build_oracle(orc, wl, k, v, b)
    keep = orc.keep_count(wl.d, sparsity)
    q = W.queries(wl)
    qp, idx = M.select_channels_shared(dev_input(q, wl.dtype), dev_f32(a), wl.hkv, keep)
    qpo, idxo = orc.queries_shared(q, a, wl.hkv, keep)
    assert np.array_equal(idx.cpu().numpy(), idxo)
    sm = W.default_sm_scale(wl.d) * sm_mult
    o_ref = ref.decode(qpo, orc.per_head(idxo, wl.group), sm)
    outs = []
    for sp in splits:
        out = M.decode_attention_shared(g, qp, idx, sm, split_tokens=sp).cpu().numpy()
        err = rel_err(out, o_ref)
        say(f"  split {sp}: max rel err {err:.3e}")
        assert err <= REL_TOL, (sp, err)
        outs.append(out)
    # the same sets laid out per head through the per-head decode (channel i + 1
    # in slot i, where the shared decode packs the kept channels into the first
    # slots: the products are summed in another order) agree to the tolerance
    per = torch.from_numpy(orc.per_head(idx.cpu().numpy(), wl.group)).cuda()
    for sp, out in zip(splits, outs):
        again = M.decode_attention(g, qp, per, sm, split_tokens=sp).cpu().numpy()
        assert rel_err(again, out) <= REL_TOL, sp
    return outs


@pytest.mark.parametrize("hq,hkv,d,cap,lens", [(1, 1, 64, 1024, [1000]), (4, 2, 128, 1344, [700, 1333]),
                                                (32, 8, 128, 5056, [5000, 2049, 0]),
                                                (64, 8, 128, 4032, [4000, 31]),
                                                (32, 8, 128, 1376, [1300, 77])])
def test_decode_shared_matches_oracle(orc, hq, hkv, d, cap, lens):
    """Decode with group-shared kept sets on every kernel: groups of one and two
    (general kernel), four and eight (matrix-core kernel, capacity a multiple of
    64) and four with a capacity that is not (general kernel); an empty row."""
    wl = W.custom(f"sh{hq}-{hkv}-{d}", 70 + hq, len(lens), hq, hkv, d, lens, cap, "bf16",
                  log_uniform_key_scales=True, student_t_queries=(hq == 64))
    outs = decode_shared_case(orc, wl, splits=(0, 64, 1024))
    if 0 in lens:
        for out in outs:
            assert not out[lens.index(0)].any()
    decode_shared_case(orc, wl, sparsity=60, sm_mult=0.05)


# ----------------------------------------------------------------------------- growing a cache

@pytest.mark.parametrize("d,cap0,cap1,lens", [(128, 96, 224, [90, 33]), (64, 1024, 1344, [1000, 0, 517]),
                                               (128, 4096, 8192, [4095, 4096])])
def test_cache_grow_matches_oracle(orc, d, cap0, cap1, lens):
    """dqk_cache_grow against the oracle's element-wise copy, byte for byte; then
    appends on the grown cache (closing the unfinished groups and passing the
    old capacity) and a decode, against the oracle doing the same."""
    wl = W.custom(f"grow{d}-{cap0}", 53, len(lens), 4 * (d // 64), d // 64, d, lens, cap0, "bf16",
                  log_uniform_key_scales=True)
    g, a, b, k, v = build_gpu(wl)
    ref = build_oracle(orc, wl, k, v, b)
    big = M.cache_grow(g, cap1)
    ref_big = ref.grow(cap1)
    say("grow", wl.describe(), "->", cap1)
    assert_same_cache(planes_np(big), ref_big)
    n = cap1 - cap0 - 40
    more = W.round_bf16(np.random.default_rng(54).standard_normal((wl.batch, wl.hkv, n, d)).astype(np.float32))[0]
    counts = np.array([n, 37, 1][:wl.batch], dtype=np.int32)
    M.transform_quantize_append(big, dev_input(more, "bf16"), dev_input(more, "bf16"), dev_f32(b), dev_i32(counts))
    ref_big.append(more, more, b, list(counts))
    assert_same_cache(planes_np(big), ref_big)
    keep = orc.keep_count(d, 40)
    q = W.queries(wl)
    qp, idx = gpu_queries(wl, q, a, keep)
    qpo, idxo = orc.queries(q, a, wl.hkv, keep)
    sm = W.default_sm_scale(d)
    err = rel_err(M.decode_attention(big, qp, idx, sm).cpu().numpy(), ref_big.decode(qpo, idxo, sm))
    say(f"  decode after grow and append: max rel err {err:.3e}")
    assert err <= REL_TOL
