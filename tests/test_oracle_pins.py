"""Pins for the CPU oracle against what the mathematics and library routines fix.

Every test here runs on the CPU.  None of them compares the oracle with itself:
each uses a closed form, a special case that reduces to a library routine
(numpy float16, numpy fp64 matmul, numpy lexsort, torch fp64 attention), brute
force on tiny inputs, or an invariance the definition implies.
"""
import itertools
import os

import numpy as np
import pytest

import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------- fp16

def _f16_reference(x):
    """numpy float16 (round to nearest even, subnormals kept) with every result
    that rounds to infinity, infinite inputs included, replaced by +-65504."""
    with np.errstate(over="ignore", invalid="ignore"):
        ref = x.astype(np.float16).view(np.uint16).copy()
    sat = ((ref & 0x7FFF) == 0x7C00) & ~np.isnan(x)
    ref[sat] = (ref[sat] & 0x8000) | 0x7BFF
    return ref


def _check_f16(orc, bits):
    x = bits.view(np.float32)
    got = orc.f16_from_f32(x)
    ref = _f16_reference(x)
    nan = np.isnan(x)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.all((got[nan] & 0x7C00) == 0x7C00) and np.all((got[nan] & 0x3FF) != 0)


@pytest.mark.slow
def test_f16_from_f32_exhaustive(orc):
    """Every positive fp32 pattern with a biased exponent in [100, 143] (from below
    half the smallest fp16 subnormal to past the overflow threshold), checked
    against numpy's float16; plus 2^24 random patterns over all 2^32 (both signs,
    zeros, infinities, NaN) and the sign symmetry of the whole range."""
    lo, hi = 100 << 23, 144 << 23
    step = 1 << 24
    for start in range(lo, hi, step):
        _check_f16(orc, np.arange(start, min(start + step, hi), dtype=np.uint32))
    rnd = np.random.default_rng(10).integers(0, 1 << 32, size=1 << 24, dtype=np.uint64)
    _check_f16(orc, rnd.astype(np.uint32))
    pos = np.arange(lo, hi, 4099, dtype=np.uint32)
    assert np.array_equal(orc.f16_from_f32((pos | 0x80000000).view(np.float32)),
                          orc.f16_from_f32(pos.view(np.float32)) | 0x8000)
    edge = np.array([0, 1, 0x7F800000, 0xFF800000, 0x477FF000, 0x477FEFFF, 0x33000000,
                     0x33000001, 0x387FC000, 0x387FE000], dtype=np.uint32)
    _check_f16(orc, edge)


def test_f32_from_f16_exhaustive(orc):
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = orc.f32_from_f16(h)
    ref = h.view(np.float16).astype(np.float32)
    both_nan = np.isnan(got) & np.isnan(ref)
    assert np.array_equal(got[~both_nan], ref[~both_nan])
    assert np.array_equal(np.isnan(got), np.isnan(ref))


# ----------------------------------------------------------------------------- quantizer

def _golden(name):
    out = {}
    for line in open(os.path.join(GOLDEN, name)):
        if line.startswith("#") or ":" not in line:
            continue
        k, v = line.split(":", 1)
        out[k.strip()] = v.split()
    return out


def test_quantizer_worked_example(orc):
    g = _golden("quantizer_worked_example.txt")
    x = np.array([float(t) for t in g["input"]], dtype=np.float32)
    s, u = orc.quantize32(x)
    assert s == int(g["sigma_bits"][0], 16)
    assert list(u) == [int(t) for t in g["codes"]]
    # packing through the cache: append the group as channel 1 of 32 tokens
    # with B = I, so k' = k exactly
    c = orc.Cache(1, 1, 32, 32)
    k = np.zeros((1, 1, 32, 32), dtype=np.float32)
    k[0, 0, :, 1] = x
    c.append(k, np.zeros_like(k), np.eye(32, dtype=np.float32)[None], [32])
    assert list(c.k_codes[0, 0, 1, :8]) == [int(t, 16) for t in g["key_bytes"]]
    kd, _ = c.dequant()
    assert list(kd[0, 0, :8, 1]) == [float(t) for t in g["decoded_first8"]]


def test_quantizer_grid_round_trip(orc):
    """x = s*(2u-3) with s an fp16 number and a level of magnitude 3 present
    re-encodes to the same (s, u) and decodes to x exactly."""
    rng = np.random.default_rng(11)
    for _ in range(400):
        e = rng.integers(-14, 15)
        s16 = np.float16(np.ldexp(1.0 + rng.integers(0, 1024) / 1024.0, e))
        s = np.float32(s16)
        u = rng.integers(0, 4, size=32)
        u[rng.integers(0, 32)] = rng.choice([0, 3])
        x = (s * (2 * u - 3)).astype(np.float32)
        sig, got = orc.quantize32(x)
        assert sig == int(np.array(s16).view(np.uint16))
        assert np.array_equal(got, u)
        assert np.array_equal(orc.f32_from_f16(np.array([sig], np.uint16))[0] * (2 * got.astype(np.float32) - 3), x)


def test_quantizer_error_bound_and_monotone(orc):
    """|x - x_hat| <= s + max(0, m - 3s) (levels +-s, +-3s with midpoint
    thresholds), and codes never decrease as x increases."""
    rng = np.random.default_rng(12)
    for trial in range(300):
        scale = 10.0 ** rng.uniform(-6, 5)
        x = (rng.standard_normal(32) * scale).astype(np.float32)
        if trial % 7 == 0:
            x = np.sort(x)
        sig, u = orc.quantize32(x)
        s = float(orc.f32_from_f16(np.array([sig], np.uint16))[0])
        xh = s * (2 * u.astype(np.float64) - 3)
        m = float(np.max(np.abs(x)))
        assert np.all(np.abs(x - xh) <= s + max(0.0, m - 3 * s) + 1e-12 * m)
        order = np.argsort(x, kind="stable")
        assert np.all(np.diff(u[order].astype(int)) >= 0)


def test_quantizer_special_groups(orc):
    sig, u = orc.quantize32(np.zeros(32, dtype=np.float32))
    assert sig == 0 and np.all(orc.f32_from_f16(np.array([sig], np.uint16))[0] * (2 * u.astype(np.float32) - 3) == 0)
    big = np.full(32, 1e6, dtype=np.float32)
    sig, u = orc.quantize32(big)
    assert sig == 0x7BFF and np.all(u == 3)           # saturated scale
    x = np.zeros(32, dtype=np.float32)
    x[5] = -7.5
    sig, u = orc.quantize32(x)
    assert orc.f32_from_f16(np.array([sig], np.uint16))[0] == np.float32(2.5) and u[5] == 0


# ----------------------------------------------------------------------------- transform

def test_transform_exact_special_matrices(orc):
    rng = np.random.default_rng(13)
    d = 64
    x = rng.standard_normal(d).astype(np.float32)
    assert np.array_equal(orc.transform(x, np.eye(d, dtype=np.float32)), x)
    perm = rng.permutation(d)
    pm = np.zeros((d, d), dtype=np.float32)
    pm[np.arange(d), perm] = 1.0                      # y[perm[i]] = x[i]
    y = orc.transform(x, pm)
    ref = np.empty_like(x)
    ref[perm] = x
    assert np.array_equal(y, ref)
    diag = (rng.choice([-1, 1], d) * np.ldexp(1.0, rng.integers(-5, 6, d))).astype(np.float32)
    assert np.array_equal(orc.transform(x, np.diag(diag)), x * diag)


def test_transform_higham_bound(orc):
    """Recursive summation of d products: |y - y_exact| <= gamma_d * sum_i |x_i m_ij|,
    gamma_d = d u / (1 - d u), u = 2^-24 (fp32, fused multiply-add)."""
    rng = np.random.default_rng(14)
    for d in (64, 128):
        u = 2.0 ** -24
        gam = d * u / (1 - d * u)
        for _ in range(20):
            x = (rng.standard_normal(d) * 10 ** rng.uniform(-3, 3)).astype(np.float32)
            m = (rng.standard_normal((d, d)) * 10 ** rng.uniform(-3, 3)).astype(np.float32)
            y = orc.transform(x, m).astype(np.float64)
            ex = x.astype(np.float64) @ m.astype(np.float64)
            bound = gam * (np.abs(x.astype(np.float64)) @ np.abs(m.astype(np.float64)))
            assert np.all(np.abs(y - ex) <= bound)


def test_transform_pair_keeps_dot_products(orc):
    """q'.k' = q.k up to fp32 rounding amplified by cond(A) (paired transforms
    with A B^T = I); the orthogonal special case A = B = R is the rotation."""
    for name in ("tiny", "gqa8k"):
        wl = W.workload(name)
        a, b = W.transforms(wl)
        rng = np.random.default_rng(15)
        for g in range(min(wl.hkv, 2)):
            cond = np.linalg.cond(a[g].astype(np.float64))
            for _ in range(10):
                q = rng.standard_normal(wl.d).astype(np.float32)
                k = rng.standard_normal(wl.d).astype(np.float32)
                qp = orc.transform(q, a[g]).astype(np.float64)
                kp = orc.transform(k, b[g]).astype(np.float64)
                exact = q.astype(np.float64) @ k.astype(np.float64)
                err = abs(qp @ kp - exact)
                assert err <= 4 * wl.d * cond * 2.0 ** -24 * np.linalg.norm(q) * np.linalg.norm(k)
    d = 64
    r, _ = np.linalg.qr(np.random.default_rng(16).standard_normal((d, d)))
    r = r.astype(np.float32)
    q = np.random.default_rng(17).standard_normal(d).astype(np.float32)
    k = np.random.default_rng(18).standard_normal(d).astype(np.float32)
    err = abs(orc.transform(q, r).astype(np.float64) @ orc.transform(k, r).astype(np.float64)
              - q.astype(np.float64) @ k.astype(np.float64))
    assert err < 1e-4


def _round_f32(x):
    """Round an exact rational to the nearest fp32 number, ties to even (IEEE
    binary32: 24-bit significand, exponent >= -126, subnormal quantum 2^-149)."""
    from fractions import Fraction
    if x == 0:
        return np.float32(0.0)
    sign = -1 if x < 0 else 1
    a = abs(Fraction(x))
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    quantum = Fraction(2) ** (max(e, -126) - 23)
    m = a / quantum
    fl = m.numerator // m.denominator
    rem = m - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return np.float32(sign * float(fl * quantum))


def _fma_chain_exact(x, col, order):
    """acc = +0; acc = fp32(x_i * m_i + acc) for i in `order`: each fused
    multiply-add evaluated exactly in rationals and rounded once to fp32."""
    from fractions import Fraction
    acc = np.float32(0.0)
    for i in order:
        acc = _round_f32(Fraction(float(x[i])) * Fraction(float(col[i])) + Fraction(float(acc)))
    return acc


def test_transform_ascending_fma_chain_order(orc):
    """The transform's reading fixes the order of the chain: ascending input
    index, one rounding per fused multiply-add.  A crafted column where the two
    orders round differently, then random columns of wide dynamic range, against
    an exact-rational evaluation of each fused multiply-add; the descending
    chain must differ somewhere, so the pin separates the two orders."""
    # 1 + 2^-24 + 2^-24: ascending rounds each addition back to 1 (tie to even);
    # descending sums the two small terms first, then 1 + 2^-23 is exact
    d = 64
    x = np.zeros(d, dtype=np.float32)
    x[:3] = [1.0, 2.0 ** -24, 2.0 ** -24]
    m = np.zeros((d, d), dtype=np.float32)
    m[:3, 0] = 1.0
    y = orc.transform(x, m)
    assert y[0] == np.float32(1.0)
    assert _fma_chain_exact(x, m[:, 0], range(d - 1, -1, -1)) == np.float32(1.0 + 2.0 ** -23)
    rng = np.random.default_rng(31)
    differs = 0
    for d in (64, 128):
        x = (rng.standard_normal(d) * 2.0 ** rng.integers(-12, 13, d)).astype(np.float32)
        m = (rng.standard_normal((d, d)) * 2.0 ** rng.integers(-12, 13, (d, d))).astype(np.float32)
        y = orc.transform(x, m)
        for j in range(0, d, 3):
            asc = _fma_chain_exact(x, m[:, j], range(d))
            assert y[j].view(np.uint32) == asc.view(np.uint32), (d, j)
            differs += asc != _fma_chain_exact(x, m[:, j], range(d - 1, -1, -1))
    assert differs > 0


def test_queries_use_the_kv_head_of_each_group(orc):
    """Query head h uses A of KV head h div G.  Each KV head gets its own signed
    power-of-two permutation matrix, so q' = q A_g is exact in fp32 and equals
    numpy's fp64 product bit for bit; any other head-to-transform mapping
    (h mod hkv, say) picks another permutation and fails.  The kept sets follow
    from the exact q' by lexsort."""
    rng = np.random.default_rng(32)
    d, hkv, batch, keep = 64, 3, 2, 38
    mats = []
    for g in range(hkv):
        m = np.zeros((d, d), dtype=np.float32)
        m[np.arange(d), rng.permutation(d)] = rng.choice([-1.0, 1.0], d) * 2.0 ** rng.integers(-4, 5, d)
        mats.append(m)
    a = np.stack(mats)
    for grp in (1, 2, 4, 8):
        hq = hkv * grp
        q = rng.standard_normal((batch, hq, d)).astype(np.float32)
        qp, idx = orc.queries(q, a, hkv, keep)
        for bb in range(batch):
            for h in range(hq):
                want = (q[bb, h].astype(np.float64) @ a[h // grp].astype(np.float64)).astype(np.float32)
                assert np.array_equal(qp[bb, h].view(np.uint32), want.view(np.uint32)), (grp, bb, h)
                c = np.arange(1, d)
                order = np.lexsort((c, -np.abs(want[1:])))
                assert np.array_equal(idx[bb, h], np.sort(np.concatenate([[0], c[order][:keep - 1]])))


# ----------------------------------------------------------------------------- selection

def test_keep_count_values(orc):
    assert [orc.keep_count(128, s) for s in (0, 40, 60)] == [128, 77, 51]
    assert orc.keep_count(64, 40) == 38
    assert orc.keep_count(128, 100) == 0 and orc.keep_count(1, 50) == 1


def _beats(qp, a, b):
    return abs(qp[a]) > abs(qp[b]) or (abs(qp[a]) == abs(qp[b]) and a < b)


def test_select_brute_force_tiny(orc):
    """Enumerate every kept set that contains channel 0: exactly one has every kept
    channel c >= 1 beating every dropped one on (|q'| desc, index asc)."""
    rng = np.random.default_rng(19)
    for trial in range(300):
        d = int(rng.integers(2, 11))
        keep = int(rng.integers(1, d + 1))
        qp = rng.standard_normal(d).astype(np.float32)
        if trial % 3 == 0:   # forced ties: duplicates, negations, signed zeros
            qp = rng.choice(np.array([0.0, -0.0, 1.5, -1.5, 2.0], dtype=np.float32), d)
        valid = []
        for rest in itertools.combinations(range(1, d), keep - 1):
            kept = set(rest)
            dropped = [c for c in range(1, d) if c not in kept]
            if all(_beats(qp, a, b) for a in kept for b in dropped):
                valid.append(sorted((0,) + rest))
        assert len(valid) == 1
        assert list(orc.select(qp, keep)) == valid[0]


def test_select_large_against_lexsort(orc):
    rng = np.random.default_rng(20)
    for d in (64, 128):
        for keep in sorted({k for k in (1, 2, 38, 51, 77, d - 1, d) if k <= d}):
            for trial in range(5):
                qp = rng.standard_normal(d).astype(np.float32)
                if trial == 1:
                    qp = np.round(qp * 2).astype(np.float32) / 2     # many ties
                if trial == 2:
                    qp[1::2] = -qp[0::2][: len(qp[1::2])]            # +-pairs tie
                c = np.arange(1, d)
                order = np.lexsort((c, -np.abs(qp[1:])))             # |q'| desc, index asc
                ref = np.sort(np.concatenate([[0], c[order][: keep - 1]]))
                assert np.array_equal(orc.select(qp, keep), ref)


def test_select_edge_counts(orc):
    qp = np.random.default_rng(21).standard_normal(128).astype(np.float32)
    assert list(orc.select(qp, 1)) == [0]
    assert list(orc.select(qp, 128)) == list(range(128))
    z = np.zeros(16, dtype=np.float32)
    z[3] = -0.0
    assert list(orc.select(z, 5)) == [0, 1, 2, 3, 4]       # all ties -> lowest indices


# ----------------------------------------------------------------------------- append

def _append_all(orc, wl, chunks):
    """Append the prefill of every unit in the given chunk sizes."""
    a, b = W.transforms(wl)
    c = orc.Cache(wl.batch, wl.hkv, wl.d, wl.cap)
    k, v = W.prefill_kv(wl)
    pos = 0
    for n in chunks:
        c.append(k[:, :, pos:pos + n], v[:, :, pos:pos + n], b, [n] * wl.batch)
        pos += n
    return c, k, v, a, b


def _same_cache(c1, c2):
    p1, p2 = c1.planes(), c2.planes()
    for name in p1:
        if name == "k_tail":
            continue
        assert np.array_equal(p1[name], p2[name]), name
    for bb in range(c1.batch):
        r = int(c1.lengths[bb]) % 32
        assert np.array_equal(c1.k_tail[bb, :, :r], c2.k_tail[bb, :, :r])


def test_append_chunking_invariance(orc):
    wl = W.workload("tiny", ctx=100)
    c_bulk, *_ = _append_all(orc, wl, [100])
    c_one, *_ = _append_all(orc, wl, [1] * 100)
    c_mix, *_ = _append_all(orc, wl, [31, 1, 33, 2, 17, 16])
    _same_cache(c_bulk, c_one)
    _same_cache(c_bulk, c_mix)
    assert list(c_bulk.lengths) == [100]


def test_append_resume_invariance(orc):
    wl = W.workload("gqa8k", batch=1, ctx=80)
    wl = W.custom("resume", 9, 1, 8, 2, 128, [80], 96, "bf16", log_uniform_key_scales=True)
    full, k, v, a, b = _append_all(orc, wl, [80])
    part = orc.Cache(wl.batch, wl.hkv, wl.d, wl.cap)
    part.append(k[:, :, :45], v[:, :, :45], b, [45])
    resumed = orc.Cache(wl.batch, wl.hkv, wl.d, wl.cap)
    for name, arr in part.planes().items():
        getattr(resumed, name)[...] = arr
    resumed.append(k[:, :, 45:80], v[:, :, 45:80], b, [35])
    _same_cache(full, resumed)


def test_append_dequant_bounds(orc):
    """Stored keys/values stay within the quantizer's error bound of the exact
    transformed inputs (k' from fp64 numpy within the Higham bound)."""
    wl = W.workload("tiny", ctx=100)
    c, k, v, a, b = _append_all(orc, wl, [100])
    kd, vd = c.dequant()
    kp = np.stack([orc.transform(k[0, 0, t], b[0]) for t in range(100)])
    ex = k[0, 0, :100].astype(np.float64) @ b[0].astype(np.float64)
    gam = 64 * 2.0 ** -24 / (1 - 64 * 2.0 ** -24)
    assert np.all(np.abs(kp - ex) <= gam * (np.abs(k[0, 0, :100]).astype(np.float64) @ np.abs(b[0]).astype(np.float64)))
    # channel 0: fp16 of k'_0
    assert np.array_equal(kd[0, 0, :100, 0], kp[:, 0].astype(np.float16).astype(np.float32))
    # channels >= 1: groups 0..2 quantized per channel, tokens 96..99 exact
    for g0 in range(0, 96, 32):
        blk = kp[g0:g0 + 32, 1:]
        m = np.abs(blk).max(0)
        s = m.astype(np.float32) / np.float32(3)
        s = s.astype(np.float16).astype(np.float64)
        err = np.abs(kd[0, 0, g0:g0 + 32, 1:] - blk)
        assert np.all(err <= s + np.maximum(0, m - 3 * s) + 1e-9)
        lv = kd[0, 0, g0:g0 + 32, 1:] / np.where(s > 0, s, 1)
        assert np.all(np.isin(lv[:, s > 0], [-3, -1, 1, 3]))
    assert np.array_equal(kd[0, 0, 96:100, 1:], kp[96:100, 1:])
    assert np.all(kd[0, 0, 100:] == 0) and np.all(vd[0, 0, 100:] == 0)
    # values: per token, groups of 32 channels
    for t in range(100):
        for j in range(wl.d // 32):
            x = v[0, 0, t, 32 * j:32 * j + 32].astype(np.float64)
            m = np.abs(x).max()
            s = float(np.float16(np.float32(m) / np.float32(3)))
            assert np.all(np.abs(vd[0, 0, t, 32 * j:32 * j + 32] - x) <= s + max(0, m - 3 * s) + 1e-9)


def test_append_capacity_clamp_and_zero(orc):
    wl = W.custom("cap", 10, 2, 2, 1, 64, [0, 0], 64, "f32")
    c = orc.Cache(2, 1, 64, 64)
    k = np.random.default_rng(3).standard_normal((2, 1, 80, 64)).astype(np.float32)
    c.append(k, k, np.eye(64, dtype=np.float32)[None], [80, 0])
    assert list(c.lengths) == [64, 0]
    assert not c.k_ch0[1].any() and not c.v_codes[1].any()
    del wl


# ----------------------------------------------------------------------------- attention

def _torch_sdpa64(q, k, v, sm):
    torch = pytest.importorskip("torch")
    qt = torch.tensor(q, dtype=torch.float64)[None, None, None]
    kt = torch.tensor(k, dtype=torch.float64)[None, None]
    vt = torch.tensor(v, dtype=torch.float64)[None, None]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=sm)
    return o[0, 0, 0].numpy()


def test_quant_off_identity_equals_plain_attention(orc):
    """Sparsity 0, no quantization, A = B = I: the pruned decode is the same fp64
    loop as plain attention, so the outputs are bitwise equal."""
    rng = np.random.default_rng(22)
    d, t = 64, 300
    q = rng.standard_normal(d).astype(np.float32)
    k = rng.standard_normal((t, d)).astype(np.float32)
    v = rng.standard_normal((t, d)).astype(np.float32)
    sm = W.default_sm_scale(d)
    eye = np.eye(d, dtype=np.float32)
    qp = orc.transform(q, eye)
    kp = np.stack([orc.transform(k[i], eye) for i in range(t)])
    got = orc.attend_dense(qp, orc.select(qp, d), kp, v, sm)
    ref = orc.plain_attention(q[None, None], k[None, None], v[None, None], [t], sm)[0, 0]
    assert np.array_equal(got, ref)


def test_quant_off_random_transform_matches_plain(orc):
    """Sparsity 0, no quantization, random A: logits agree to the invariance bound,
    so the outputs agree closely."""
    wl = W.workload("tiny")
    a, b = W.transforms(wl)
    rng = np.random.default_rng(23)
    d, t = 64, 256
    q = rng.standard_normal(d).astype(np.float32)
    k = rng.standard_normal((t, d)).astype(np.float32)
    v = rng.standard_normal((t, d)).astype(np.float32)
    sm = W.default_sm_scale(d)
    qp = orc.transform(q, a[0])
    kp = np.stack([orc.transform(k[i], b[0]) for i in range(t)])
    got = orc.attend_dense(qp, np.arange(d, dtype=np.int32), kp, v, sm)
    ref = orc.plain_attention(q[None, None], k[None, None], v[None, None], [t], sm)[0, 0]
    assert np.abs(got - ref).max() <= 1e-4 * np.abs(ref).max()


def test_plain_attention_matches_torch(orc):
    rng = np.random.default_rng(24)
    q = rng.standard_normal((2, 4, 32)).astype(np.float32)
    k = rng.standard_normal((2, 2, 40, 32)).astype(np.float32)
    v = rng.standard_normal((2, 2, 40, 32)).astype(np.float32)
    lens = [40, 17]
    out = orc.plain_attention(q, k, v, lens, 0.3)
    for bb in range(2):
        for h in range(4):
            ref = _torch_sdpa64(q[bb, h], k[bb, h // 2, :lens[bb]], v[bb, h // 2, :lens[bb]], 0.3)
            assert np.allclose(out[bb, h], ref, rtol=0, atol=2e-7 * np.abs(ref).max())


def _small_cache(orc, kind="gqa8k", batch=2, ctx=200, **kw):
    if kind == "custom":
        wl = W.custom(ctx=ctx, batch=batch, **kw)
    else:
        wl = W.workload(kind, batch=batch, ctx=ctx)
    a, b = W.transforms(wl)
    c = orc.Cache(wl.batch, wl.hkv, wl.d, wl.cap)
    k, v = W.prefill_kv(wl)
    c.append(k, v, b, list(wl.ctx))
    return wl, a, b, c


def test_decode_matches_torch_on_dequantized_cache(orc):
    """Library reduction: the pruned logit is (q' masked to its kept channels) . K~,
    so decode equals fp64 attention of the masked q' over the dequantized cache."""
    for sm_mult in (1.0, 0.01):
        wl, a, b, c = _small_cache(orc, ctx=200)
        q = W.queries(wl)
        keep = orc.keep_count(wl.d, 40)
        qp, idx = orc.queries(q, a, wl.hkv, keep)
        sm = W.default_sm_scale(wl.d) * sm_mult
        out = c.decode(qp, idx, sm)
        kd, vd = c.dequant()
        for bb in range(wl.batch):
            for h in range(wl.hq):
                mask = np.zeros(wl.d)
                mask[idx[bb, h]] = 1.0
                g = h // wl.group
                n = int(c.lengths[bb])
                ref = _torch_sdpa64(qp[bb, h].astype(np.float64) * mask, kd[bb, g, :n],
                                    vd[bb, g, :n], sm)
                assert np.allclose(out[bb, h], ref, rtol=0, atol=2e-7 * np.abs(ref).max())


def test_decode_special_cases(orc):
    # one token: the output is that token's stored value
    wl, a, b, c = _small_cache(orc, "custom", name="one", cid=11, batch=1, hq=2, hkv=1, d=64,
                               ctx=[1], cap=32, dtype="f32")
    q = W.queries(wl)
    qp, idx = orc.queries(q, a, 1, 38)
    out = c.decode(qp, idx, 0.125)
    _, vd = c.dequant()
    assert np.array_equal(out[0, 0], vd[0, 0, 0]) and np.array_equal(out[0, 1], vd[0, 0, 0])
    # q' = 0: every logit is 0, the output is the mean of the stored values
    wl, a, b, c = _small_cache(orc, "custom", name="flat", cid=12, batch=1, hq=1, hkv=1, d=64,
                               ctx=[77], cap=96, dtype="f32")
    qp = np.zeros((1, 1, 64), dtype=np.float32)
    idx = np.arange(38, dtype=np.int32)[None, None]
    out = c.decode(qp, idx, 0.125)
    _, vd = c.dequant()
    assert np.allclose(out[0, 0], vd[0, 0, :77].astype(np.float64).mean(0), rtol=0, atol=1e-6)
    # empty sequence: zeros
    c.lengths[0] = 0
    assert not c.decode(np.ones((1, 1, 64), np.float32), idx, 0.125).any()


def test_decode_logit_shift_invariance(orc):
    """Adding the same constant to every logit leaves the output unchanged: with
    every stored channel-0 key equal, changing q'_0 shifts all logits alike."""
    rng = np.random.default_rng(25)
    d, t = 64, 150
    k = rng.standard_normal((t, d)).astype(np.float32)
    k[:, 0] = 1.0
    v = rng.standard_normal((t, d)).astype(np.float32)
    qp = rng.standard_normal(d).astype(np.float32)
    idx = orc.select(qp, 38)
    base = orc.attend_dense(qp, idx, k, v, 0.2)
    for shift in (-5.0, 3.0, 40.0):
        q2 = qp.copy()
        q2[0] += shift
        assert np.allclose(orc.attend_dense(q2, idx, k, v, 0.2), base, rtol=0,
                           atol=1e-6 * np.abs(base).max())


# ----------------------------------------------------------------------------- bytes

def test_decode_bytes_closed_form(orc):
    """Bytes a pruned decode must touch, marked element by element, equal the
    closed form: per (batch row, KV head) with union U of kept channels >= 1,
    T tokens and Tb = 32 floor(T/32):
    |U| Tb/4 + 2|U| Tb/32 + 2T + 4|U|(T-Tb) + d ceil(T/4) + 2T d/32."""
    wl, a, b, c = _small_cache(orc, "custom", name="bytes", cid=13, batch=2, hq=8, hkv=2,
                               d=128, ctx=[200, 77], cap=224, dtype="bf16",
                               log_uniform_key_scales=True)
    keep = 77
    qp, idx = orc.queries(W.queries(wl), a, wl.hkv, keep)
    got = c.decode_bytes(idx)
    exp = np.zeros(7, dtype=np.int64)
    for bb in range(wl.batch):
        t = int(c.lengths[bb])
        tb = t // 32 * 32
        for g in range(wl.hkv):
            u = set()
            for h in range(g * wl.group, (g + 1) * wl.group):
                u |= set(int(x) for x in idx[bb, h] if x != 0)
            n = len(u)
            exp += [n * tb // 4, 2 * n * tb // 32, 2 * t, 4 * n * (t - tb),
                    wl.d * ((t + 3) // 4), 2 * t * wl.d // 32,
                    wl.group * (8 * keep + 4 * wl.d)]
    assert list(got.astype(np.int64)) == list(exp)


def test_value_packing_layout(orc):
    """Value code of token t, channel c sits at bits 2(t mod 16) of 32-bit word
    (t div 16)*d + c.  Tokens whose 32-channel groups are the grid values
    s*(2u-3) with u = (t + c) mod 4 (and a +-3 level in every group) give known
    codes, so every word is a closed form."""
    d, n = 64, 40
    u = (np.arange(n)[:, None] + np.arange(d)[None, :]) % 4
    v = (2.0 * u - 3).astype(np.float32)          # s = 1 in every group
    c = orc.Cache(1, 1, d, 64)
    z = np.zeros((1, 1, n, d), dtype=np.float32)
    c.append(z, v[None, None], np.eye(d, dtype=np.float32)[None], [n])
    for blk in range((n + 15) // 16):
        for ch in range(d):
            want = 0
            for t in range(16 * blk, min(16 * blk + 16, n)):
                want |= int(u[t, ch]) << (2 * (t % 16))
            assert int(c.v_codes[0, 0, blk, ch]) == want
    assert np.all(c.v_scales[0, 0, :n] == 0x3C00)


# ----------------------------------------------------------------------------- group-shared selection

def _score_beats(score, a, b):
    return score[a] > score[b] or (score[a] == score[b] and a < b)


def test_select_shared_single_head_is_per_head(orc):
    """A group of one: the score is |q'| (0 + |x| is exact), so the shared set is
    the per-head set, itself pinned by brute force and lexsort."""
    rng = np.random.default_rng(40)
    for d in (8, 64, 128):
        for keep in (1, 2, d // 2, d - 1, d):
            qp = rng.standard_normal((1, d)).astype(np.float32)
            assert np.array_equal(orc.select_shared(qp, keep), orc.select(qp[0], keep))


def test_select_shared_equal_magnitudes_match_one_head(orc):
    """Heads whose |q'| rows are equal (signs flipped at random) and hold at most
    20 significant bits: every partial sum is exact, so score = G |q'| and the
    shared set is that of any one head."""
    rng = np.random.default_rng(41)
    for grp in (2, 4, 8):
        for d in (64, 128):
            row = (rng.integers(-(1 << 12), 1 << 12, d) / 256.0).astype(np.float32)
            qp = (row[None] * rng.choice([-1.0, 1.0], (grp, d))).astype(np.float32)
            for keep in (1, 38, 51, 77, d):
                if keep <= d:
                    assert np.array_equal(orc.select_shared(qp, keep), orc.select(row, keep))


def test_select_shared_brute_force_tiny(orc):
    """Every kept set containing channel 0 is enumerated; exactly one has every
    kept channel >= 1 beating every dropped one on (score desc, index asc), where
    the score is the fp32 sum of |q'| over the group's heads in ascending order
    (numpy float32 scalars: one IEEE rounding per addition)."""
    rng = np.random.default_rng(42)
    for trial in range(200):
        d = int(rng.integers(2, 11))
        grp = int(rng.choice([1, 2, 3, 4, 8]))
        keep = int(rng.integers(1, d + 1))
        qp = rng.standard_normal((grp, d)).astype(np.float32)
        if trial % 3 == 0:   # forced ties
            qp = rng.choice(np.array([0.0, -0.0, 1.5, -1.5, 2.0], dtype=np.float32), (grp, d))
        score = []
        for c in range(d):
            acc = np.float32(0.0)
            for h in range(grp):
                acc = np.float32(acc + np.float32(abs(qp[h, c])))
            score.append(acc)
        valid = []
        for rest in itertools.combinations(range(1, d), keep - 1):
            kept = set(rest)
            dropped = [c for c in range(1, d) if c not in kept]
            if all(_score_beats(score, a, b) for a in kept for b in dropped):
                valid.append(sorted((0,) + rest))
        assert len(valid) == 1
        assert list(orc.select_shared(qp, keep)) == valid[0]


def test_select_shared_summation_order(orc):
    """The group's score is added in ascending head order.  Channel 1 holds
    1, 2^-24, 2^-24 over three heads: ascending, each addition ties and rounds
    to even, leaving 1; channel 2 holds 2^-24, 2^-24, 1: ascending gives 2^-23,
    then 1 + 2^-23 (exact).  So channel 2 wins the single free slot; summed in
    descending order the two scores would swap and channel 1 would win."""
    qp = np.zeros((3, 4), dtype=np.float32)
    qp[:, 1] = [1.0, 2.0 ** -24, 2.0 ** -24]
    qp[:, 2] = [2.0 ** -24, 2.0 ** -24, 1.0]
    assert list(orc.select_shared(qp, 2)) == [0, 2]
    assert list(orc.select_shared(qp[::-1].copy(), 2)) == [0, 1]


def test_select_shared_large_against_lexsort(orc):
    rng = np.random.default_rng(43)
    for grp in (2, 4, 8):
        for d in (64, 128):
            for keep in (1, 38, 51, 77, d):
                if keep > d:
                    continue
                qp = rng.standard_normal((grp, d)).astype(np.float32)
                score = np.zeros(d, dtype=np.float32)
                for h in range(grp):
                    score = (score + np.abs(qp[h])).astype(np.float32)
                c = np.arange(1, d)
                order = np.lexsort((c, -score[1:]))
                ref = np.sort(np.concatenate([[0], c[order][:keep - 1]]))
                assert np.array_equal(orc.select_shared(qp, keep), ref)


def test_queries_shared_groups(orc):
    """q' equals the per-head call's; each (row, KV head) set is the shared
    selection of that group's rows."""
    wl = W.workload("gqa8k", batch=2, ctx=64)
    a, _ = W.transforms(wl)
    q = W.queries(wl)
    qp1, _ = orc.queries(q, a, wl.hkv, 77)
    qp2, idx = orc.queries_shared(q, a, wl.hkv, 77)
    assert np.array_equal(qp1.view(np.uint32), qp2.view(np.uint32))
    assert idx.shape == (2, wl.hkv, 77)
    for bb in range(2):
        for g in range(wl.hkv):
            rows = qp1[bb, g * wl.group:(g + 1) * wl.group]
            assert np.array_equal(idx[bb, g], orc.select_shared(rows, 77))
    assert orc.per_head(idx, wl.group).shape == (2, wl.hq, 77)


# ----------------------------------------------------------------------------- growing a cache

def test_grow_then_append_equals_building_large(orc):
    """Nothing stored depends on the capacity: a cache built at capacity 96,
    grown to 224 and appended to is byte for byte the cache the same appends
    build at capacity 224 (ragged rows, an unfinished key group at the grow, a
    group closed after it), and it decodes to the same output."""
    wl = W.custom("grow", 50, 2, 8, 2, 128, [90, 33], 224, "bf16", log_uniform_key_scales=True)
    a, b = W.transforms(wl)
    k, v = W.prefill_kv(wl)
    small = orc.Cache(2, 2, 128, 96)
    small.append(k[:, :, :90], v[:, :, :90], b, [90, 33])
    grown = small.grow(224)
    assert list(grown.lengths) == [90, 33]
    big = orc.Cache(2, 2, 128, 224)
    big.append(k[:, :, :90], v[:, :, :90], b, [90, 33])
    rng = np.random.default_rng(51)
    more = W.round_bf16(rng.standard_normal((2, 2, 100, 128)).astype(np.float32))[0]
    grown.append(more, more, b, [100, 7])
    big.append(more, more, b, [100, 7])
    for name, arr in big.planes().items():
        g = grown.planes()[name]
        if name == "k_tail":
            for bb in range(2):
                r = int(big.lengths[bb]) % 32
                assert np.array_equal(g[bb, :, :r], arr[bb, :, :r])
        else:
            assert np.array_equal(g, arr), name
    qp, idx = orc.queries(W.queries(wl), a, 2, 77)
    sm = W.default_sm_scale(128)
    assert np.array_equal(grown.decode(qp, idx, sm).view(np.uint32), big.decode(qp, idx, sm).view(np.uint32))


def test_grow_same_capacity_is_a_copy(orc):
    wl = W.custom("grow2", 52, 1, 4, 1, 64, [70], 96, "f32")
    _, b = W.transforms(wl)
    k, v = W.prefill_kv(wl)
    c = orc.Cache(1, 1, 64, 96)
    c.append(k[:, :, :70], v[:, :, :70], b, [70])
    g = c.grow(96)
    for name, arr in c.planes().items():
        assert np.array_equal(g.planes()[name], arr), name
