"""CPU checks of the C ABI: the library loads, exports every declared entry point,
and rejects invalid arguments on the host before any device work.  No call here
reaches a kernel launch."""
import ctypes as C
import os
import re

import pytest

import bit_quantized_decode_dqk_amd as M

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dqk.h")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, -1, -2, -3


def declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dqk_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    L = M.lib()
    names = declared()
    assert "dqk_decode_attention" in names and "dqk_transform_quantize_append" in names
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(M.EXPORTS)


def test_status_strings():
    L = M.lib()
    for s in (OK, INVALID, UNSUPPORTED, WORKSPACE, -4):
        assert L.dqk_status_str(s)
    assert L.dqk_status_str(OK) == b"ok"


def test_plane_bytes():
    assert M.cache_plane_bytes(1, 8, 128, 131104) == [
        8 * 128 * 131104 // 4, 8 * 128 * (131104 // 32) * 2, 8 * 131104 * 2, 8 * 32 * 128 * 4,
        8 * (131104 // 16) * 128 * 4, 8 * 131104 * 4 * 2, 8]   # lengths + arrival counters
    out = (C.c_size_t * 7)()
    L = M.lib()
    assert L.dqk_cache_plane_bytes(1, 1, 96, 64, out) == UNSUPPORTED
    assert L.dqk_cache_plane_bytes(1, 1, 64, 48, out) == INVALID
    assert L.dqk_cache_plane_bytes(0, 1, 64, 64, out) == INVALID
    assert L.dqk_cache_plane_bytes(1, 1, 64, 64, None) == INVALID


def fake_cache(**kw):
    """A cache descriptor with aligned, non-null placeholder pointers."""
    vals = dict(batch=2, num_kv_heads=2, head_dim=128, capacity=256)
    vals.update({k: v for k, v in kw.items() if k in vals})
    ptrs = {n: 0x10000 * (i + 1) for i, n in enumerate(M.PLANES)}
    ptrs.update({k: v for k, v in kw.items() if k in ptrs})
    return M._Cache(vals["batch"], vals["num_kv_heads"], vals["head_dim"], vals["capacity"],
                    *(ptrs[n] for n in M.PLANES))


def test_cache_validation_without_gpu():
    L = M.lib()
    out = C.c_size_t(0)
    assert L.dqk_decode_workspace_bytes(C.byref(fake_cache()), 8, 0, C.byref(out)) == OK
    assert out.value == 2 * 2 * 1 * 4 * 132 * 4          # 1 default split covers 256 tokens
    assert L.dqk_decode_workspace_bytes(C.byref(fake_cache()), 8, 64, C.byref(out)) == OK
    assert out.value == 2 * 2 * 4 * 4 * 132 * 4
    for bad in (dict(capacity=100), dict(batch=0), dict(k_codes=0), dict(v_codes=0x10004),
                dict(lengths=0)):
        assert L.dqk_decode_workspace_bytes(C.byref(fake_cache(**bad)), 8, 0, C.byref(out)) == INVALID
    assert L.dqk_decode_workspace_bytes(C.byref(fake_cache(head_dim=96)), 8, 0, C.byref(out)) == UNSUPPORTED
    assert L.dqk_decode_workspace_bytes(C.byref(fake_cache()), 6, 0, C.byref(out)) == UNSUPPORTED
    assert L.dqk_decode_workspace_bytes(C.byref(fake_cache()), 8, 48, C.byref(out)) == INVALID
    assert L.dqk_decode_workspace_bytes(C.byref(fake_cache()), 8, 2048, C.byref(out)) == OK
    assert out.value == 2 * 2 * 1 * 4 * 132 * 4          # one split longer than the capacity
    assert L.dqk_decode_workspace_bytes(C.byref(fake_cache()), 8, -32, C.byref(out)) == INVALID
    assert L.dqk_decode_workspace_bytes(C.byref(fake_cache()), 16, 1056, C.byref(out)) == OK
    assert L.dqk_decode_workspace_bytes(None, 8, 0, C.byref(out)) == INVALID


def test_default_split_for_groups_of_four():
    """Default split of the four-head decode, read back through the workspace
    size (one partial of G heads x (d + 4) floats per split and (row, KV head)):
    about 512 workgroups (two per compute unit on 256), at least 256 tokens of
    capacity each, unless the capacity alone gives more than 21 blocks per slot.
    Groups of eight run one eight-head workgroup per split, on 128-token blocks:
    the same rule in those blocks, with fixed splits of 31 of them (3968 tokens)."""
    L = M.lib()
    out = C.c_size_t(0)

    def splits(batch, hkv, cap, group=4):
        c = fake_cache(batch=batch, num_kv_heads=hkv, capacity=cap)
        assert L.dqk_decode_workspace_bytes(C.byref(c), group * hkv, 0, C.byref(out)) == OK
        per = batch * hkv * group * 132 * 4
        assert out.value % per == 0
        return out.value // per

    # more than 21 blocks per slot of 512 from the capacity alone: whole-block
    # splits of 21 blocks (5376 tokens)
    assert splits(16, 8, 65536, 8) == 17       # 128 units x 512 blocks of 128: 3968-token splits
    assert splits(8, 8, 131072) == 25          # 64 units x 512 blocks
    assert splits(8, 8, 32768) == 8            # 64 x 128 blocks = 8192: balanced, 8 per unit
    assert splits(8, 8, 32768 + 192) == 8      # 64 x 129 blocks: still balanced
    assert splits(1, 8, 131072, 8) == 64        # 8 eight-head workgroups per split index
    assert splits(1, 1, 4096, 8) == 16          # at least 256 tokens per split

    assert splits(1, 8, 131072) == 64
    assert splits(1, 8, 131328) == 64          # 513 blocks: one split of nine
    assert splits(1, 8, 131072 + 768) == 64
    assert splits(1, 8, 32768) == 64           # 128 blocks: 2 per split
    assert splits(4, 8, 8192) == 16            # 32 units x 16 splits of 2 blocks
    assert splits(1, 1, 512) == 2              # at least 256 tokens per split


def test_decode_validation_without_gpu():
    L = M.lib()
    c = C.byref(fake_cache())
    q, idx, out, ws = 0x20000, 0x30000, 0x40000, 0x50000
    big = 1 << 30
    assert L.dqk_decode_attention(c, None, idx, 8, 77, 0.1, 0, out, ws, big, None) == INVALID
    assert L.dqk_decode_attention(c, q, idx, 8, 0, 0.1, 0, out, ws, big, None) == INVALID
    assert L.dqk_decode_attention(c, q, idx, 8, 129, 0.1, 0, out, ws, big, None) == INVALID
    assert L.dqk_decode_attention(c, q, idx, 7, 77, 0.1, 0, out, ws, big, None) == INVALID
    assert L.dqk_decode_attention(c, q, idx, 6, 77, 0.1, 0, out, ws, big, None) == UNSUPPORTED
    assert L.dqk_decode_attention(c, q, idx, 8, 77, float("nan"), 0, out, ws, big, None) == INVALID
    assert L.dqk_decode_attention(c, q, idx, 8, 77, 0.1, 33, out, ws, big, None) == INVALID
    assert L.dqk_decode_attention(c, q, idx, 8, 77, 0.1, 0, out, None, big, None) == WORKSPACE
    assert L.dqk_decode_attention(c, q, idx, 8, 77, 0.1, 0, out, ws, 16, None) == WORKSPACE
    assert L.dqk_decode_attention(c, q, idx, 8, 77, 0.1, 0, out, ws + 4, big, None) == WORKSPACE


def test_noalloc_decode_validation_without_gpu():
    """The decode entry point without a workspace validates like the decode and
    refuses, before anything is launched, a shape whose partials exceed its
    16 MiB device scratch."""
    L = M.lib()
    q, idx, out = 0x20000, 0x30000, 0x40000
    c = C.byref(fake_cache())
    assert L.dqk_decode_attention_noalloc(c, None, idx, 8, 77, 0.1, 0, out, None) == INVALID
    assert L.dqk_decode_attention_noalloc(c, q, idx, 8, 0, 0.1, 0, out, None) == INVALID
    assert L.dqk_decode_attention_noalloc(c, q, idx, 6, 77, 0.1, 0, out, None) == UNSUPPORTED
    assert L.dqk_decode_attention_noalloc(c, q, idx, 8, 77, 0.1, 48, out, None) == INVALID
    big = C.byref(fake_cache(batch=64, num_kv_heads=8, capacity=131072))
    need = C.c_size_t(0)
    assert L.dqk_decode_workspace_bytes(big, 32, 256, C.byref(need)) == OK
    assert need.value > M.DECODE_SCRATCH_BYTES
    assert L.dqk_decode_attention_noalloc(big, q, idx, 32, 77, 0.1, 256, out, None) == WORKSPACE


def test_cache_grow_validation_without_gpu():
    """dqk_cache_grow refuses differing shapes, a smaller destination and planes
    that overlap, before anything is launched."""
    L = M.lib()
    src = fake_cache()
    far = {n: 0x1000000 * (i + 1) for i, n in enumerate(M.PLANES)}
    dst = fake_cache(capacity=512, **far)
    assert L.dqk_cache_grow(None, C.byref(dst), None) == INVALID
    assert L.dqk_cache_grow(C.byref(src), None, None) == INVALID
    assert L.dqk_cache_grow(C.byref(src), C.byref(fake_cache(capacity=128, **far)), None) == INVALID
    assert L.dqk_cache_grow(C.byref(src), C.byref(fake_cache(capacity=512, batch=3, **far)), None) == INVALID
    assert L.dqk_cache_grow(C.byref(src), C.byref(fake_cache(capacity=512, num_kv_heads=1, **far)), None) == INVALID
    assert L.dqk_cache_grow(C.byref(src), C.byref(fake_cache(capacity=512, head_dim=64, **far)), None) == INVALID
    assert L.dqk_cache_grow(C.byref(src), C.byref(fake_cache(capacity=512)), None) == INVALID   # same planes
    assert L.dqk_cache_grow(C.byref(src), C.byref(fake_cache(capacity=100, **far)), None) == INVALID


def test_stream_read_validation_without_gpu():
    """The read probe rejects null or misaligned pointers and sizes that are not
    whole 16-byte elements before launching anything."""
    L = M.lib()
    buf, sink = 0x20000, 0x30000
    assert L.dqk_stream_read(buf, 1 << 20, None, None) == INVALID
    assert L.dqk_stream_read(buf, 1 << 20, sink + 4, None) == INVALID
    assert L.dqk_stream_read(buf, (1 << 20) + 8, sink, None) == INVALID
    assert L.dqk_stream_read(None, 1 << 20, sink, None) == INVALID
    assert L.dqk_stream_read(buf + 8, 1 << 20, sink, None) == INVALID


def test_stream_read_config_validation_without_gpu():
    L = M.lib()
    buf, sink = 0x20000, 0x30000
    assert L.dqk_stream_read_config(buf, 1 << 20, sink, 0, 4, None) == INVALID
    assert L.dqk_stream_read_config(buf, 1 << 20, sink, 2049, 4, None) == INVALID
    assert L.dqk_stream_read_config(buf, 1 << 20, sink, 256, 3, None) == INVALID
    assert L.dqk_stream_read_config(buf, 1 << 20, sink, 256, 32, None) == INVALID
    assert L.dqk_stream_read_config(buf + 8, 1 << 20, sink, 256, 4, None) == INVALID
    assert L.dqk_stream_read_config(buf, 1 << 20, None, 256, 4, None) == INVALID


def test_append_select_dequant_validation_without_gpu():
    L = M.lib()
    c = C.byref(fake_cache())
    k, v, b, n = 0x20000, 0x30000, 0x40000, 0x50000
    assert L.dqk_transform_quantize_append(c, None, v, 1, b, n, 4, None) == INVALID
    assert L.dqk_transform_quantize_append(c, k, v, 7, b, n, 4, None) == INVALID
    assert L.dqk_transform_quantize_append(c, k, v, 1, b, None, 4, None) == INVALID
    assert L.dqk_transform_quantize_append(c, k, v, 1, b, n, -1, None) == INVALID
    assert L.dqk_transform_quantize_append(c, k, v, 1, b, n, 257, None) == INVALID
    assert L.dqk_transform_quantize_append(c, k, v, 1, b, n, 0, None) == OK   # nothing to do
    assert L.dqk_transform_quantize_append(C.byref(fake_cache(head_dim=256)), k, v, 1, b, n, 4,
                                           None) == UNSUPPORTED
    q, a, qp, idx = 0x20000, 0x30000, 0x40000, 0x50000
    assert L.dqk_select_channels(q, 1, a, 2, 8, 2, 128, 0, qp, idx, None) == INVALID
    assert L.dqk_select_channels(q, 1, a, 2, 8, 2, 128, 129, qp, idx, None) == INVALID
    assert L.dqk_select_channels(q, 1, a, 2, 8, 3, 128, 77, qp, idx, None) == INVALID
    assert L.dqk_select_channels(q, 1, a, 2, 8, 2, 80, 77, qp, idx, None) == UNSUPPORTED
    assert L.dqk_select_channels(None, 1, a, 2, 8, 2, 128, 77, qp, idx, None) == INVALID
    assert L.dqk_dequant_reference(c, None, 0x20000, None) == INVALID
    assert L.dqk_dequant_reference(C.byref(fake_cache(capacity=0)), 0x10, 0x20, None) == INVALID


def test_fused_append_select_validation_without_gpu():
    """dqk_append_select rejects what either of its two parts rejects (fake cache:
    batch 2, 2 KV heads, head_dim 128, capacity 256)."""
    L = M.lib()
    c = C.byref(fake_cache())
    k, v, b, n = 0x20000, 0x30000, 0x40000, 0x50000
    q, a, qp, idx = 0x60000, 0x70000, 0x80000, 0x90000

    def call(cache=c, k=k, v=v, b=b, n=n, max_new=1, q=q, a=a, hq=8, keep=77, dtype=1, qp=qp,
             idx=idx):
        return L.dqk_append_select(cache, k, v, b, n, max_new, q, a, hq, keep, dtype, qp, idx, None)

    assert call(k=None) == INVALID
    assert call(n=None) == INVALID
    assert call(max_new=-1) == INVALID
    assert call(max_new=257) == INVALID
    assert call(dtype=7) == INVALID
    assert call(q=None) == INVALID
    assert call(a=None) == INVALID
    assert call(idx=None) == INVALID
    assert call(hq=0) == INVALID
    assert call(hq=7) == INVALID          # not a multiple of the KV heads
    assert call(hq=6) == UNSUPPORTED      # group of 3
    assert call(keep=0) == INVALID
    assert call(keep=129) == INVALID
    assert call(cache=C.byref(fake_cache(head_dim=256))) == UNSUPPORTED
    assert call(cache=C.byref(fake_cache(capacity=100))) == INVALID
    assert call(cache=None) == INVALID


def test_bf16_decode_validation_without_gpu():
    L = M.lib()
    out = C.c_size_t(0)
    assert L.dqk_bf16_decode_workspace_bytes(1, 32, 8, 128, 131072, 0, C.byref(out)) == OK
    assert out.value == 8 * 64 * 4 * 132 * 4    # 2048-token splits by default
    assert L.dqk_bf16_decode_workspace_bytes(1, 32, 8, 96, 1024, 0, C.byref(out)) == UNSUPPORTED
    args = [0x20000, 0x30000, 0x40000, 0x50000, 1, 32, 8, 128, 1024, 0.1, 0, 0x60000, 0x70000,
            1 << 30, None]
    bad = list(args)
    bad[1] = 0x30004                      # misaligned keys
    assert L.dqk_bf16_decode_attention(*bad) == INVALID
    bad = list(args)
    bad[0] = 0x20008                      # misaligned queries
    assert L.dqk_bf16_decode_attention(*bad) == INVALID
    bad = list(args)
    bad[12] = None
    assert L.dqk_bf16_decode_attention(*bad) == WORKSPACE
    bad = list(args)
    bad[5] = 24
    assert L.dqk_bf16_decode_attention(*bad) == UNSUPPORTED


def test_keep_count_matches_oracle(orc):
    for d in (64, 128):
        for s in range(0, 101):
            assert M.keep_for_sparsity(d, s) == orc.keep_count(d, s)


def test_binding_raises_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(M, "_lib", None)
    monkeypatch.setattr(M, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(M.DqkError):
        M.lib()
