"""The decode entry point that allocates nothing (dqk_decode_attention_noalloc),
called through the C ABI, against dqk_decode_attention with a caller workspace:
the same kernels and split, so the outputs must be bitwise equal.  Several calls
in a row share the library's one device scratch; each later call is smaller than
the first, so stale partials of the earlier call sit past and inside its range."""
import numpy as np
import pytest
import torch

import bit_quantized_decode_dqk_amd as M
import workloads as W
from gpu_util import dev_f32, dev_i32, dev_input, say

pytestmark = pytest.mark.gpu


def _case(wl, split, keep_pct=40):
    a, b = W.transforms(wl)
    k, v = W.prefill_kv(wl)
    cache = M.Cache(wl.batch, wl.hkv, wl.d, wl.cap)
    n = max(wl.ctx)
    M.transform_quantize_append(cache, dev_input(k[:, :, :n], wl.dtype), dev_input(v[:, :, :n], wl.dtype),
                                dev_f32(b), dev_i32(np.array(wl.ctx)))
    keep = M.keep_for_sparsity(wl.d, keep_pct)
    qp, idx = M.select_channels(dev_input(W.queries(wl), wl.dtype), dev_f32(a), wl.hkv, keep)
    return cache, qp, idx


def test_noalloc_decode_matches_workspace_decode():
    cases = [
        (W.custom("na-g4", 90, 3, 32, 8, 128, [5000, 2049, 257], 5056, "bf16",
                  log_uniform_key_scales=True), 0),         # matrix-core kernel, default split
        (W.custom("na-g4b", 91, 2, 32, 8, 128, [3000, 0], 3008, "bf16",
                  log_uniform_key_scales=True), 512),       # smaller, a fixed split, an empty row
        (W.custom("na-g8", 93, 2, 16, 2, 128, [2500, 700], 2560, "bf16",
                  log_uniform_key_scales=True), 0),         # the eight-head kernel, smaller
        (W.custom("na-g2", 92, 2, 4, 2, 64, [700, 31], 768, "f32"), 0),   # general kernel, smaller
    ]
    sm = W.default_sm_scale(128)
    for wl, split in cases:
        say("no-alloc decode:", wl.describe(), "split", split)
        cache, qp, idx = _case(wl, split)
        ws = torch.empty(M.decode_workspace_bytes(cache, wl.hq, split), dtype=torch.uint8, device="cuda")
        ref = torch.empty((wl.batch, wl.hq, wl.d), dtype=torch.float32, device="cuda")
        M.decode_attention(cache, qp, idx, sm, split, ref, ws)
        for rep in range(2):
            out = torch.full((wl.batch, wl.hq, wl.d), float("nan"), dtype=torch.float32, device="cuda")
            M.decode_attention_noalloc(cache, qp, idx, sm, split, out)
            torch.cuda.synchronize()
            assert np.array_equal(out.cpu().numpy().view(np.uint32), ref.cpu().numpy().view(np.uint32)), (wl.name, rep)
        assert ws.numel() <= M.DECODE_SCRATCH_BYTES

