"""Decode-step benchmark: Dual-QK INT2 pruned decode attention at 128K context.

One step = the whole hot path for one new token of every sequence in the batch:
append (key transform + 2-bit quantize/pack of the new K/V), query transform +
channel selection, pruned decode attention with split-K and combine.
Workload: batch 1, 32 query / 8 KV heads, head_dim 128, 131072-token context,
bf16 inputs, 40% query-channel sparsity (seeded synthetic data).

Several copies of the cache are kept in HBM and the steps rotate through them,
so consecutive steps never find their cache in the 256 MB Infinity Cache: the
measured rate is HBM streaming.  Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

HBM_PEAK_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------- byte accounting

def decode_bytes(idx: np.ndarray, lengths, hkv: int, d: int, keep: int) -> int:
    """Algorithmic bytes of one pruned decode: per (row, KV head) with union U of kept
    channels >= 1 over the group's heads, T tokens, Tb = 32*floor(T/32):
    |U|*Tb/4 (codes) + 2|U|*Tb/32 (scales) + 2T (channel 0) + 4|U|(T-Tb) (tail)
    + d*ceil(T/4) (value codes) + 2T*d/32 (value scales), plus per query head
    q' and indices of kept channels (8*keep) and the fp32 output (4d)."""
    batch, hq, _ = idx.shape
    grp = hq // hkv
    total = 0
    for b in range(batch):
        t = int(lengths[b])
        tb = t // 32 * 32
        for g in range(hkv):
            sel = idx[b, g * grp:(g + 1) * grp].ravel()
            u = len(set(int(c) for c in sel if c != 0))
            total += u * tb // 4 + 2 * u * tb // 32 + 2 * t + 4 * u * (t - tb)
            total += d * ((t + 3) // 4) + 2 * t * d // 32
            total += grp * ((8 * keep if t > 0 else 0) + 4 * d)
    return total


def select_bytes(batch: int, hq: int, hkv: int, d: int, keep: int, in_bytes: int) -> int:
    """q in, A of every KV head, q' and indices out."""
    return batch * hq * d * in_bytes + hkv * d * d * 4 + batch * hq * (4 * d + 4 * keep)


def append_bytes(batch: int, hkv: int, d: int, positions, in_bytes: int) -> int:
    """One new token per (row, KV head): k and v in, B_g in, channel 0, tail row,
    the d value words read and written, value scales; a token closing its
    32-token group also reads 31 tail rows and writes (d-1) 8-byte code runs and
    (d-1) key scales."""
    total = 0
    for b in range(batch):
        p = int(positions[b])
        per = 2 * d * in_bytes + d * d * 4 + 2 + 4 * d + 8 * d + 2 * (d // 32)
        if p % 32 == 31:
            per += 31 * 4 * d + (d - 1) * 10
        total += hkv * per
    return total


# ----------------------------------------------------------------------------- profiles

KERNEL_SOURCES = ("bit_quantized_decode_dqk_amd/csrc/dqk_decode.hip",
                  "bit_quantized_decode_dqk_amd/csrc/dqk_decode8.hip",
                  "bit_quantized_decode_dqk_amd/csrc/dqk_host.h",
                  "bit_quantized_decode_dqk_amd/csrc/dqk_decode4.hip",
                  "bit_quantized_decode_dqk_amd/csrc/dqk_decode_ops.h",
                  "bit_quantized_decode_dqk_amd/csrc/dqk_combine.hip",
                  "bit_quantized_decode_dqk_amd/csrc/dqk_wave.h",
                  "bit_quantized_decode_dqk_amd/csrc/dqk_internal.h")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_kernel_ctx128k_traffic.txt")


def kernel_code(text: str) -> str:
    """C/C++ source with comments removed and whitespace collapsed: what the
    compiler sees of it (string literals in these sources hold no comment marks)."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash(root: str = ROOT, read=None) -> str:
    """Hash of the decode kernels' code (comments and layout ignored), stamped into the
    counter summary so that a summary taken on other code is not used."""
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        if read is None:
            with open(os.path.join(root, rel), encoding="utf-8") as f:
                text = f.read()
        else:
            text = read(rel)
        h.update(kernel_code(text).encode())
    return h.hexdigest()[:16]


def recorded_traffic():
    """HBM bytes per decode launch from the committed counter summary, or None when
    the summary is absent or was taken on different kernel sources."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    fields = {}
    for line in open(TRAFFIC_FILE):
        if ":" in line and not line.startswith((" ", "#")):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    if fields.get("source_hash") != kernel_source_hash():
        return None
    try:
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def summarize_rocprof(directory: str, kernel_regex: str, copy_mib: int) -> None:
    """Print a short text summary of rocprofv3 csv output under `directory`:
    kernel statistics (--kernel-trace --stats) and, when present, per-dispatch
    FETCH_SIZE / WRITE_SIZE of the kernels matching `kernel_regex`, with the
    counter scaled by its reading on a plain copy of `copy_mib` MiB."""
    import csv
    import glob
    import re
    pat = re.compile(kernel_regex)
    for path in sorted(glob.glob(os.path.join(directory, "**", "*kernel_stats.csv"), recursive=True)):
        rows = list(csv.DictReader(open(path)))
        print(f"kernel stats ({os.path.relpath(path, directory)}):")
        print(f"  {'calls':>6} {'avg_us':>9} {'min_us':>9} {'max_us':>9} {'pct':>6}  kernel")
        for r in rows:
            print(f"  {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:9.2f} "
                  f"{float(r['MinNs']) / 1e3:9.2f} {float(r['MaxNs']) / 1e3:9.2f} "
                  f"{float(r['Percentage']):6.2f}  {r['Name'][:110]}")
    for path in sorted(glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True)):
        per = {}
        names = {}
        for r in csv.DictReader(open(path)):
            key = int(r["Dispatch_Id"])
            per.setdefault(key, {})
            per[key][r["Counter_Name"]] = per[key].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
            names[key] = r["Kernel_Name"]
        counters = sorted({c for v in per.values() for c in v})
        for cname in counters:
            target = [per[k][cname] for k in sorted(per) if pat.search(names[k]) and cname in per[k]]
            copies = [per[k][cname] for k in sorted(per)
                      if "copybuffer" in names[k].lower() and cname in per[k]]
            print(f"counter {cname} ({os.path.relpath(path, directory)}): "
                  f"{len(target)} dispatches of /{kernel_regex}/")
            if not target:
                continue
            avg = sum(target) / len(target)
            print(f"  {cname}_avg_kib_per_dispatch: {avg:.1f}")
            if copies and copy_mib > 0:
                big = max(copies)
                factor = copy_mib * 1024.0 / big
                print(f"  copy_kernel_{cname}_kib: {big:.1f} for {copy_mib} MiB moved "
                      f"(factor {factor:.4f} bytes per counted byte)")
                print(f"  {cname}_bytes_per_dispatch_scaled: {avg * 1024.0 * factor:.0f}")


# ----------------------------------------------------------------------------- CPU baseline

def cpu_model() -> str:
    """The host CPU's model name (lscpu, else /proc/cpuinfo)."""
    import subprocess
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                return line.split(":", 1)[1].strip()
    except (OSError, subprocess.SubprocessError):
        pass
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, a, b, keep, sm, budget_s: float = 20.0):
    """The oracle, as written, on a bounded sample: one KV head (its G query heads)
    of the workload at full context: untimed cache build, then timed repeats of
    append-1 + select + decode with OpenMP over query heads.  Rate in GB/s of the
    same algorithmic bytes."""
    import oracle
    ncpu = os.cpu_count() or 1
    threads = max(1, min(ncpu, 16))
    os.environ.setdefault("OMP_NUM_THREADS", str(threads))
    g = 0
    t_ctx = int(wl.ctx[0])
    sub = W.custom("cpu-sample", wl.cid, 1, wl.group, 1, wl.d, [t_ctx], wl.cap, wl.dtype)
    kk, vv = W.unit_kv(wl, 0, g, 0, t_ctx)
    c = oracle.Cache(1, 1, wl.d, wl.cap)
    t0 = time.time()
    c.append(kk[None, None], vv[None, None], b[g:g + 1], [t_ctx])
    build_s = time.time() - t0
    q = W.queries(wl, 0)[:, g * wl.group:(g + 1) * wl.group]
    knew = np.random.default_rng(7).standard_normal((1, 1, 1, wl.d)).astype(np.float32)
    reps, spent, nbytes = 0, 0.0, 0
    while spent < budget_s and reps < 50:
        t0 = time.perf_counter()
        c.append(knew, knew, b[g:g + 1], [1])
        qp, idx = oracle.queries(q, a[g:g + 1], 1, keep)
        c.decode(qp, idx, sm, nthreads=threads)
        spent += time.perf_counter() - t0
        nbytes += (decode_bytes(idx, c.lengths, 1, wl.d, keep)
                   + select_bytes(1, wl.group, 1, wl.d, keep, 2)
                   + append_bytes(1, 1, wl.d, c.lengths - 1, 2))
        reps += 1
    # the same step with the decode on one thread
    reps1, spent1, nbytes1 = 0, 0.0, 0
    while spent1 < budget_s / 3 and reps1 < 10:
        t0 = time.perf_counter()
        c.append(knew, knew, b[g:g + 1], [1])
        qp, idx = oracle.queries(q, a[g:g + 1], 1, keep)
        c.decode(qp, idx, sm, nthreads=1)
        spent1 += time.perf_counter() - t0
        nbytes1 += (decode_bytes(idx, c.lengths, 1, wl.d, keep)
                    + select_bytes(1, wl.group, 1, wl.d, keep, 2)
                    + append_bytes(1, 1, wl.d, c.lengths - 1, 2))
        reps1 += 1
    del sub
    # the decode's OpenMP loop runs over the sample's query heads: at most that many
    # threads are busy
    used = min(threads, wl.group)
    return {"value": round(nbytes / spent / 1e9, 4), "unit": "GB/s", "cores": used,
            "kind": "oracle", "cpu_model": cpu_model(), "cpu_count": ncpu,
            "sample": (f"1 of {wl.hkv} KV heads ({wl.group} query heads) of the workload at "
                       f"{t_ctx} tokens: append 1 + select + decode, {reps} repeats in "
                       f"{spent:.1f}s (cache build {build_s:.1f}s untimed); OpenMP over the "
                       f"{wl.group} query heads ({threads} threads offered)"),
            "ms_per_unit_step": round(1e3 * spent / reps, 2),
            "one_thread": {"value": round(nbytes1 / spent1 / 1e9, 4), "unit": "GB/s", "cores": 1,
                           "ms_per_unit_step": round(1e3 * spent1 / reps1, 2), "repeats": reps1}}


# ----------------------------------------------------------------------------- GPU

def calibration_copy(torch, mib: int) -> None:
    """A device-to-device copy of a known size (three times), the reference that
    scales the HBM byte counters of a profiled run (summarize_rocprof)."""
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--sparsity", type=int, default=40)
    ap.add_argument("--copies", type=int, default=6, help="cache copies rotated through")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true")
    ap.add_argument("--split", type=int, default=0)
    ap.add_argument("--graph", action=argparse.BooleanOptionalAction, default=True,
                    help="also time the steps captured as one HIP graph (the reported value)")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="after the timed steps, copy this many MiB device to device "
                         "(a known-size reference for HBM byte counters)")
    ap.add_argument("--summarize-rocprof", metavar="DIR",
                    help="print a summary of rocprofv3 csv output under DIR and exit")
    ap.add_argument("--kernel-regex", default="decode_kernel")
    ap.add_argument("--only-workload", choices=("tiny", "gqa8k", "append32k", "ragged64k"),
                    help="time only this other workload's steps (for a profiler run) and exit")
    args = ap.parse_args()
    if args.summarize_rocprof:
        summarize_rocprof(args.summarize_rocprof, args.kernel_regex, args.calibrate_copy_mib)
        print(f"source_hash: {kernel_source_hash()}")
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import bit_quantized_decode_dqk_amd as M

    torch.cuda.set_device(0)
    if args.only_workload:
        print(json.dumps(run_configs(M, torch, names=(args.only_workload,))), flush=True)
        if args.calibrate_copy_mib > 0:
            calibration_copy(torch, args.calibrate_copy_mib)
        return
    dev = "cuda"
    wl = W.workload("ctx128k", steps=256)
    keep = M.keep_for_sparsity(wl.d, args.sparsity)
    sm = W.default_sm_scale(wl.d)
    ctx = int(wl.ctx[0])
    log(f"workload {wl.describe()}, keep {keep}")

    t0 = time.time()
    a, b = W.transforms(wl)
    kscale = W.key_scales(wl)
    k_pre = np.zeros((wl.batch, wl.hkv, ctx, wl.d), dtype=np.uint16)
    v_pre = np.zeros_like(k_pre)
    for bb in range(wl.batch):
        for g in range(wl.hkv):
            kk, vv = W.unit_kv(wl, bb, g, 0, ctx, kscale)
            k_pre[bb, g] = W.bf16_bits(kk)
            v_pre[bb, g] = W.bf16_bits(vv)
    log(f"inputs generated in {time.time() - t0:.1f}s")

    def to_bf16(bits):
        return torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)

    a_d = torch.from_numpy(a).to(dev)
    b_d = torch.from_numpy(b).to(dev)
    k_d, v_d = to_bf16(k_pre), to_bf16(v_pre)
    caches = [M.Cache(wl.batch, wl.hkv, wl.d, wl.cap) for _ in range(args.copies)]
    M.transform_quantize_append(caches[0], k_d, v_d, b_d,
                                torch.full((wl.batch,), ctx, dtype=torch.int32, device=dev))
    for c in caches[1:]:
        for name, t in caches[0].planes().items():
            getattr(c, name).copy_(t)
    torch.cuda.synchronize()
    log(f"{args.copies} cache copies of {caches[0].nbytes() / 1e6:.1f} MB built")
    # input statistics: condition number of the query transforms, and the largest
    # transformed key magnitudes (all channels, and channel 0 alone), over the prefill
    cond_a = float(max(np.linalg.cond(a[g].astype(np.float64)) for g in range(wl.hkv)))
    kmax, k0max = 0.0, 0.0
    for g in range(wl.hkv):
        kp = torch.matmul(k_d[:, g].float(), b_d[g])      # k' = k B_g, fp32
        kmax = max(kmax, float(kp.abs().max()))
        k0max = max(k0max, float(kp[..., 0].abs().max()))
        del kp
    inputs = {"cond_A_max": round(cond_a, 1), "max_abs_k_prime": round(kmax, 1),
              "max_abs_k_prime_ch0": round(k0max, 1)}
    log(f"inputs: {inputs}")

    nstep = args.warmup + args.steps
    # step inputs: the eager steps, then the steps captured in the graph (replayed twice)
    ninputs = nstep + (args.steps if args.graph else 0)
    step_kv = torch.randn((ninputs, wl.batch, wl.hkv, 1, wl.d), device=dev).to(torch.bfloat16)
    step_q = torch.stack([to_bf16(W.bf16_bits(W.queries(wl, i))) for i in range(ninputs)])
    ones = torch.ones((wl.batch,), dtype=torch.int32, device=dev)
    qp = torch.empty((wl.batch, wl.hq, wl.d), dtype=torch.float32, device=dev)
    idx = torch.empty((wl.batch, wl.hq, keep), dtype=torch.int32, device=dev)
    out = torch.empty((wl.batch, wl.hq, wl.d), dtype=torch.float32, device=dev)
    ws = torch.empty(M.decode_workspace_bytes(caches[0], wl.hq, args.split), dtype=torch.uint8,
                     device=dev)

    # algorithmic bytes of every step in the order the steps run (selections are
    # deterministic given q; a step's bytes depend on its cache's length)
    graph_idx = list(range(nstep, ninputs))
    schedule = list(range(nstep)) + graph_idx + graph_idx   # eager, graph warm replay, timed replay
    lens = [np.full(wl.batch, ctx, dtype=np.int64) for _ in caches]
    step_bytes, dec_bytes = [], []
    idx_of = {}
    for i in schedule:
        ci = i % len(caches)
        if i not in idx_of:
            M.select_channels(step_q[i], a_d, wl.hkv, keep, qp, idx)
            idx_of[i] = idx.cpu().numpy()
        pos = lens[ci].copy()
        lens[ci] += 1
        db = decode_bytes(idx_of[i], lens[ci], wl.hkv, wl.d, keep)
        dec_bytes.append(db)
        step_bytes.append(db + select_bytes(wl.batch, wl.hq, wl.hkv, wl.d, keep, 2)
                          + append_bytes(wl.batch, wl.hkv, wl.d, pos, 2))

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(nstep)]

    def step(i):
        c = caches[i % len(caches)]
        e = ev[i]
        e[0].record()
        M.append_select(c, step_kv[i], step_kv[i], b_d, ones, step_q[i], a_d, keep, qp, idx)
        e[1].record()
        M.decode_attention(c, qp, idx, sm, args.split, out, ws)
        e[2].record()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.warmup, nstep):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    ms_step = 1e3 * wall / args.steps
    timed = range(args.warmup, nstep)
    dec_ms = [ev[i][1].elapsed_time(ev[i][2]) for i in timed]
    pre_ms = [ev[i][0].elapsed_time(ev[i][1]) for i in timed]
    tot_bytes = sum(step_bytes[i] for i in timed)
    gbs = tot_bytes / wall / 1e9
    dec_avg_ms = float(np.mean(dec_ms))
    dec_gbs = float(np.mean([dec_bytes[i] for i in timed])) / (dec_avg_ms * 1e-3) / 1e9
    log(f"step {ms_step * 1e3:.1f} us, decode (partial+combine) {dec_avg_ms * 1e3:.1f} us "
        f"(p10 {np.percentile(dec_ms, 10) * 1e3:.1f} p90 {np.percentile(dec_ms, 90) * 1e3:.1f}), "
        f"append+select {np.mean(pre_ms) * 1e3:.1f} us, {gbs:.0f} GB/s step, {dec_gbs:.0f} GB/s decode")
    step_us = [(ev[i][0].elapsed_time(ev[i][2])) * 1e3 for i in timed]
    eager = {"ms_per_step": round(ms_step, 5), "value": round(gbs, 2),
             "decode_us_in_step": round(dec_avg_ms * 1e3, 2),
             "step_us_events": {"median": round(float(np.median(step_us)), 2),
                                "p10": round(float(np.percentile(step_us, 10)), 2),
                                "p90": round(float(np.percentile(step_us, 90)), 2)}}

    if args.graph:
        # The same step, K more times, captured once as a HIP graph (no host work per
        # launch) and replayed: one untimed replay, then the timed one.
        def step_plain(i):
            c = caches[i % len(caches)]
            M.append_select(c, step_kv[i], step_kv[i], b_d, ones, step_q[i], a_d, keep, qp, idx)
            M.decode_attention(c, qp, idx, sm, args.split, out, ws)

        graph = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(graph):
            for i in graph_idx:
                step_plain(i)
        graph.replay()
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        graph.replay()
        torch.cuda.synchronize()
        gwall = time.perf_counter() - t_start
        g_bytes = sum(step_bytes[len(schedule) - args.steps:])
        ms_step = 1e3 * gwall / args.steps
        gbs = g_bytes / gwall / 1e9
        log(f"graph-replayed step {ms_step * 1e3:.1f} us, {gbs:.0f} GB/s step")

    if args.calibrate_copy_mib > 0:
        calibration_copy(torch, args.calibrate_copy_mib)

    # The dominant kernel pair for the roofline: the decode alone, launched back to back
    # (in the eager step loop the host launches trail the GPU, so the in-step events also
    # hold launch gaps).
    roof_us, roof_bytes = time_decode(M, torch, wl, caches, step_q[0], a_d, keep, sm, args.split,
                                      out, ws, n=max(args.steps, 20) + 5)
    roof_gbs = roof_bytes / roof_us / 1e3
    log(f"decode back to back: {roof_us:.2f} us, {roof_gbs:.0f} GB/s")

    extras = {}
    if not args.no_extras:
        extras = run_extras(M, torch, wl, caches, a_d, b_d, step_q, qp, idx, out, ws, k_d, v_d,
                            sm, args, roof_us)
        extras["other_workloads"] = run_configs(M, torch)
        extras["transform_fit"] = transform_fit_report(M, torch)
        extras["stream_peak"] = stream_peak(M, torch)

    result = {
        "metric": "decode attention effective HBM GB/s + tokens/s at 128K ctx, INT2, 40% sparsity",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16 MFMA operands (logit weights as two f16 limbs), f32 accumulate",
        "data": "synthetic (seeded; bf16 q/k/v, log-uniform key channel scales, channel 0 x8)",
        "config": {"workload": "ctx128k: batch 1, 32/8 heads, head_dim 128, context 131072, "
                               f"INT2 K/V groups of 32, {args.sparsity}% query-channel sparsity, "
                               "step = append 1 token + select + decode",
                   "global_batch": wl.batch, "seq_len": ctx, "parallelism": "none (1 GPU)",
                   "keep": keep, "cache_copies": args.copies, "inputs": inputs,
                   "timing": ("the K steps captured once as a HIP graph and replayed "
                              "(untimed replay first); the eager loop is under 'eager'"
                              if args.graph else "eager launches")},
        "tokens_per_s": round(wl.batch / (ms_step * 1e-3), 1),
        "roofline": {"bound": "hbm", "achieved": round(roof_gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(roof_gbs / HBM_PEAK_GBS, 4),
                     "traffic": recorded_traffic(),
                     "kernel": "pruned decode (decode4 partial + combine launches, back to back)",
                     "bytes_per_launch": int(roof_bytes),
                     "avg_us": round(roof_us, 2)},
    }
    if args.graph:
        result["eager"] = eager
    if extras:
        result["extras"] = extras
        read_peak = extras.get("stream_peak", {}).get("read_GB/s")
        if read_peak:   # the practical ceiling: a plain streaming read measured in this process
            result["roofline"]["measured_read_peak"] = read_peak
            result["roofline"]["frac_of_measured_read_peak"] = round(roof_gbs / read_peak, 4)
    if extras:
        result["vs_pages"] = pages_comparison(M, wl, extras, roof_us, roof_bytes)
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample ...")
        result["cpu_baseline"] = cpu_baseline(wl, a, b, keep, sm)
    print(json.dumps(result), flush=True)


def transform_fit_report(M, torch, d: int = 128, n_keys: int = 8192, n_q: int = 256,
                         sparsity: int = 40):
    """The paired transforms fitted from covariances (calibrate.fit_transforms) against
    a shared random rotation and no transform, on synthetic statistics: keys with the
    workloads' per-channel scales (log-uniform 0.5..20, channel 0 x8), queries with a
    decaying spectrum i^-1.5 in a random basis.  Keys pass through the library's own
    append (transform, INT2 quantize) and dequant kernels; queries through its
    selection kernel.  Reported per method: the share of |q'|^2 in the kept channels,
    the relative error of the pruned logits (exact keys, then stored INT2 keys) against
    q.k, and of the attention output against exact attention (fp64, host)."""
    from bit_quantized_decode_dqk_amd import calibrate as CAL
    rng = np.random.default_rng(np.random.SeedSequence([0, 6, 0]))
    s = np.exp(rng.uniform(np.log(0.5), np.log(20.0), d))
    s[0] *= 8.0
    sk = np.diag(s ** 2)
    v, _ = np.linalg.qr(rng.standard_normal((d, d)))
    e = np.arange(1, d + 1, dtype=np.float64) ** -1.5
    sq = (v * e) @ v.T
    keys = (rng.standard_normal((n_keys, d)) * s).astype(np.float32)
    vals = rng.standard_normal((n_keys, d)).astype(np.float32)
    qs = (rng.standard_normal((n_q, d)) * np.sqrt(e)) @ v.T
    qs = qs.astype(np.float32)
    keep = M.keep_for_sparsity(d, sparsity)
    sm = 1.0 / np.sqrt(d)
    z_ex = qs.astype(np.float64) @ keys.astype(np.float64).T
    nq_att = 64

    def attend(z, vv):
        z = z * sm
        w = np.exp(z - z.max(axis=1, keepdims=True))
        return (w @ vv) / w.sum(axis=1, keepdims=True)

    o_ex = attend(z_ex[:nq_att], vals.astype(np.float64))
    methods = {"dual_qk_alpha0.5": CAL.fit_transforms(sk, sq, 0.5)[:2],
               "dual_qk_alpha1.0": CAL.fit_transforms(sk, sq, 1.0)[:2],
               "shared_rotation": CAL.rotation_transforms(d, seed=5),
               "identity": (np.eye(d, dtype=np.float32), np.eye(d, dtype=np.float32))}
    out = {"keep": keep, "keys": n_keys, "queries": n_q,
           "what": ("share of |q'|^2 kept; relative Frobenius error of pruned logits (exact k', "
                    "stored INT2 k') and of attention outputs, against exact q.k attention; "
                    "relative MSE of the stored INT2 keys in the transformed space and mapped "
                    "back to the original one")}
    for name, (a, b) in methods.items():
        cache = M.Cache(1, 1, d, n_keys)
        kd = torch.from_numpy(keys).cuda().view(1, 1, n_keys, d)
        vd = torch.from_numpy(vals).cuda().view(1, 1, n_keys, d)
        M.transform_quantize_append(cache, kd, vd, torch.from_numpy(b).cuda()[None],
                                    torch.tensor([n_keys], dtype=torch.int32, device="cuda"))
        kq, vq = M.dequant_reference(cache)
        # each query a batch row of one head over the one KV head
        qp, idx = M.select_channels(torch.from_numpy(qs).cuda()[:, None].contiguous(),
                                    torch.from_numpy(a).cuda()[None], 1, keep)
        qp = qp[:, 0].double().cpu().numpy()
        mask = np.zeros_like(qp)
        np.put_along_axis(mask, idx[:, 0].long().cpu().numpy(), 1.0, axis=1)
        qm = qp * mask
        kexact = keys.astype(np.float64) @ b.astype(np.float64)
        z_prune = qm @ kexact.T
        z_int2 = qm @ kq[0, 0].double().cpu().numpy().T
        e_kept = float(np.mean((qm ** 2).sum(1) / (qp ** 2).sum(1)))
        rel = lambda z: float(np.linalg.norm(z - z_ex) / np.linalg.norm(z_ex))
        o = attend(z_int2[:nq_att], vq[0, 0].double().cpu().numpy())
        # INT2 key error: in the transformed space, and mapped back (k = k' A^T, since
        # A B^T = I), where the methods share one space
        kt = kq[0, 0].double().cpu().numpy()
        mse_t = float(((kt - kexact) ** 2).sum() / (kexact ** 2).sum())
        kback = kt @ a.astype(np.float64).T
        k64 = keys.astype(np.float64)
        mse_o = float(((kback - k64) ** 2).sum() / (k64 ** 2).sum())
        out[name] = {"energy_kept": round(e_kept, 4), "logit_err_pruned": round(rel(z_prune), 4),
                     "logit_err_pruned_int2": round(rel(z_int2), 4),
                     "attn_out_err_int2_pruned": round(float(np.linalg.norm(o - o_ex) / np.linalg.norm(o_ex)), 4),
                     "int2_key_rel_mse_transformed": round(mse_t, 4),
                     "int2_key_rel_mse_original": round(mse_o, 4)}
        del cache
    return out


def pages_comparison(M, wl, extras, dec_us, dec_bytes):
    """Our computed analogues of the three figures the pages give for Dual-QK at 128K
    context (tech.dede.sh summary, "Results at 128K context" and "Throughput on
    SGLang"; arXiv abstract): 6.8x KV-cache compression, an estimated 8.3x reduction
    of KV reads, and up to 3.75x decode throughput, each against unpruned BF16.  The
    pages' format, models and hardware are not stated, so theirs are context only."""
    ctx = int(wl.ctx[0])
    units = wl.batch * wl.hkv
    bf16_kv = units * ctx * wl.d * 2 * 2
    planes = M.cache_plane_bytes(wl.batch, wl.hkv, wl.d, ctx)[:6]   # codes, scales, ch0, tail
    out = {"storage_ratio_vs_bf16": {"ours": round(bf16_kv / sum(planes), 3), "pages": 6.8,
                                     "basis": "bf16 K+V bytes / stored INT2 planes at 131072 tokens"},
           "read_reduction_vs_bf16": {"ours_per_head_selection": round(bf16_kv / dec_bytes, 3),
                                      "pages_estimate": 8.3,
                                      "basis": "bf16 K+V bytes / algorithmic bytes of one decode"}}
    sh = extras.get("decode_shared_s40")
    if sh:
        out["read_reduction_vs_bf16"]["ours_group_shared_selection"] = round(bf16_kv / sh["bytes"], 3)
    bf = extras.get("bf16_unpruned_decode")
    if bf:
        sp = {"measured": round(bf["us"] / dec_us, 3), "pages_up_to": 3.75,
              "basis": "bf16 comparator time / pruned INT2 decode time, same context and GPU"}
        peak = extras.get("stream_peak", {}).get("read_GB/s")
        if peak:   # the bf16 read at the best measured read rate: a comparator at its ceiling
            sp["vs_bf16_at_measured_read_ceiling"] = round(bf["bytes"] / peak / 1e3 / dec_us, 3)
        out["decode_speedup_vs_bf16"] = sp
    return out


def time_decode(M, torch, wl, caches, q, a_d, keep, sm, split, out, ws, n=40, skip=5,
                shared=False):
    """Back-to-back decode launches (partial + combine) over the rotating caches at
    their current lengths, each bracketed by HIP events on the launch stream; the host
    stays ahead of the GPU, so an interval is the two kernels and the gap between
    them.  shared: group-shared kept sets (one per KV head).  Returns (mean us per
    launch, mean algorithmic bytes per launch)."""
    qp = torch.empty((wl.batch, wl.hq, wl.d), dtype=torch.float32, device=out.device)
    if shared:
        idx = torch.empty((wl.batch, wl.hkv, keep), dtype=torch.int32, device=out.device)
        M.select_channels_shared(q, a_d, wl.hkv, keep, qp, idx)
        idx_np = np.repeat(idx.cpu().numpy(), wl.group, axis=1)   # the same set for each head
        decode = M.decode_attention_shared
    else:
        idx = torch.empty((wl.batch, wl.hq, keep), dtype=torch.int32, device=out.device)
        M.select_channels(q, a_d, wl.hkv, keep, qp, idx)
        idx_np = idx.cpu().numpy()
        decode = M.decode_attention
    nbytes = [decode_bytes(idx_np, c.lengths.cpu().numpy(), wl.hkv, wl.d, keep) for c in caches]
    ts = []
    for i in range(n):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        decode(caches[i % len(caches)], qp, idx, sm, split, out, ws)
        e1.record()
        ts.append((e0, e1))
    torch.cuda.synchronize()
    us = float(np.mean([a.elapsed_time(b) for a, b in ts[skip:]])) * 1e3
    return us, float(np.mean([nbytes[i % len(caches)] for i in range(skip, n)]))


def run_extras(M, torch, wl, caches, a_d, b_d, step_q, qp, idx, out, ws, k_d, v_d, sm, args,
               dec_us):
    """Decode-only timings for the sparsity sweep and the unpruned BF16 comparator."""
    res = {}
    for s in (0, 40, 60):
        keep = M.keep_for_sparsity(wl.d, s)
        us, nb = time_decode(M, torch, wl, caches, step_q[0], a_d, keep, sm, args.split, out, ws)
        res[f"decode_s{s}"] = {"us": round(us, 2), "GB/s": round(nb / us / 1e3, 1),
                               "bytes": int(nb)}
    # group-shared selection: one kept set per KV head, so the dropped channels leave
    # the key reads of the whole group
    keep = M.keep_for_sparsity(wl.d, 40)
    us, nb = time_decode(M, torch, wl, caches, step_q[0], a_d, keep, sm, args.split, out, ws,
                         shared=True)
    res["decode_shared_s40"] = {"us": round(us, 2), "GB/s": round(nb / us / 1e3, 1),
                                "bytes": int(nb), "frac_of_8TB/s": round(nb / us / 1e3 / HBM_PEAK_GBS, 4),
                                "selection": "group-shared (one kept set per KV head)"}
    # bulk (prefill) append of the whole context into an empty cache: the key
    # transform (one fp32 FMA chain of d products per output), quantize and pack
    ctx = int(wl.ctx[0])
    counts = torch.full((wl.batch,), ctx, dtype=torch.int32, device=qp.device)
    fresh = M.Cache(wl.batch, wl.hkv, wl.d, wl.cap)
    ts = []
    for _ in range(4):
        for t in fresh.planes().values():
            t.zero_()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        M.transform_quantize_append(fresh, k_d, v_d, b_d, counts)
        e1.record()
        ts.append((e0, e1))
    torch.cuda.synchronize()
    us = float(np.mean([x.elapsed_time(y) for x, y in ts[1:]])) * 1e3
    fma = wl.batch * wl.hkv * ctx * wl.d * wl.d
    moved = (2 * wl.batch * wl.hkv * ctx * wl.d * 2 + wl.hkv * wl.d * wl.d * 4
             + sum(M.cache_plane_bytes(wl.batch, wl.hkv, wl.d, ctx)[:6]))
    res["bulk_append_128k"] = {"us": round(us, 1), "GB/s": round(moved / us / 1e3, 1),
                               "bytes": int(moved), "fma": int(fma),
                               "TFLOP/s": round(2 * fma / us / 1e6, 2),
                               "frac_of_fp32_vector_157.3": round(2 * fma / us / 1e6 / 157.3, 4),
                               "what": (f"{wl.batch}x{wl.hkv} units x {ctx} tokens appended in one "
                                        "call: bf16 k, v in; k' = k B (fp32 FMA chains); INT2 planes out")}
    # growing a full cache into a larger one (every plane re-strided)
    # (one untimed call, then five timed ones into the same destination: the copy is idempotent)
    grown = M.Cache(wl.batch, wl.hkv, wl.d, wl.cap + 32768)
    M.cache_grow(fresh, wl.cap + 32768, out=grown)
    torch.cuda.synchronize()
    gts = []
    for _ in range(5):
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        M.cache_grow(fresh, wl.cap + 32768, out=grown)
        t1.record()
        gts.append((t0, t1))
    torch.cuda.synchronize()
    gus = float(np.mean([a.elapsed_time(b) for a, b in gts])) * 1e3
    moved = 2 * fresh.nbytes()   # every plane of the source read once and written once
    res["cache_grow"] = {"us": round(gus, 1), "GB/s": round(moved / gus / 1e3, 1),
                         "bytes": int(moved), "from_cap": wl.cap, "to_cap": wl.cap + 32768}
    del fresh, grown
    torch.cuda.empty_cache()
    # unpruned bf16 decode over the raw cache (2 copies rotate: 537 MB each)
    k2, v2 = k_d.clone(), v_d.clone()
    pairs = [(k_d, v_d), (k2, v2)]
    lengths = torch.full((wl.batch,), ctx, dtype=torch.int32, device=qp.device)
    wsb = torch.empty(M.bf16_decode_workspace_bytes(wl.batch, wl.hq, wl.hkv, wl.d, ctx),
                      dtype=torch.uint8, device=qp.device)
    ts = []
    for i in range(30):
        kk, vv = pairs[i % 2]
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        M.bf16_decode_attention(step_q[i % len(step_q)], kk, vv, lengths, sm, 0, out, wsb)
        e1.record()
        ts.append((e0, e1))
    torch.cuda.synchronize()
    us = float(np.mean([a.elapsed_time(b) for a, b in ts[5:]])) * 1e3
    nb = wl.batch * wl.hkv * ctx * wl.d * 2 * 2 + wl.batch * wl.hq * wl.d * (2 + 4)
    res["bf16_unpruned_decode"] = {"us": round(us, 2), "GB/s": round(nb / us / 1e3, 1),
                                   "bytes": nb,
                                   "speedup_int2_pruned_vs_bf16": round(us / dec_us, 3)}
    del k2, v2
    return res



def stream_peak(M, torch, mib: int = 4096, reps: int = 10):
    """Practical HBM ceilings on a 4 GiB buffer (far past the 256 MB Infinity
    Cache): the library's plain streaming-read kernel, and a device copy (read +
    write, torch), both in GB/s of bytes moved.  Context for the roofline
    fraction."""
    n = (mib << 20) // 4
    x = torch.ones(n, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    sink = torch.empty(M.STREAM_READ_SINK_WORDS, dtype=torch.int32, device="cuda")
    res = {}
    for name, fn, moved in (("read", lambda: M.stream_read(x, sink), 4 * n),
                            ("copy", lambda: y.copy_(x), 8 * n)):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        res[f"{name}_GB/s"] = round(moved * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)
    # the probe's launch shape swept: workgroups x 16-byte loads in flight per thread
    sweep = {}
    for wg in (256, 512, 1024, 2048):
        for lif in (1, 2, 4, 8, 16):
            M.stream_read_config(x, wg, lif, sink)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(4):
                M.stream_read_config(x, wg, lif, sink)
            e1.record()
            torch.cuda.synchronize()
            sweep[f"{wg}x{lif}"] = round(4 * 4 * n / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)
    best = max(sweep, key=sweep.get)
    res["read_sweep_GB/s"] = sweep
    res["read_best"] = {"config": best + " (workgroups x loads in flight)", "GB/s": sweep[best]}
    res["read_GB/s"] = max(res["read_GB/s"], sweep[best])
    del x, y
    torch.cuda.empty_cache()
    log(f"stream peak: {res}")
    return res


def run_configs(M, torch, steps: int = 32, names=("tiny", "gqa8k", "append32k", "ragged64k")):
    """The other workloads, one step each as on the 128K line: select + decode (the
    tiny G = 1 case, GQA 32/8 at 8K, the ragged batch of 16 with G = 8) or the fused
    append-1 + select, then decode (the 32K append loop, 64 steps).  Queries follow
    each workload's recipe; the prefill K/V are drawn on the GPU from the same
    distributions (timing does not depend on their values).  Cache copies rotate so
    that at least 512 MB is streamed between visits to one copy.  Each is timed as a
    captured HIP graph of its steps, replayed once untimed and once timed."""
    dev = "cuda"
    res = {}
    for name in names:
        t0 = time.time()
        wl = W.workload(name)
        appends = wl.steps > 0
        n = wl.steps if appends else steps
        keep = M.keep_for_sparsity(wl.d, wl.sparsity[0])
        sm = W.default_sm_scale(wl.d)
        # room for the eager warmup step and the two replays' appends
        cap = W._cap_for(max(wl.ctx) + (2 * n + 8 if appends else 0))
        cap = (cap + 63) // 64 * 64
        a, b = W.transforms(wl)
        a_d, b_d = torch.from_numpy(a).to(dev), torch.from_numpy(b).to(dev)
        kscale = torch.from_numpy(W.key_scales(wl)).to(dev)
        fdt = torch.float32 if wl.dtype == "f32" else torch.bfloat16
        gen = torch.Generator(device=dev)
        gen.manual_seed(1000 + wl.cid)
        ctx_np = np.array(wl.ctx, dtype=np.int64)
        cache0 = M.Cache(wl.batch, wl.hkv, wl.d, cap)
        chunk = min(8192, cap)
        for pos in range(0, int(ctx_np.max()), chunk):   # bounded staging memory
            nn = np.clip(ctx_np - pos, 0, chunk)
            k = torch.randn((wl.batch, wl.hkv, chunk, wl.d), generator=gen, device=dev)
            k *= kscale[None, :, None, :]
            v = torch.randn((wl.batch, wl.hkv, chunk, wl.d), generator=gen, device=dev)
            v[..., 0] *= 8.0
            M.transform_quantize_append(cache0, k.to(fdt), v.to(fdt), b_d,
                                        torch.from_numpy(nn.astype(np.int32)).to(dev))
            del k, v
        torch.cuda.synchronize()
        ncopy = int(min(16, max(1, -(-512_000_000 // cache0.nbytes()))))
        caches = [cache0] + [M.Cache(wl.batch, wl.hkv, wl.d, cap) for _ in range(ncopy - 1)]
        for c in caches[1:]:
            for pname, t in cache0.planes().items():
                getattr(c, pname).copy_(t)
        qs = torch.stack([torch.from_numpy(W.queries(wl, i)).to(dev).to(fdt)
                          for i in range(n + 1)])
        kv = torch.randn((n + 1, wl.batch, wl.hkv, 1, wl.d), generator=gen, device=dev).to(fdt)
        ones = torch.ones((wl.batch,), dtype=torch.int32, device=dev)
        qp = torch.empty((wl.batch, wl.hq, wl.d), dtype=torch.float32, device=dev)
        idx = torch.empty((wl.batch, wl.hq, keep), dtype=torch.int32, device=dev)
        out = torch.empty((wl.batch, wl.hq, wl.d), dtype=torch.float32, device=dev)
        ws = torch.empty(M.decode_workspace_bytes(cache0, wl.hq), dtype=torch.uint8, device=dev)

        # algorithmic bytes of the timed replay (steps 1..n), lengths as they will be
        lengths = [np.array(wl.ctx, dtype=np.int64) for _ in caches]
        inb = 4 if wl.dtype == "f32" else 2

        def advance(i):
            ci = i % len(caches)
            M.select_channels(qs[i], a_d, wl.hkv, keep, qp, idx)
            nb = select_bytes(wl.batch, wl.hq, wl.hkv, wl.d, keep, inb)
            if appends:
                nb += append_bytes(wl.batch, wl.hkv, wl.d, lengths[ci], inb)
                lengths[ci] = lengths[ci] + 1
            db = decode_bytes(idx.cpu().numpy(), lengths[ci], wl.hkv, wl.d, keep)
            return nb + db, db

        def step(i):
            c = caches[i % len(caches)]
            if appends:
                M.append_select(c, kv[i], kv[i], b_d, ones, qs[i], a_d, keep, qp, idx)
            else:
                M.select_channels(qs[i], a_d, wl.hkv, keep, qp, idx)
            M.decode_attention(c, qp, idx, sm, 0, out, ws)

        step(0)                                   # eager warmup (appends to copy 0)
        torch.cuda.synchronize()
        if appends:
            lengths[0] = lengths[0] + 1
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(1, n + 1):
                step(i)
        graph.replay()                            # untimed replay
        torch.cuda.synchronize()
        for i in range(1, n + 1):                 # lengths after the untimed replay
            if appends:
                lengths[i % len(caches)] = lengths[i % len(caches)] + 1
        per = [advance(i) for i in range(1, n + 1)]
        tot, dec_tot = sum(x[0] for x in per), sum(x[1] for x in per)
        torch.cuda.synchronize()
        ts = time.perf_counter()
        graph.replay()
        torch.cuda.synchronize()
        wall = time.perf_counter() - ts
        us = 1e6 * wall / n
        res[name] = {"us_per_step": round(us, 2), "GB/s": round(tot / wall / 1e9, 1),
                     "tokens_per_s": round(wl.batch / (us * 1e-6), 1),
                     "bytes_per_step": int(tot / n), "decode_bytes_per_step": int(dec_tot / n),
                     "steps": n, "cache_copies": len(caches),
                     "step": ("append 1 + select + decode" if appends else "select + decode"),
                     "workload": wl.describe()}
        log(f"{name}: {us:.1f} us/step, {tot / wall / 1e9:.0f} GB/s "
            f"({len(caches)} copies, setup {time.time() - t0:.1f}s)")
        del graph, caches, cache0, qs, kv, ws
        torch.cuda.empty_cache()
    return res

if __name__ == "__main__":
    main()
