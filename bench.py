#!/usr/bin/env python3
"""Benchmark of the QVG KV-cache compress/decompress hot path on one MI355X.

Default workload: a Self-Forcing-Wan-1.3B-shaped cache, 12 K + 12 V heads of
32760 tokens (21 latent frames x 30x52 patches), d=128, bf16; k-means C=256,
8 iterations, T=2 stages, INT2 with G=64 and E4M3 scales.  One step = one
compress of all 24 head-tensors followed by one fused decompress of the
record (every step of the hot path), inputs resident in HBM.

Prints one JSON line: throughput (head-tensor token rows per second through
the whole step), the dominant kernel's roofline from HIP events recorded on
its launch stream, and the CPU oracle's throughput on a bounded sample of the
same workload (run on this host's cores), with a bit-exact parity check of
that sample.

Other workloads (--workload): decode (decode-side dequant of a 40 x 262144
token, T=4 record), stream (20 chunks of 3 frames, warm-started against cold
k-means, per-chunk time and MSE, and the whole history reconstructed from
its 20 chunk records in one pass), large (32 K + 32 V head-tensors x 131072
tokens, T=4, INT2 and INT4, per-stage MSE curve and record sizes), pro (the
self-forcing-shaped cache at the QVG-Pro operating point, T=4 and groups of
16, chosen per tensor kind), attn (attention of --nq queries per head over the
decode-side K and V records with the rotary tables, keys and values rebuilt
on chip, against an unfused consumer: the keys decompressed to bf16 and the
values to fp32 (the unrounded reconstruction the fused kernel uses), then
rotary keys and the attention in torch).
--copy-calibration runs only a plain 256 MiB device copy,
the reference that the HBM byte counters of the kernels are scaled by.

The `traffic` field of a roofline is the kernel's measured HBM bytes per
launch, read from profiles/<kernel>_<workload>_pmc.txt, and null when the
kernel's sources have changed since those counters were taken.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from means_residual_compression_amd import qvg, synth  # noqa: E402

METRIC = "compress tokens/s and fused-dequant GB/s (% of HBM roofline), d=128 C=256 T=2"
HBM_PEAK_GBPS = 8000.0      # MI355X HBM3E
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16/bf16 MFMA


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# Sources whose text determines each timed kernel's code.
CSRC = os.path.join(ROOT, "means_residual_compression_amd", "csrc")
KERNEL_SOURCES = {
    "kmeans_assign": ["qvg_kmeans.hip", "qvg_common.h", "qvg_internal.h"],
    "fused_dequant": ["qvg_quant.hip", "qvg_common.h", "qvg_internal.h"],
    "attention": ["qvg_attn.hip", "qvg_attn.h", "qvg_common.h", "qvg_internal.h"],
}
COPY_BYTES = 256 << 20


def source_digest(kernel):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def stored_traffic(kernel, workload):
    """HBM bytes per launch from the committed counter summary, or None when
    there is none or the kernel's sources changed after it was taken."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_pmc.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as fh:
        for line in fh:
            parts = line.split()
            if len(parts) == 2 and not line.startswith("#"):
                vals[parts[0]] = parts[1]
    if vals.get("source_sha256") != source_digest(kernel) or "hbm_bytes_per_launch" not in vals:
        return None
    return float(vals["hbm_bytes_per_launch"])


def copy_calibration():
    """A plain device copy of known size (read COPY_BYTES, write COPY_BYTES),
    run a few times: the reference for scaling FETCH_SIZE / WRITE_SIZE."""
    dev = torch.device("cuda:0")
    a = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    for _ in range(5):
        torch.mul(a, 1.0, out=b)  # an elementwise kernel: reads a once, writes b once
    torch.cuda.synchronize()
    return {"copy_bytes": COPY_BYTES, "launches": 5}


# ------------------------------------------------------------------ helpers
def kernel_times(names):
    out = {}
    for k in names:
        ms, n = qvg.timing_read(k)
        if n:
            out[k] = {"total_ms": ms, "launches": n, "avg_ms": ms / n}
    return out


def dequant_bytes(H, N, d, C, T, bits, G, out_bytes=2, c_bytes=2):
    """Algorithmic HBM bytes of one fused dequant launch: read codes, scales
    and T assignment bytes per token and each stage's centroid table once,
    write the reconstructed row."""
    per_tok = d * bits // 8 + d // G + T + d * out_bytes
    return H * N * per_tok + H * T * C * d * c_bytes


def cpu_model():
    """The host CPU's model name (for the baseline's record)."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _event_ms(fn, reps):
    """Average milliseconds of `reps` calls of fn between two events on the
    current stream (for torch's own fill and copy kernels)."""
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    fn()
    e0.record(s)
    for _ in range(reps):
        fn()
    e1.record(s)
    e1.synchronize()
    return e0.elapsed_time(e1) / reps


def decode_leg(reps=100):
    """The decode-side read path at its full size: a video-shaped cache of 20 K
    + 20 V head-tensors x 262144 tokens (39x40 grid, scene cut every 21 frames,
    drawn on the device) compressed on the GPU at T=4, C=256, INT2 G=64, 8
    iterations; then the fused dequant of that record, `reps` launches, against
    HBM's peak, with the measured fill and copy rates of the same output buffer
    beside it."""
    dev = torch.device("cuda:0")
    c = synth.CONFIGS["long_video"]
    N, d, hk = 262144, 128, 20
    log("drawing the decode-side cache on the device and compressing it ...")
    x = torch.cat([synth.video_cache_device(4, k, hk, c["Hg"], c["Wg"], d, synth.OUTLIER_SCALE[k],
                                            N, c["scene_len"], torch.bfloat16, dev)
                   for k in c["kinds"]])
    H = x.shape[0]
    p = qvg.params(C=256, T=4, iters=8, bits=2, group=64, seed=4)
    rec = qvg.compress(x, p)
    out = torch.empty_like(x)
    for _ in range(3):
        qvg.decompress(rec, p, out=out)
    torch.cuda.synchronize()
    qvg.timing_reset()
    qvg.timing_enable(True)
    for _ in range(reps):
        qvg.decompress(rec, p, out=out)
    torch.cuda.synchronize()
    qvg.timing_enable(False)
    ms, n = qvg.timing_read("fused_dequant")
    avg = ms / n
    nbytes = dequant_bytes(H, N, d, p.C, p.T, p.bits, p.group)
    gbps = nbytes / (avg * 1e-3) / 1e9
    out_bytes = out.numel() * out.element_size()
    fill_ms = _event_ms(lambda: out.fill_(1.0), 20)
    copy_ms = _event_ms(lambda: out.copy_(x), 20)
    res = {"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
           "frac": gbps / HBM_PEAK_GBPS, "traffic": stored_traffic("fused_dequant", "decode"),
           "kernel": "fused_dequant", "per_launch": f"{nbytes} B", "avg_ms": avg,
           "launches": n,
           "workload": "record from GPU compress of a video-shaped cache, 20 K + 20 V "
                       "head-tensors x 262144 tokens, d=128, T=4, C=256, INT2 G=64",
           "measured_ceilings_GBps": {"fill (write only, same buffer)": out_bytes / (fill_ms * 1e-3) / 1e9,
                                      "copy (read + write)": 2 * out_bytes / (copy_ms * 1e-3) / 1e9}}
    del x, rec, out
    torch.cuda.empty_cache()
    return res


def timed(step, steps, warmup):
    """Wall time per step of `steps` steps after `warmup` untimed ones, with
    no per-kernel events inside the timed region (each event pair costs a
    few microseconds of GPU time), followed by a second pass of `steps`
    steps with HIP events recorded around every library launch on its
    stream, which gives the per-kernel durations (kernel_times)."""
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    qvg.timing_reset()
    qvg.timing_enable(True)
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    qvg.timing_enable(False)
    return (t1 - t0) * 1e3 / steps


def cpu_baseline_selfforcing(x_cpu, p, idx, rec_gpu, heads):
    """Oracle compress + decompress of `heads` head-tensors (all tokens, all
    iterations) on the host's cores; also checks the GPU record of those
    head-tensors bit for bit."""
    import oracle
    ncores = len(os.sched_getaffinity(0))
    sel = list(range(0, x_cpu.shape[0], max(1, x_cpu.shape[0] // heads)))[:heads]
    xs = x_cpu[sel].contiguous()
    xb = xs.view(torch.int16).numpy().view(np.uint16)
    threads = min(ncores, len(sel))
    t0 = time.perf_counter()
    ref = oracle.compress(xb, C=p.C, T=p.T, iters=p.iters, bits=p.bits, G=p.group,
                          init_idx=idx[sel], threads=threads)
    ref_out = oracle.decompress(ref["codes"], ref["scales"], ref["assign"], ref["cent"], p.bits,
                                p.group, threads=threads)
    dt = time.perf_counter() - t0
    parity = all(np.array_equal(getattr(rec_gpu, f)[sel].cpu().numpy(), ref[k])
                 for f, k in (("codes", "codes"), ("scales", "scales"), ("assign", "assign")))
    parity = parity and np.array_equal(
        rec_gpu.centroids[sel].cpu().view(torch.int16).numpy().view(np.uint16), ref["cent"])
    tokens = len(sel) * xs.shape[1]
    return {"value": tokens / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{len(sel)} of {x_cpu.shape[0]} head-tensors, all {xs.shape[1]} tokens, "
                      f"all {p.T}x{p.iters} k-means iterations, compress + decompress "
                      f"({dt:.1f} s wall, {ncores} host cores visible)"}, parity, ref_out, sel


# --------------------------------------------------------------- workloads
def concurrent_calls(parts, steps, warmup):
    """Wall time per step when independent compress + decompress calls run on
    streams of their own (default priority), one per part (x, params,
    init_idx, workspace, record, output); the current stream waits for all."""
    dev = torch.device("cuda:0")
    sts = [torch.cuda.Stream(dev) for _ in parts]

    def step():
        cur = torch.cuda.current_stream(dev)
        for st, (x, p, idx, ws, rec, out) in zip(sts, parts):
            st.wait_stream(cur)
            with torch.cuda.stream(st):
                qvg.compress(x, p, init_idx=idx, ws=ws, out=rec)
                qvg.decompress(rec, p, out=out)
        for st in sts:
            cur.wait_stream(st)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


def run_selfforcing(args):
    dev = torch.device("cuda:0")
    c = synth.CONFIGS["self_forcing"]
    log("generating the self-forcing-shaped cache ...")
    x_cpu = synth.config_cache("self_forcing")
    H, N, d = x_cpu.shape
    p = qvg.params(C=c["C"], T=c["T"], iters=c["iters"], bits=c["bits"], group=c["group"])
    idx = synth.init_indices(1, H, p.T, N, p.C)
    idx_pinned = torch.from_numpy(idx).pin_memory()
    x = x_cpu.to(dev)
    ws = qvg.alloc_workspace(qvg.workspace_size(H, N, d, x.dtype, p), dev)
    rec = qvg.empty_record(H, N, d, p, x.dtype, dev)
    out = torch.empty_like(x)

    def step():
        qvg.compress(x, p, init_idx=idx_pinned, ws=ws, out=rec)
        qvg.decompress(rec, p, out=out)

    ms = timed(step, args.steps, args.warmup)
    kt = kernel_times(qvg.KERNELS)
    log(json.dumps(kt, indent=1))
    tokens = H * N
    compress_ms = sum(v["total_ms"] for k, v in kt.items() if k != "fused_dequant") / args.steps
    dq = kt["fused_dequant"]
    dq_bytes = dequant_bytes(H, N, d, p.C, p.T, p.bits, p.group)
    dq_gbps = dq_bytes / (dq["avg_ms"] * 1e-3) / 1e9
    asg = kt["kmeans_assign"]
    asg_flops = 2.0 * H * N * p.C * d
    asg_tflops = asg_flops / (asg["avg_ms"] * 1e-3) / 1e12
    dominant = max(kt, key=lambda k: kt[k]["total_ms"])
    rooflines = {
        "kmeans_assign": {"bound": "mfma", "achieved": asg_tflops, "peak": MFMA_F16_PEAK_TFLOPS,
                          "unit": "TFLOP/s", "frac": asg_tflops / MFMA_F16_PEAK_TFLOPS,
                          "traffic": stored_traffic("kmeans_assign", "selfforcing"),
                          "kernel": "kmeans_assign",
                          "per_launch": f"{asg_flops:.4g} flop (2*N*C*d over {H} head-tensors)",
                          "avg_ms": asg["avg_ms"]},
        "fused_dequant": {"bound": "hbm", "achieved": dq_gbps, "peak": HBM_PEAK_GBPS,
                          "unit": "GB/s", "frac": dq_gbps / HBM_PEAK_GBPS,
                          "traffic": stored_traffic("fused_dequant", "selfforcing"),
                          "kernel": "fused_dequant",
                          "per_launch": f"{dq_bytes} B", "avg_ms": dq["avg_ms"]},
    }
    # the other hot-path kernels against HBM: algorithmic bytes per launch
    # (bf16 input x: 2 B per element; stage t also reads t assignment bytes
    # per token; averages over the T stages where launches differ by stage)
    hbm_bytes = {
        # one read of the stage residual's sources per full update (the first
        # iteration of a stage; later ones move only the changed tokens and
        # are timed as kmeans_delta)
        "kmeans_accumulate": H * N * (2 * d + (p.T - 1) / 2),
        # x and every stage's assignment in; codes and scales out
        "group_quant_pack": H * N * (2 * d + p.T + d * p.bits / 8 + d / p.group),
        # x (+ assignments) in; fp16 fragments and per-token bounds out
        "kmeans_prepare": H * N * (4 * d + 8 + (p.T - 1) / 2),
        "absmax": H * N * 2 * d,
    }
    for k, nb in hbm_bytes.items():
        if k in kt:
            gb = nb / (kt[k]["avg_ms"] * 1e-3) / 1e9
            rooflines[k] = {"bound": "hbm", "achieved": gb, "peak": HBM_PEAK_GBPS,
                            "unit": "GB/s", "frac": gb / HBM_PEAK_GBPS, "traffic": None,
                            "kernel": k, "per_launch": f"{nb:.0f} B",
                            "avg_ms": kt[k]["avg_ms"]}
    if dominant not in rooflines:
        dominant = "kmeans_assign"
    res = {
        "metric": METRIC,
        "value": tokens / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16",
        "arith": "bf16 in/out; fp16 MFMA distance keys, fp64 exact distances and means, "
                 "fp32 residuals and quantization",
        "video_tokens_per_s": N / (ms * 1e-3),
        "data": "synthetic",
        "config": {"workload": "self-forcing-wan-1.3b-shaped KV cache: 12 K + 12 V head-tensors "
                               "x 32760 tokens (21 frames x 30x52), d=128, bf16",
                   "head_tensors": H, "tokens": N, "d": d, "C": p.C, "T": p.T,
                   "iters": p.iters, "bits": p.bits, "group": p.group,
                   "step": "compress (all head-tensors) + fused decompress"},
        "roofline": rooflines[dominant],
        "roofline_other": {k: v for k, v in rooflines.items() if k != dominant},
        "compress_ms": compress_ms,
        "compress_tokens_per_s": tokens / (compress_ms * 1e-3),
        "dequant_ms": dq["avg_ms"],
        "dequant_GBps": dq_gbps,
        "dequant_hbm_frac": dq_gbps / HBM_PEAK_GBPS,
        "kernels_avg_ms": {k: round(v["avg_ms"], 5) for k, v in kt.items()},
        "kernels_launches_per_step": {k: v["launches"] // args.steps for k, v in kt.items()},
        "record_bytes_per_head_tensor": rec.nbytes() // H,
    }
    if not args.no_decode_leg:
        res["roofline_other"]["fused_dequant_decode"] = decode_leg()
    if not args.no_cpu_baseline:
        log("oracle baseline on the host cores ...")
        cb, parity, _, _ = cpu_baseline_selfforcing(x_cpu, p, idx, rec,
                                                    args.cpu_heads or min(
                                                        len(os.sched_getaffinity(0)), H))
        res["cpu_baseline"] = cb
        res["parity_sample_bit_exact"] = bool(parity)
    else:
        res["cpu_baseline"] = None
    return res


def run_decode(args):
    """Decode-side: fused dequant of a 40 x 262144 token, d=128, T=4, C=256,
    INT2 G=64 record with bf16 centroids, repeated."""
    dev = torch.device("cuda:0")
    H, N, d, T, C, bits, G = 40, 262144, 128, 4, 256, 2, 64
    log("drawing the decode-side record ...")
    codes, scales, assign, cent = synth.random_record(4, H, N, d, T, C, bits, G)
    rec = qvg.Record(torch.from_numpy(codes).to(dev), torch.from_numpy(scales).to(dev),
                     torch.from_numpy(assign).to(dev), cent.to(dev))
    p = qvg.params(C=C, T=T, iters=1, bits=bits, group=G)
    out = torch.empty((H, N, d), dtype=torch.bfloat16, device=dev)
    ms = timed(lambda: qvg.decompress(rec, p, out=out), args.steps, args.warmup)
    kt = kernel_times(["fused_dequant"])
    dq = kt["fused_dequant"]
    nbytes = dequant_bytes(H, N, d, C, T, bits, G)
    gbps = nbytes / (dq["avg_ms"] * 1e-3) / 1e9
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        ncores = len(os.sched_getaffinity(0))
        sel = list(range(min(16, H, ncores)))
        cb = cent.view(torch.int16).numpy().view(np.uint16)
        t0 = time.perf_counter()
        oracle.decompress(codes[sel], scales[sel], assign[sel], cb[sel], bits, G, out_bf16=True,
                          threads=len(sel))
        dt = time.perf_counter() - t0
        cpu = {"value": dequant_bytes(len(sel), N, d, C, T, bits, G) / dt / 1e9, "unit": "GB/s",
               "cores": len(sel), "kind": "oracle", "cpu_model": cpu_model(),
               "sample": f"{len(sel)} of {H} head-tensors, all {N} tokens, decompress "
                         f"({dt:.2f} s wall, {ncores} host cores visible)"}
    return {"metric": "fused-dequant GB/s (decode-side record, d=128 C=256 T=4)",
            "value": gbps, "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": "decode-side record 40 heads x 262144 tokens, d=128, INT2 "
                                   "G=64, T=4, C=256, bf16 centroids and output"},
            "roofline": {"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS,
                         "unit": "GB/s", "frac": gbps / HBM_PEAK_GBPS,
                         "traffic": stored_traffic("fused_dequant", "decode"),
                         "kernel": "fused_dequant", "per_launch": f"{nbytes} B",
                         "avg_ms": dq["avg_ms"]},
            "cpu_baseline": cpu}


def run_attn(args):
    """Attention of Nq queries per head over the decode-side K and V records
    (40 x 262144 tokens each, d=128, T=4, C=256, INT2 G=64, bf16 centroids),
    pre-rotary keys rotated after reconstruction, with the keys and values
    rebuilt on chip; against it, the unfused consumer (keys decompressed to bf16,
    values to fp32, keys rotated and the attention evaluated with torch)."""
    dev = torch.device("cuda:0")
    H, N, d, T, C, bits, G, Nq = 40, 262144, 128, 4, 256, 2, 64, args.nq
    recs, host0 = [], []
    for seed in (4, 104):
        log(f"drawing the decode-side record (seed {seed}) ...")
        codes, scales, assign, cent = synth.random_record(seed, H, N, d, T, C, bits, G)
        recs.append(qvg.Record(torch.from_numpy(codes).to(dev), torch.from_numpy(scales).to(dev),
                               torch.from_numpy(assign).to(dev), cent.to(dev)))
        host0.append((codes[:1].copy(), scales[:1].copy(), assign[:1].copy(),
                      cent[:1].view(torch.int16).numpy().view(np.uint16).copy()))
        del codes, scales, assign
    p = qvg.params(C=C, T=T, iters=1, bits=bits, group=G)
    cos, sin = (t.to(dev) for t in synth.rope_tables(N, d))
    q = synth.queries(9, H, Nq, d).to(dev)
    scale = float(np.float32(1.0 / np.sqrt(d)))
    ws = qvg.alloc_workspace(qvg.attention_workspace_size(H, Nq, N, d, p), dev)
    out = torch.empty((H, Nq, d), dtype=torch.float32, device=dev)
    step = lambda: qvg.attention(q, recs[0], p, recs[1], p, scale, rope=(cos, sin), ws=ws,
                                 out=out)
    ms = timed(step, args.steps, args.warmup)
    at = kernel_times(["attention"])["attention"]
    # algorithmic bytes: per token and head the codes, scales and T assignment
    # bytes of K and of V; each stage's centroid table of both; the rotary
    # tables, queries and output once
    per_tok = 2 * (d * bits // 8 + d // G + T)
    nbytes = H * N * per_tok + 2 * H * T * C * d * 2 + 2 * N * (d // 2) * 4 + 2 * H * Nq * d * 4
    gbps = nbytes / (at["avg_ms"] * 1e-3) / 1e9
    # the unfused consumer: the records decompressed (keys bf16, values fp32),
    # the keys rotated and the attention evaluated with torch (bf16 score
    # products, fp32 softmax and value products), every intermediate in HBM
    kd = torch.empty((H, N, d), dtype=torch.bfloat16, device=dev)
    # values as the fused kernel takes them: the reconstruction unrounded
    # (fp32), so both consumers compute the same attention
    vd = torch.empty((H, N, d), dtype=torch.float32, device=dev)
    qT = q.transpose(1, 2).contiguous().to(torch.bfloat16)  # [H, d, Nq]
    cosf, sinf = cos[None], sin[None]

    def unfused():
        qvg.decompress(recs[0], p, out=kd)
        qvg.decompress(recs[1], p, out_dtype=torch.float32, out=vd)
        x1, x2 = kd[..., : d // 2].float(), kd[..., d // 2:].float()
        kr = torch.cat((x1 * cosf - x2 * sinf, x2 * cosf + x1 * sinf), -1).to(torch.bfloat16)
        s = torch.bmm(kr, qT).float() * scale                       # [H, N, Nq]
        w = torch.softmax(s, dim=1).transpose(1, 2).contiguous()    # [H, Nq, N]
        return torch.bmm(w, vd)                                     # fp32

    ms_unfused = timed(unfused, max(3, args.steps // 2), 1)
    dq = kernel_times(["fused_dequant"])["fused_dequant"]
    cpu = None
    if not args.no_cpu_baseline:
        # the oracle's attention of head-tensor 0: keys decompressed (bf16) and
        # rotated, values reconstructed unrounded, softmax and products in fp64
        import oracle
        (kc, ks, ka, kcent), (vc, vs, va, vcent) = host0
        q0 = q[:1].cpu().numpy()
        rope = (cos.cpu().numpy(), sin.cpu().numpy())
        t0 = time.perf_counter()
        kb = oracle.decompress(kc, ks, ka, kcent, bits, G, out_bf16=True, threads=1)
        vx = oracle.reconstruct_exact(vc, vs, va, vcent, bits, G)
        oracle.attention(q0, kb, vx, scale, rope)
        dt = time.perf_counter() - t0
        cpu = {"value": (nbytes / H) / dt / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle", "cpu_model": cpu_model(),
               "sample": f"head-tensor 0 of {H}, all {N} tokens, {Nq} queries "
                         f"({dt:.2f} s wall, one thread; numpy fp64)"}
    return {"metric": "fused dequant-attention GB/s (decode-side K and V records, d=128 "
                      "C=256 T=4)",
            "value": gbps, "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": f"attention of {Nq} queries per head over decode-side K "
                                   f"and V records, 40 heads x 262144 tokens, d=128, INT2 "
                                   f"G=64, T=4, C=256, bf16 centroids, rotary keys"},
            "roofline": {"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS,
                         "unit": "GB/s", "frac": gbps / HBM_PEAK_GBPS,
                         "traffic": stored_traffic("attention", "attn") if Nq == 1 else None,
                         "kernel": "attention", "per_launch": f"{nbytes} B",
                         "avg_ms": at["avg_ms"]},
            "unfused": {"decompress_k_and_v_ms": 2 * dq["avg_ms"],
                        "total_ms": ms_unfused,
                        "fused_attention_ms": at["avg_ms"],
                        "bf16_kv_bytes_avoided": 2 * H * N * d * 2 * 2},
            "cpu_baseline": cpu}


def _mse(x, y):
    """Mean squared error per head-tensor in fp64 (measurement only)."""
    return ((x.double() - y.double()) ** 2).mean(dim=(1, 2))


def _events_ms(fn):
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    r = fn()
    e1.record(s)
    e1.synchronize()
    return e0.elapsed_time(e1), r


def cpu_baseline_stream(chunks_cpu, p, idx0, iters_warm):
    """The oracle on the host's cores: chunk 0 cold (untimed, for its cache),
    then the given warm chunks, each warm-started from the previous chunk's
    fp32 centroids, timed."""
    import oracle
    ncores = len(os.sched_getaffinity(0))
    H, N = chunks_cpu[0].shape[:2]
    threads = min(ncores, H)

    def host(x):
        return x.view(torch.int16).numpy().view(np.uint16) if x.dtype == torch.bfloat16 \
            else x.numpy()
    ref = oracle.compress(host(chunks_cpu[0]), C=p.C, T=p.T, iters=p.iters, bits=p.bits,
                          G=p.group, init_idx=idx0, threads=threads)
    cache = ref["cache"]
    t0 = time.perf_counter()
    for x in chunks_cpu[1:]:
        ref = oracle.compress(host(x), C=p.C, T=p.T, iters=iters_warm, bits=p.bits, G=p.group,
                              init_c=cache, threads=threads)
        cache = ref["cache"]
    dt = time.perf_counter() - t0
    nw = len(chunks_cpu) - 1
    return {"value": nw * H * N / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"warm chunks 1-{nw} of the stream, all {H} head-tensors x {N} tokens, "
                      f"{iters_warm} iterations per stage from the previous chunk's cache, after "
                      f"chunk 0 cold (untimed); {dt:.1f} s wall, {ncores} host cores visible"}


def run_stream(args):
    """A 60-frame stream in 20 chunks of 3 frames (4680 tokens) of 12 K + 12 V
    head-tensors: cold chunks (10 iterations from seeded rows) against warm
    chunks (3 iterations from the previous chunk's fp32 centroids)."""
    dev = torch.device("cuda:0")
    c = synth.CONFIGS["stream"]
    log("generating the stream chunks ...")
    chunks, chunks_cpu = [], []
    for ci in range(c["chunks"]):
        parts = [synth.stream_chunk(2, k, c["heads"], ci, c["F"], c["Hg"], c["Wg"], c["d"],
                                    c["outlier"][k], c["dtype"]) for k in c["kinds"]]
        xc = torch.cat(parts, 0)
        if ci < 5:  # the host baseline's sample
            chunks_cpu.append(xc)
        chunks.append(xc.to(dev))
    H, N, d = chunks[0].shape
    p = qvg.params(C=c["C"], T=c["T"], iters=c["iters"], bits=c["bits"], group=c["group"])
    ws = qvg.alloc_workspace(qvg.workspace_size(H, N, d, chunks[0].dtype, p), dev)
    rec = qvg.empty_record(H, N, d, p, chunks[0].dtype, dev)
    out = torch.empty_like(chunks[0])
    cache = torch.zeros((H, p.T, p.C, d), dtype=torch.float32, device=dev)
    idx = [torch.from_numpy(synth.init_indices(2000 + ci, H, p.T, N, p.C)).pin_memory()
           for ci in range(c["chunks"])]
    res_modes = {}
    for mode in ("cold", "warm"):
        for _ in range(args.warmup):  # warm-up passes over the first chunks
            qvg.compress(chunks[0], p, init_idx=idx[0], ws=ws, out=rec, cache_out=cache)
        torch.cuda.synchronize()
        times, mses = [], []
        for ci, x in enumerate(chunks):
            if mode == "cold" or ci == 0:
                ms, _ = _events_ms(lambda: qvg.compress(x, p, init_idx=idx[ci], ws=ws, out=rec,
                                                        cache_out=cache))
            else:
                ms, _ = _events_ms(lambda: qvg.compress_stream(x, p, c["iters_warm"], cache, True,
                                                               ws=ws, out=rec))
            qvg.decompress(rec, p, out=out)
            times.append(ms)
            mses.append(_mse(out, x).mean().item())
        res_modes[mode] = {"ms_per_chunk": times, "mse_per_chunk": mses,
                           "total_ms": sum(times),
                           "tokens_per_s": H * N * len(chunks) / (sum(times) * 1e-3)}
    warm, cold = res_modes["warm"], res_modes["cold"]
    eager_cache = cache.clone()  # after the eager warm chain
    # the warm chain again with each chunk's compress replayed from a HIP graph
    # captured once per chunk (same buffers): launches without host gaps
    graphs = []
    for x in chunks[1:]:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            qvg.compress_stream(x, p, c["iters_warm"], cache, True, ws=ws, out=rec)
        graphs.append(g)
    for timed_pass in (False, True):  # the first pass uploads the graphs
        qvg.compress(chunks[0], p, init_idx=idx[0], ws=ws, out=rec, cache_out=cache)
        torch.cuda.synchronize()
        gtimes = [_events_ms(g.replay)[0] for g in graphs]
        torch.cuda.synchronize()
    graph_res = {"ms_per_warm_chunk": gtimes,
                 "tokens_per_s": H * N * len(gtimes) / (sum(gtimes) * 1e-3),
                 "final_cache_equals_eager_chain": bool(torch.equal(cache, eager_cache)),
                 "speedup_vs_eager_warm": (sum(warm["ms_per_chunk"][1:]) / sum(gtimes))}
    del graphs
    # the whole history through the compressed-cache container: warm records of
    # all chunks kept, then reconstructed in one pass against one decompress
    # call per chunk
    kv = qvg.CompressedKVCache(p, c["iters_warm"])
    for ci, x in enumerate(chunks):
        kv.append(x, init_idx=idx[0] if ci == 0 else None)
    hist = torch.empty((H, kv.n_tokens(), d), dtype=chunks[0].dtype, device=dev)
    per = [torch.empty_like(chunks[0]) for _ in chunks]
    for _ in range(max(1, args.warmup)):
        kv.reconstruct(out=hist)
    hms = min(_events_ms(lambda: kv.reconstruct(out=hist))[0] for _ in range(5))
    sms = min(_events_ms(lambda: [qvg.decompress(r, p, out=o) for r, o in zip(kv.records, per)])[0]
              for _ in range(5))
    hbytes = sum(dequant_bytes(H, r.codes.shape[1], d, p.C, p.T, p.bits, p.group)
                 for r in kv.records)
    history = {"chunks": len(kv), "tokens_per_head": kv.n_tokens(),
               "record_bytes": kv.nbytes(), "bf16_bytes": H * kv.n_tokens() * d * 2,
               "reconstruct_ms": hms, "reconstruct_GBps": hbytes / (hms * 1e-3) / 1e9,
               "reconstruct_hbm_frac": hbytes / (hms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
               "per_chunk_decompress_ms": sms}
    del kv, hist, per
    # per-kernel durations over one more warm pass (HIP events around every
    # launch); the roofline is the k-means assign's, the dominant kernel
    qvg.timing_reset()
    qvg.timing_enable(True)
    for x in chunks[1:]:
        qvg.compress_stream(x, p, c["iters_warm"], cache, True, ws=ws, out=rec)
    torch.cuda.synchronize()
    qvg.timing_enable(False)
    kt = kernel_times(qvg.KERNELS)
    asg = kt["kmeans_assign"]
    asg_flops = 2.0 * H * N * p.C * d
    asg_tflops = asg_flops / (asg["avg_ms"] * 1e-3) / 1e12
    roofline = {"bound": "mfma", "achieved": asg_tflops, "peak": MFMA_F16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": asg_tflops / MFMA_F16_PEAK_TFLOPS, "traffic": None,
                "kernel": "kmeans_assign",
                "per_launch": f"{asg_flops:.4g} flop (2*N*C*d over {H} head-tensors)",
                "avg_ms": asg["avg_ms"]}
    cb = None
    if not args.no_cpu_baseline:
        log("oracle baseline on the host cores ...")
        cb = cpu_baseline_stream(chunks_cpu, p, synth.init_indices(2000, H, p.T, N, p.C),
                                 c["iters_warm"])
    return {"metric": "streamed compress tokens/s (warm-started chunks)",
            "value": warm["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
            "steps": len(chunks), "warmup": args.warmup,
            "ms_per_step": warm["total_ms"] / len(chunks), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": "stream of 20 chunks x 3 frames (4680 tokens), 12 K + 12 V "
                                   "head-tensors, d=128, bf16, C=256, T=2, INT2 G=64; warm: 3 "
                                   "iterations from the cache, cold: 10 from seeded rows"},
            "warm": warm, "cold": cold, "warm_graph": graph_res, "history": history,
            "warm_speedup": cold["total_ms"] / warm["total_ms"],
            "mse_ratio_warm_over_cold": float(np.mean(warm["mse_per_chunk"][1:]) /
                                              np.mean(cold["mse_per_chunk"][1:])),
            "roofline": roofline, "kernels_avg_ms": {k: round(v["avg_ms"], 5) for k, v in kt.items()},
            "cpu_baseline": cb}


def run_pro(args):
    """The self-forcing-shaped cache at the QVG-Pro operating point, chosen per
    tensor kind (K and V head-tensors go through separate calls, each with its
    own parameters): T=4 stages, INT2, groups of 16 channels, C=256, 8
    iterations.  One step = compress K + compress V + fused decompress of both
    records.  Also reports the record sizes and compression ratio against bf16,
    the per-kind MSE beside the QVG operating point's (T=1, G=64), and an
    oracle check of one K and one V head-tensor, bit for bit."""
    import oracle
    dev = torch.device("cuda:0")
    c = synth.CONFIGS["self_forcing"]
    log("generating the self-forcing-shaped cache ...")
    x_cpu = synth.config_cache("self_forcing")
    H, N, d = x_cpu.shape
    nk = c["heads"]
    kinds = {"K": slice(0, nk), "V": slice(nk, H)}
    pre = {k: qvg.preset("pro", iters=c["iters"]) for k in kinds}
    x = x_cpu.to(dev)
    xs = {k: x[s].contiguous() for k, s in kinds.items()}
    idx = {k: synth.init_indices(50 + i, nk, pre[k].T, N, pre[k].C) for i, k in enumerate(kinds)}
    idx_p = {k: torch.from_numpy(v).pin_memory() for k, v in idx.items()}
    ws = {k: qvg.alloc_workspace(qvg.workspace_size(nk, N, d, x.dtype, pre[k]), dev) for k in kinds}
    rec = {k: qvg.empty_record(nk, N, d, pre[k], x.dtype, dev) for k in kinds}
    out = {k: torch.empty_like(xs[k]) for k in kinds}

    def step():
        for k in kinds:
            qvg.compress(xs[k], pre[k], init_idx=idx_p[k], ws=ws[k], out=rec[k])
        for k in kinds:
            qvg.decompress(rec[k], pre[k], out=out[k])

    ms = timed(step, args.steps, args.warmup)
    kt = kernel_times(qvg.KERNELS)
    log(json.dumps(kt, indent=1))
    # the K and V calls on two streams of their own (their latency-bound
    # kernels overlap); the records must come out the same
    before = {k: [getattr(rec[k], f).clone() for f in ("codes", "scales", "assign", "centroids")]
              for k in kinds}
    ms2 = concurrent_calls([(xs[k], pre[k], idx_p[k], ws[k], rec[k], out[k]) for k in kinds],
                           args.steps, args.warmup)
    same = all(torch.equal(a, getattr(rec[k], f)) for k in kinds
               for a, f in zip(before[k], ("codes", "scales", "assign", "centroids")))
    two_streams = {"calls": 2, "ms_per_step": ms2, "tokens_per_s": H * N / (ms2 * 1e-3),
                   "records_equal_sequential": bool(same)}
    del before
    dq = kt["fused_dequant"]
    dq_bytes = sum(dequant_bytes(nk, N, d, pre[k].C, pre[k].T, pre[k].bits, pre[k].group)
                   for k in kinds)
    dq_gbps = dq_bytes / (dq["total_ms"] / args.steps * 1e-3) / 1e9
    asg = kt["kmeans_assign"]
    asg_tflops = 2.0 * nk * N * 256 * d / (asg["avg_ms"] * 1e-3) / 1e12
    per_kind = {}
    for k in kinds:
        qvg.decompress(rec[k], pre[k], out=out[k])
        qp = qvg.preset("qvg", iters=c["iters"])
        rq = qvg.compress(xs[k], qp, init_idx=torch.from_numpy(idx[k][:, :qp.T].copy()))
        oq = qvg.decompress(rq, qp)
        per_kind[k] = {
            "record_bytes_per_head_tensor": rec[k].nbytes() // nk,
            "compression_ratio_vs_bf16": N * d * 2 / (rec[k].nbytes() / nk),
            "mse": _mse(out[k], xs[k]).mean().item(),
            "qvg_record_bytes_per_head_tensor": rq.nbytes() // nk,
            "qvg_compression_ratio_vs_bf16": N * d * 2 / (rq.nbytes() / nk),
            "qvg_mse": _mse(oq, xs[k]).mean().item()}
        del rq, oq
    res = {
        "metric": "compress+decompress tokens/s, QVG-Pro operating point (d=128 C=256 T=4 G=16)",
        "value": H * N / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "self-forcing-wan-1.3b-shaped KV cache: 12 K + 12 V head-tensors "
                               "x 32760 tokens, d=128, bf16, QVG-Pro per kind: C=256, T=4, "
                               "INT2, G=16, 8 iterations",
                   "presets": {k: {f: getattr(v, f) for f in ("C", "T", "iters", "bits", "group")}
                               for k, v in pre.items()}},
        "roofline": {"bound": "mfma", "achieved": asg_tflops, "peak": MFMA_F16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": asg_tflops / MFMA_F16_PEAK_TFLOPS,
                     "traffic": None, "kernel": "kmeans_assign", "avg_ms": asg["avg_ms"]},
        "dequant_GBps": dq_gbps, "dequant_hbm_frac": dq_gbps / HBM_PEAK_GBPS,
        "two_streams": two_streams,
        "per_kind": per_kind,
        "kernels_avg_ms": {k: round(v["avg_ms"], 5) for k, v in kt.items()},
    }
    if args.no_cpu_baseline:
        res["cpu_baseline"] = None
        return res
    log("oracle check of one K and one V head-tensor ...")
    # both kinds use the same preset here, so one oracle call (a thread each)
    xb = torch.cat([xs[k][:1] for k in kinds]).cpu().view(torch.int16).numpy().view(np.uint16)
    ib = np.concatenate([idx[k][:1] for k in kinds])
    pk = pre["K"]
    t0 = time.perf_counter()
    ref = oracle.compress(xb, C=pk.C, T=pk.T, iters=pk.iters, bits=pk.bits, G=pk.group,
                          init_idx=ib, threads=2)
    dt = time.perf_counter() - t0
    parity = True
    for i, k in enumerate(kinds):
        for f in ("codes", "scales", "assign"):
            parity &= np.array_equal(getattr(rec[k], f)[:1].cpu().numpy(), ref[f][i:i + 1])
        parity &= np.array_equal(rec[k].centroids[:1].cpu().view(torch.int16).numpy()
                                 .view(np.uint16), ref["cent"][i:i + 1])
    res["cpu_baseline"] = {"value": 2 * N / dt, "unit": "tokens/s", "cores": 2, "kind": "oracle", "cpu_model": cpu_model(),
                           "sample": f"head-tensor 0 of K and of V, all {N} tokens, all "
                                     f"{pk.T}x{pk.iters} k-means iterations, compress only "
                                     f"({dt:.1f} s wall, a thread per head-tensor)"}
    res["parity_sample_bit_exact"] = bool(parity)
    return res


def run_large(args):
    """The long-video cache: 32 K + 32 V head-tensors x 131072 tokens (4 scenes
    of 21 frames on a 39x40 grid), d=128, bf16, C=256, 8 iterations, T=4,
    INT2 and INT4 (G=64); the per-stage MSE curve and the record sizes."""
    dev = torch.device("cuda:0")
    c = synth.CONFIGS["long_video"]
    heads = args.large_heads or c["heads"]
    log(f"generating the long-video cache ({2 * heads} head-tensors) ...")
    x = synth.config_cache("long_video", heads=heads, workers=min(16, len(os.sched_getaffinity(0)))).to(dev)
    H, N, d = x.shape
    idx = torch.from_numpy(synth.init_indices(3, H, c["T"], N, c["C"])).pin_memory()
    out = torch.empty_like(x)
    res = {}
    for bits in (2, 4):
        p = qvg.params(C=c["C"], T=c["T"], iters=c["iters"], bits=bits, group=c["group"])
        ws = qvg.alloc_workspace(qvg.workspace_size(H, N, d, x.dtype, p), dev)
        rec = qvg.empty_record(H, N, d, p, x.dtype, dev)
        ms = timed(lambda: qvg.compress(x, p, init_idx=idx, ws=ws, out=rec), args.steps,
                   args.warmup)
        kt = kernel_times(qvg.KERNELS)
        dms, _ = _events_ms(lambda: qvg.decompress(rec, p, out=out))
        mse = _mse(out, x)
        asg = kt["kmeans_assign"]
        asg_tflops = 2.0 * H * N * p.C * d / (asg["avg_ms"] * 1e-3) / 1e12
        res[f"int{bits}"] = {
            "compress_ms": ms, "compress_tokens_per_s": H * N / (ms * 1e-3),
            "decompress_ms": dms, "mse_K": mse[:heads].mean().item(),
            "mse_V": mse[heads:].mean().item(),
            "record_bytes_per_head_tensor": rec.nbytes() // H,
            "compression_ratio_vs_bf16": N * d * 2 / (rec.nbytes() / H),
            "quantized_share": (rec.codes.numel() + rec.scales.numel()) / rec.nbytes(),
            "assign_tflops": asg_tflops, "assign_mfma_frac": asg_tflops / MFMA_F16_PEAK_TFLOPS,
            "kernels_avg_ms": {k: round(v["avg_ms"], 5) for k, v in kt.items()}}
        del ws, rec
    # per-stage MSE curve (INT2): stage count t = 0..T with the same seeded rows
    curve = {"K": [], "V": []}
    for t in range(c["T"] + 1):
        p = qvg.params(C=c["C"], T=t, iters=c["iters"], bits=2, group=c["group"])
        rec = qvg.compress(x, p, init_idx=idx[:, :t].contiguous() if t else None)
        qvg.decompress(rec, p, out=out)
        mse = _mse(out, x)
        curve["K"].append(mse[:heads].mean().item())
        curve["V"].append(mse[heads:].mean().item())
        del rec
    for k in ("K", "V"):
        curve[k + "_reduction_vs_naive"] = [curve[k][0] / m for m in curve[k]]
    r2 = res["int2"]
    cb = None
    if not args.no_cpu_baseline:
        # the oracle on the host's cores: INT2 compress (all T x iters k-means
        # iterations) of a bounded sample, the first 24576 tokens of 8 K and 8 V
        # head-tensors, each sampled head clustered on its own
        import oracle
        log("oracle baseline on the host cores ...")
        ncores = len(os.sched_getaffinity(0))
        sel = list(range(0, heads, max(1, heads // 8)))[:8]
        sel = sel + [heads + i for i in sel]
        ns = min(N, 24576)
        xs = x[sel, :ns].cpu().contiguous()
        xb = xs.view(torch.int16).numpy().view(np.uint16)
        threads = min(ncores, len(sel))
        p = qvg.params(C=c["C"], T=c["T"], iters=c["iters"], bits=2, group=c["group"])
        idx_s = synth.init_indices(33, len(sel), p.T, ns, p.C)
        t0 = time.perf_counter()
        ref = oracle.compress(xb, C=p.C, T=p.T, iters=p.iters, bits=p.bits, G=p.group,
                              init_idx=idx_s, threads=threads)
        dt = time.perf_counter() - t0
        # the same sample through the GPU path at the configured 8 iterations:
        # INT2 records bit for bit, and INT4 codes and scales against the
        # oracle's quantizer applied to its own final residual
        xs_dev = xs.to(dev)
        rec2 = qvg.compress(xs_dev, p, init_idx=idx_s)
        p4 = qvg.params(C=p.C, T=p.T, iters=p.iters, bits=4, group=p.group)
        rec4 = qvg.compress(xs_dev, p4, init_idx=idx_s)
        torch.cuda.synchronize()
        parity = all(np.array_equal(getattr(rec2, f).cpu().numpy(), ref[f])
                     for f in ("codes", "scales", "assign"))
        parity = parity and np.array_equal(
            rec2.centroids.cpu().view(torch.int16).numpy().view(np.uint16), ref["cent"])
        parity4 = True
        for i in range(len(sel)):
            r = oracle.bf16_bits_to_f32(xb[i])
            for t in range(p.T):
                r = oracle.subtract(r, ref["assign"][i, t].astype(np.int32),
                                    oracle.bf16_bits_to_f32(ref["cent"][i, t]))
            c4, s4 = oracle.quantize(r, 4, p.group)
            parity4 = parity4 and np.array_equal(rec4.codes[i].cpu().numpy(), c4) and \
                np.array_equal(rec4.scales[i].cpu().numpy(), s4)
        cb = {"value": len(sel) * ns / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
              "cpu_model": cpu_model(),
              "sample": f"first {ns} tokens of {len(sel)} of {H} head-tensors, INT2, all "
                        f"{p.T}x{p.iters} k-means iterations, compress ({dt:.1f} s wall, "
                        f"{ncores} host cores visible)",
              "parity_sample_bit_exact": {"int2_record": bool(parity),
                                          "int4_codes_scales": bool(parity4)}}
    return {"metric": "compress tokens/s, d=128 C=256 T=4 (long-video cache)",
            "value": r2["compress_tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": r2["compress_ms"],
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic",
            "config": {"workload": f"long-video cache: {heads} K + {heads} V head-tensors x "
                                   "131072 tokens (4 scenes x 21 frames x 39x40), d=128, bf16, "
                                   "C=256, 8 iterations, T=4, G=64",
                       "head_tensors": H, "tokens": N},
            "int2": r2, "int4": res["int4"], "mse_curve_int2": curve,
            "roofline": {"bound": "mfma", "achieved": r2["assign_tflops"],
                         "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": r2["assign_mfma_frac"], "traffic": None,
                         "kernel": "kmeans_assign"},
            "cpu_baseline": cb}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="selfforcing",
                    choices=["selfforcing", "decode", "stream", "large", "pro", "attn"])
    ap.add_argument("--nq", type=int, default=1, help="queries per head (attn workload)")
    ap.add_argument("--large-heads", type=int, default=None,
                    help="K (and V) head-tensors of the long-video cache (default 32)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode-leg", action="store_true",
                    help="skip the decode-side dequant at 40 x 262144 tokens in the default run")
    ap.add_argument("--cpu-heads", type=int, default=None)
    ap.add_argument("--copy-calibration", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: head-tensors are independent and the path "
              "exchanges nothing between GPUs, so there is no multi-GPU step to time. "
              "Use --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a HIP device", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        print(json.dumps(copy_calibration()), flush=True)
        return
    qvg.lib()
    res = {"selfforcing": run_selfforcing, "decode": run_decode, "stream": run_stream,
           "large": run_large, "pro": run_pro, "attn": run_attn}[args.workload](args)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
