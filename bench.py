#!/usr/bin/env python3
"""Benchmark of the exact-attention hot path on one MI355X.

Headline (``value``): forward-attention throughput in TFLOP/s on the causal
MHA workload B=8, H=32, N=4096, d=128 (bf16 inputs drawn N(0,1)*0.5 from a
seed, scale 1/sqrt(128)).  One timed step is one ``attn_fwd`` call that
builds the block mask in its workspace and runs the forward kernel, i.e. the
whole forward path.  FLOPs count 4*d per visible (query, key) pair.

The same JSON line also carries:
  roofline      the forward kernel alone (prebuilt block mask), timed with
                HIP events on the stream it is launched on, against the bf16
                dense MFMA peak; every prefill workload in ``configs`` carries
                its own block of the same form;
  decode        split-KV decode (split + combine kernels) on B=16, 32 query
                heads over 8 KV heads, T=32768, lens U[1024, 32768], chunk
                1024: HBM GB/s of the algorithmic K/V bytes, against 8 TB/s;
  backward      attn_bwd (dQ, dK, dV) on the headline workload with a seeded
                output gradient: TFLOP/s at 2.5x the forward's FLOPs (five
                products per visible pair), against the bf16 MFMA peak;
  varlen        attn_fwd_varlen on the GQA document workload packed into
                [B*N, H, d] with its documents as the sequences (config 7,
                on config 4's inputs);
  alibi         the forward kernel on the headline workload with the ALiBi
                distance bias, slopes 2^(-8(h+1)/H) (config 8, on config 2's
                inputs);
  fp8           the FP8 forward kernel on the headline workload's inputs,
                Q and K rotated by a random-sign Hadamard matrix and all
                three block-quantized to E4M3 (config 9): TFLOP/s against
                the fp8 dense MFMA peak, plus the quantization time;
  configs       every workload's time and throughput;
  cpu_baseline  the fp64 oracle timed on the host cores on a bounded sample
                of the headline workload (rows of a few heads).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                       [--configs 1,2,3,4,5,6,7,8,9]

Configs 7, 8 and 9 generate the inputs of the workload they derive from but
time only themselves unless that workload is listed too, so that a profiler
run can hold one workload's dispatches alone.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import attn_inputs as gen  # noqa: E402

METRIC = "fwd attention TFLOPS & % bf16 MFMA peak; decode split-KV HBM GB/s"
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16
MFMA_FP8_PEAK_TFLOPS = 5000.0   # MI355X dense fp8
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E
# Backward FLOPs: five products per visible pair (S recomputed, dP, dV, dK,
# dQ), 2*d each, against the forward's two.
BWD_FLOP_FACTOR = 2.5
CSRC = os.path.join(ROOT, "exact_attention_15_amd", "csrc")

# HBM bytes per launch, per workload, from two rocprofv3 --pmc runs
# (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch) of this script, each scaled
# by what the same counter reads for a device copy of known size
# (--calibrate-copy): FETCH_SIZE counts half of the bytes a copy reads,
# WRITE_SIZE all of those it writes.  A figure holds only for the kernel
# source it was taken on; if the sources' sha256 differs it is reported as
# null (stale).  The build script is hashed with the sources, since its
# per-file compiler flags change the kernels' machine code too.
_FWD_SRC = ["fwd.hip", "tile.h", "common.h", "../build.py"]
MEASURED_TRAFFIC = {
    # workload: (kernels, sources, sha256 of their concatenation, bytes per launch, summary)
    "causal_b8_h32_n4096_d128": (
        "k_attn_fwd_d128",
        ["fwd.hip", "tile.h", "common.h", "../build.py"],
        "0f81c7e8ff75e4a65c09cbb88236dc9e615987a9d7641cfa7af8da17b39feca1",
        1098892425,
        "profiles/k_attn_fwd_d128_causal_b8_h32_n4096_d128.md"),
    "window1024_softcap50_b4_h32_n16384_d128": (
        "k_attn_fwd_d128_softcap",
        ["fwd.hip", "tile.h", "common.h", "../build.py"],
        "0f81c7e8ff75e4a65c09cbb88236dc9e615987a9d7641cfa7af8da17b39feca1",
        2444712249,
        "profiles/k_attn_fwd_d128_softcap_window1024_softcap50_b4_h32_n16384_d128.md"),
    "gqa32x8_docs_causal_b2_n8192_d128": (
        "k_attn_fwd_d128",
        ["fwd.hip", "tile.h", "common.h", "../build.py"],
        "0f81c7e8ff75e4a65c09cbb88236dc9e615987a9d7641cfa7af8da17b39feca1",
        351172670,
        "profiles/k_attn_fwd_d128_gqa32x8_docs_causal_b2_n8192_d128.md"),
    "varlen_gqa32x8_docs_causal_b2_n8192_d128": (
        "k_mask_tiles + k_mask_order + k_attn_fwd_d128",
        ["fwd.hip", "tile.h", "common.h", "../build.py", "mask.hip"],
        "b0e43b10366c5b1e028c3f7ac4189ffc2cfa6945442ea44477fe003fbcd55d28",
        349854851,
        "profiles/attn_fwd_varlen_gqa32x8_docs_b2_n8192_d128.md"),
    "alibi_causal_b8_h32_n4096_d128": (
        "k_attn_fwd_d128_alibi",
        ["fwd.hip", "tile.h", "common.h", "../build.py"],
        "0f81c7e8ff75e4a65c09cbb88236dc9e615987a9d7641cfa7af8da17b39feca1",
        1161138002,
        "profiles/k_attn_fwd_d128_alibi_causal_b8_h32_n4096_d128.md"),
    "fp8_causal_b8_h32_n4096_d128": (
        "k_attn_fwd8_d128",
        ["fwd8.hip", "tile.h", "common.h", "../build.py"],
        "2a0a81eb691acfce4ebc5c2a5145541e608f76b8a66157b914f202e244cea4fc",
        686732329,
        "profiles/k_attn_fwd8_d128_causal_b8_h32_n4096_d128.md"),
    "decode_b16_gqa32x8_t32768_d128_chunk1024": (
        "k_decode_split + k_decode_combine",
        ["decode.hip", "common.h", "../build.py"],
        "c3772f0195e9a3d4a50501737135247e92e96facd1467ab377dc3f2ee413cb07",
        961753627,
        "profiles/k_decode_split_decode_b16_gqa32x8_t32768_d128.md"),
    "bwd_causal_b8_h32_n4096_d128": (
        "all kernels of one attn_bwd call",
        ["bwd.hip", "tile.h", "common.h", "mask.hip", "../build.py"],
        "43b774b8bfb2726cddb7538a6bcbf31850ba715ed95577eaed6001944a16e372",
        3284480928,
        "profiles/k_bwd_d128_causal_b8_h32_n4096_d128.md"),
}

# Forward kernel that each prefill workload runs.
FWD_KERNEL = {1: "k_attn_fwd_d64", 2: "k_attn_fwd_d128", 3: "k_attn_fwd_d128_softcap",
              4: "k_attn_fwd_d128"}
# Workloads timed on another workload's inputs: varlen packs workload 4,
# ALiBi and FP8 run on workload 2's Q, K, V.
DERIVED_FROM = {7: 4, 8: 2, 9: 2}


def sources_sha256(names) -> str:
    import hashlib
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(CSRC, n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload: str):
    """Counter-measured HBM bytes per launch on ``workload`` or None if there
    is no figure for the current source."""
    entry = MEASURED_TRAFFIC.get(workload)
    if entry is None:
        return None
    _, names, digest, nbytes, _ = entry
    return nbytes if sources_sha256(names) == digest else None


def mfma_roofline(tflops: float, peak: float, workload: str, **extra):
    return dict({"bound": "mfma", "achieved": round(tflops, 2), "peak": peak, "unit": "TFLOP/s",
                 "frac": round(tflops / peak, 4), "traffic": measured_traffic(workload)}, **extra)


# ---------------------------------------------------------------------------
# Algorithmic work accounting (host, closed forms from the mask intervals).
# ---------------------------------------------------------------------------
def row_intervals(kind: str, N: int, *, window=None, doc_offsets=None):
    """Visible key interval [lo, hi] of every query row (one batch row)."""
    i = np.arange(N, dtype=np.int64)
    lo = np.zeros(N, np.int64)
    hi = np.full(N, N - 1, np.int64)
    if kind in ("causal", "docs_causal"):
        hi = np.minimum(hi, i)
    if kind == "window_softcap":
        lo = np.maximum(lo, i - window)
        hi = np.minimum(hi, i + window)
    if doc_offsets is not None:
        offs = np.asarray(doc_offsets, np.int64)
        idx = np.searchsorted(offs, i, side="right") - 1
        lo = np.maximum(lo, offs[idx])
        hi = np.minimum(hi, offs[idx + 1] - 1)
    return lo, hi


def visible_pairs(kind: str, B: int, N: int, *, window=None, doc_rows=None) -> int:
    """Visible (query, key) pairs of one head, summed over the batch."""
    total = 0
    for b in range(B):
        lo, hi = row_intervals(kind, N, window=window,
                               doc_offsets=None if doc_rows is None else doc_rows[b])
        total += int(np.maximum(hi - lo + 1, 0).sum())
    return total


def fwd_flops(pairs_per_head: int, H: int, d: int) -> float:
    """QK^T and PV: 2*d each per visible pair."""
    return 4.0 * d * pairs_per_head * H


def score_matrix_bytes(B, H, N, elem_bytes=2) -> int:
    """Bytes of a materialised [B, H, N, N] score matrix."""
    return B * H * N * N * elem_bytes


def kv_cache_bytes(B, Hkv, T, d, elem_bytes=2) -> int:
    """Bytes of a K and V cache pair [B, Hkv, T, d]."""
    return 2 * B * Hkv * T * d * elem_bytes


def decode_bytes(lens, Hkv, Hq, d) -> int:
    """Algorithmic HBM bytes of one decode step: the valid K and V rows, the
    queries, the outputs and the LSE (the partials are workspace traffic and
    are not counted)."""
    lens = np.asarray(lens, np.int64)
    B = len(lens)
    return int(lens.sum()) * Hkv * d * 2 * 2 + B * Hq * d * 2 * 2 + B * Hq * 4 + B * 4


def fwd_io_bytes(B, Hq, Hkv, N, d) -> int:
    """Compulsory HBM bytes of the forward pass: Q, K, V read once, O and
    LSE written once."""
    return (B * Hq * N * d + 2 * B * Hkv * N * d) * 2 + B * Hq * N * d * 2 + B * Hq * N * 4


# ---------------------------------------------------------------------------
# Workloads
# ---------------------------------------------------------------------------
def fwd_workload(cfg_id: int, device):
    import torch
    c = gen.CONFIGS[cfg_id]
    docs = c["kind"] == "docs_causal"
    q, k, v, doc_rows = gen.fwd_inputs(c["seed"], c["B"], c["Hq"], c["Hkv"], c["N"], c["d"],
                                       c["factor"], docs=docs)
    w = dict(cfg=c, q_bits=q, k_bits=k, v_bits=v, doc_rows=doc_rows)
    w["q"], w["k"], w["v"] = (to_dev(x, device) for x in (q, k, v))
    w["scale"] = 1.0 / math.sqrt(c["d"])
    kw_dev, kw_ref = {}, {}
    if c["kind"] in ("causal", "docs_causal"):
        kw_dev["causal"] = kw_ref["causal"] = True
    if c["kind"] == "window_softcap":
        kw_dev["window"] = kw_ref["window"] = c["window"]
        kw_dev["softcap"] = kw_ref["softcap"] = c["softcap"]
    if docs:
        padded, _ = gen.pad_offsets(doc_rows, c["N"])
        kw_ref["doc_offsets"] = padded
        kw_dev["doc_offsets"] = torch.from_numpy(padded).to(device)
    w["kw_dev"], w["kw_ref"] = kw_dev, kw_ref
    w["pairs_per_head"] = visible_pairs(c["kind"], c["B"], c["N"], window=c.get("window"),
                                        doc_rows=doc_rows)
    w["flops"] = fwd_flops(w["pairs_per_head"], c["Hq"], c["d"])
    return w


def decode_workload(device):
    import torch
    c = gen.CONFIGS[5]
    q, kc, vc, lens = gen.decode_inputs(c["seed"], c["B"], c["Hq"], c["Hkv"], c["T"], c["d"])
    w = dict(cfg=c, q_bits=q, k_bits=kc, v_bits=vc, lens=lens)
    w["q"], w["k"], w["v"] = (to_dev(x, device) for x in (q, kc, vc))
    w["lens_dev"] = torch.from_numpy(lens).to(device)
    w["scale"] = 1.0 / math.sqrt(c["d"])
    w["bytes"] = decode_bytes(lens, c["Hkv"], c["Hq"], c["d"])
    return w


def to_dev(bits, device):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


# ---------------------------------------------------------------------------
# Timing
# ---------------------------------------------------------------------------
def time_launches(fn, steps: int, warmup: int):
    """Average ms per call: warmup calls, then `steps` calls between HIP events
    recorded on the current stream (the stream the library launches on)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        fn()
    stop.record()
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / steps


def warm_gpu(fn, seconds: float = 0.3):
    """Run ``fn`` back to back for about ``seconds`` so that timing starts on
    a GPU at its steady-state clock (the first ~0.1 s of work after idle runs
    several percent slower)."""
    import torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n = 1
    while time.perf_counter() - t0 < seconds:
        for _ in range(n):
            fn()
        torch.cuda.synchronize()
        n = min(2 * n, 64)


def time_each(fn, steps: int):
    """Per-call ms (events around every call) for median/min/p90."""
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for a, b in evs:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    t = np.array([a.elapsed_time(b) for a, b in evs])
    return dict(median_ms=float(np.median(t)), min_ms=float(t.min()),
                p90_ms=float(np.percentile(t, 90)))


def bench_fwd(ea, w, steps, warmup):
    import torch
    c = w["cfg"]
    spec = ea.MaskSpec(**w["kw_dev"])
    B, N = c["B"], c["N"]
    o = torch.empty((B, c["Hq"], N, c["d"]), dtype=torch.bfloat16, device=w["q"].device)
    lse = torch.empty((B, c["Hq"], N), dtype=torch.float32, device=w["q"].device)
    bm = ea.mask_build(spec, B, N)

    def step_with_mask_build():
        ea.fwd(w["q"], w["k"], w["v"], spec=spec, scale=w["scale"], out=o, lse=lse)

    def kernel_only():
        ea.fwd(w["q"], w["k"], w["v"], spec=spec, scale=w["scale"], block_mask=bm, out=o, lse=lse)

    def mask_only():
        ea.mask_build(spec, B, N)

    warm_gpu(step_with_mask_build)
    ms_kernel = time_launches(kernel_only, steps, warmup)
    ms_step = time_launches(step_with_mask_build, steps, warmup)
    dist = time_each(kernel_only, max(steps, 20))
    ms_mask = time_launches(mask_only, max(steps // 2, 5), 2)
    return dict(ms_step=ms_step, ms_kernel=ms_kernel, ms_mask_build=ms_mask, dist=dist,
                tflops_step=w["flops"] / (ms_step * 1e-3) / 1e12,
                tflops_kernel=w["flops"] / (ms_kernel * 1e-3) / 1e12)


def bench_decode(ea, w, steps, warmup):
    import torch
    c = w["cfg"]
    o = torch.empty((c["B"], c["Hq"], c["d"]), dtype=torch.bfloat16, device=w["q"].device)
    lse = torch.empty((c["B"], c["Hq"]), dtype=torch.float32, device=w["q"].device)
    ws = torch.empty(ea.decode_workspace_bytes(c["B"], c["Hq"], c["T"], c["d"], c["chunk"]),
                     dtype=torch.uint8, device=w["q"].device)

    def step():
        ea.decode(w["q"], w["k"], w["v"], w["lens_dev"], scale=w["scale"], chunk=c["chunk"],
                  out=o, lse=lse, workspace=ws)

    warm_gpu(step)
    ms = time_launches(step, steps, warmup)
    dist = time_each(step, max(steps, 20))
    return dict(ms=ms, dist=dist, gbs=w["bytes"] / (ms * 1e-3) / 1e9)


def bench_bwd(ea, w, steps, warmup):
    """attn_bwd (block masks, dQ kernel with the per-row prep, dK/dV kernel) on the
    forward workload ``w`` with its own forward outputs and a seeded dO."""
    import torch
    c = w["cfg"]
    B, Hq, Hkv, N, d = c["B"], c["Hq"], c["Hkv"], c["N"], c["d"]
    dev = w["q"].device
    spec = ea.MaskSpec(**w["kw_dev"])
    g = to_dev(gen.dout_input(c["dout_seed"], B, Hq, N, d), dev)
    o, lse = ea.fwd(w["q"], w["k"], w["v"], spec=spec, scale=w["scale"])
    dq = torch.empty_like(w["q"])
    dk = torch.empty_like(w["k"])
    dv = torch.empty_like(w["v"])
    ws = torch.empty(ea.bwd_workspace_bytes(B, Hq, N, spec), dtype=torch.uint8, device=dev)

    def step():
        ea.bwd(w["q"], w["k"], w["v"], o, lse, g, spec=spec, scale=w["scale"], dq=dq, dk=dk, dv=dv,
               workspace=ws)

    warm_gpu(step)
    ms = time_launches(step, steps, warmup)
    dist = time_each(step, max(steps, 10))
    return dict(ms=ms, dist=dist)


def bench_varlen(ea, w, steps, warmup):
    """attn_fwd_varlen (block mask for the packed sequences + forward kernel)
    on the document workload ``w`` packed into [B*N, H, d] with its documents
    as the sequences."""
    import torch
    c = w["cfg"]
    B, N = c["B"], c["N"]
    pk = lambda t: t.transpose(1, 2).reshape(B * N, t.shape[1], t.shape[3]).contiguous()
    q, k, v = pk(w["q"]), pk(w["k"]), pk(w["v"])
    cu = np.concatenate([w["doc_rows"][b][:-1] + b * N for b in range(B)] + [[B * N]]).astype(np.int32)
    cud = torch.from_numpy(cu).to(q.device)
    o = torch.empty_like(q)
    lse = torch.empty((c["Hq"], B * N), dtype=torch.float32, device=q.device)
    ws = torch.empty(ea.fwd_varlen_workspace_bytes(B * N, B * N), dtype=torch.uint8, device=q.device)

    def step():
        ea.fwd_varlen(q, k, v, cud, cud, causal=True, scale=w["scale"], out=o, lse=lse, workspace=ws)

    warm_gpu(step)
    ms = time_launches(step, steps, warmup)
    return dict(ms=ms, nseq=len(cu) - 1, tflops=w["flops"] / (ms * 1e-3) / 1e12)


def bench_fp8(ea, w, steps, warmup):
    """Quantization (three attn_quantize_fp8 calls: Q and K rotated, V with
    one scale per head) and the FP8 forward kernel with a prebuilt block
    mask, on the forward workload ``w``."""
    import torch
    c = w["cfg"]
    B, Hq, N, d = c["B"], c["Hq"], c["N"], c["d"]
    dev = w["q"].device
    signs = torch.from_numpy(gen.hadamard_signs(c["signs_seed"], d)).to(dev)
    spec = ea.MaskSpec(**w["kw_dev"])
    q8, qs = ea.quantize_fp8(w["q"], signs=signs)
    k8, ks = ea.quantize_fp8(w["k"], signs=signs)
    v8, vs = ea.quantize_fp8(w["v"], per_head=True)
    o = torch.empty((B, Hq, N, d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=dev)
    bm = ea.mask_build(spec, B, N)

    def quantize():
        ea.quantize_fp8(w["q"], signs=signs, out=q8, scales=qs)
        ea.quantize_fp8(w["k"], signs=signs, out=k8, scales=ks)
        ea.quantize_fp8(w["v"], per_head=True, out=v8, scales=vs)

    def kernel_only():
        ea.fwd_fp8(q8, k8, v8, qs, ks, vs, spec=spec, scale=w["scale"], block_mask=bm, out=o, lse=lse)

    warm_gpu(kernel_only)
    ms_kernel = time_launches(kernel_only, steps, warmup)
    dist = time_each(kernel_only, max(steps, 20))
    ms_quant = time_launches(quantize, max(steps // 2, 5), 2)
    # algorithmic HBM bytes of the three quantize calls: bf16 in, E4M3 out
    # (V's per-head scale reads its input twice; that is not counted)
    qbytes = 3 * B * Hq * N * d * (2 + 1)
    return dict(ms_kernel=ms_kernel, dist=dist, ms_quant=ms_quant,
                tflops_kernel=w["flops"] / (ms_kernel * 1e-3) / 1e12,
                quant_gbs=qbytes / (ms_quant * 1e-3) / 1e9)


def cpu_baseline(w, target_s=15.0):
    """The fp64 oracle on whole (batch row, head) slices of the workload, timed
    on the host cores; throughput in the metric's unit (TFLOP/s).  One slice
    is timed first to size the sample at about ``target_s`` seconds."""
    import oracle
    c = w["cfg"]
    N, B, Hq = c["N"], c["B"], c["Hq"]
    units = [(b, h) for b in range(B) for h in range(Hq)]  # batch row major

    def pairs_of(b):
        lo, hi = row_intervals(c["kind"], N, window=c.get("window"),
                               doc_offsets=None if w["doc_rows"] is None else w["doc_rows"][b])
        return int(np.maximum(hi - lo + 1, 0).sum())

    def run(sel):
        rows = np.array([(b, h, i) for b, h in sel for i in range(N)], np.int32)
        t0 = time.perf_counter()
        oracle.fwd(w["q_bits"], w["k_bits"], w["v_bits"], scale=w["scale"], rows=rows,
                   **w["kw_ref"])
        return time.perf_counter() - t0

    t = run(units[:1])
    n = int(max(1, min(len(units), round(target_s / max(t, 1e-3)))))
    if n > 1:
        t += run(units[1:n])
    flops = sum(fwd_flops(pairs_of(b), 1, c["d"]) for b, _ in units[:n])
    return {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": oracle.threads(),
            "kind": "oracle",
            "sample": f"all {N} query rows of the first {n} of {len(units)} (batch row, head) "
                      f"slices of {c['name']} ({flops / 1e9:.1f} GFLOP, {t:.1f} s wall)"}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--configs", default="1,2,3,4,5,6,7,8,9")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run one device-to-device copy of MIB MiB (a known-size "
                         "kernel for scaling the HBM byte counters), then exit")
    args = ap.parse_args(argv)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the forward and decode kernels run on a single "
              "MI355X and no multi-GPU path is built (use --gpus 1).", file=sys.stderr)
        return 2

    import torch
    import exact_attention_15_amd as ea
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    dev = torch.device("cuda", 0)
    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n}))
        return 0
    ea.library()
    cfg_ids = [int(x) for x in args.configs.split(",") if x]

    results = {}
    headline = None
    varlen_res = None
    alibi_res = None
    fp8_res = None
    bases = sorted({c for c in cfg_ids if c in FWD_KERNEL}
                   | {DERIVED_FROM[c] for c in cfg_ids if c in DERIVED_FROM})
    for cid in bases:
        print(f"[bench] config {cid}: generating inputs", file=sys.stderr, flush=True)
        w = fwd_workload(cid, dev)
        c = w["cfg"]
        r = None
        if cid in cfg_ids:
            r = bench_fwd(ea, w, args.steps, args.warmup)
            results[c["name"]] = {
                "ms_step": round(r["ms_step"], 4), "ms_kernel": round(r["ms_kernel"], 4),
                "ms_mask_build": round(r["ms_mask_build"], 4),
                "kernel_median_ms": round(r["dist"]["median_ms"], 4),
                "kernel_min_ms": round(r["dist"]["min_ms"], 4),
                "kernel_p90_ms": round(r["dist"]["p90_ms"], 4),
                "tflops_step": round(r["tflops_step"], 2),
                "tflops_kernel": round(r["tflops_kernel"], 2),
                "frac_mfma_peak": round(r["tflops_kernel"] / MFMA_BF16_PEAK_TFLOPS, 4),
                "flops": w["flops"], "visible_pairs_per_head": w["pairs_per_head"],
                "roofline": mfma_roofline(r["tflops_kernel"], MFMA_BF16_PEAK_TFLOPS, c["name"],
                                          kernel=FWD_KERNEL[cid]),
            }
            print(f"[bench] config {cid} {c['name']}: {r['ms_kernel']:.3f} ms kernel, "
                  f"{r['tflops_kernel']:.1f} TFLOP/s", file=sys.stderr, flush=True)
        if cid == 4 and 7 in cfg_ids:
            rv = bench_varlen(ea, w, args.steps, args.warmup)
            name = "varlen_" + c["name"]
            varlen_res = {
                "workload": name, "sequences": rv["nseq"],
                "ms": round(rv["ms"], 4), "tflops": round(rv["tflops"], 2),
                "roofline": mfma_roofline(rv["tflops"], MFMA_BF16_PEAK_TFLOPS, name,
                                          kernels="k_mask_tiles + k_mask_order + k_attn_fwd_d128 "
                                                  "(one attn_fwd_varlen call, timed together)"),
            }
            results[name] = {"ms": varlen_res["ms"], "tflops": varlen_res["tflops"]}
            print(f"[bench] config 7 (config 4 packed, varlen): {rv['ms']:.3f} ms, "
                  f"{rv['tflops']:.1f} TFLOP/s", file=sys.stderr, flush=True)
        if cid == 2 and 8 in cfg_ids:
            # the same workload with the ALiBi distance bias (geometric slopes)
            slopes = torch.tensor([2.0 ** (-8.0 * (h + 1) / c["Hq"]) for h in range(c["Hq"])],
                                  dtype=torch.float32, device=dev)
            wa = dict(w, kw_dev=dict(w["kw_dev"], alibi_slopes=slopes))
            ra = bench_fwd(ea, wa, args.steps, args.warmup)
            name = "alibi_" + c["name"]
            alibi_res = {
                "workload": name, "slopes": "2^(-8(h+1)/H)",
                "ms_step": round(ra["ms_step"], 4), "ms_kernel": round(ra["ms_kernel"], 4),
                "tflops_kernel": round(ra["tflops_kernel"], 2),
                "roofline": mfma_roofline(ra["tflops_kernel"], MFMA_BF16_PEAK_TFLOPS, name,
                                          kernel="k_attn_fwd_d128_alibi"),
            }
            results[name] = {"ms_kernel": alibi_res["ms_kernel"],
                             "tflops_kernel": alibi_res["tflops_kernel"]}
            print(f"[bench] config 8 (config 2 with ALiBi): {ra['ms_kernel']:.3f} ms kernel, "
                  f"{ra['tflops_kernel']:.1f} TFLOP/s", file=sys.stderr, flush=True)
        if cid == 2 and 9 in cfg_ids:
            rf = bench_fp8(ea, dict(w, cfg=gen.CONFIGS[9]), args.steps, args.warmup)
            name = gen.CONFIGS[9]["name"]
            fp8_res = {
                "workload": name,
                "rotation": "diag(random signs) * Hadamard / sqrt(128) on Q and K",
                "ms_kernel": round(rf["ms_kernel"], 4),
                "kernel_median_ms": round(rf["dist"]["median_ms"], 4),
                "tflops_kernel": round(rf["tflops_kernel"], 2),
                "ms_quantize_qkv": round(rf["ms_quant"], 4),
                "quantize_gbs": round(rf["quant_gbs"], 1),
                "roofline": mfma_roofline(rf["tflops_kernel"], MFMA_FP8_PEAK_TFLOPS, name,
                                          kernel="k_attn_fwd8_d128"),
            }
            results[name] = {"ms_kernel": fp8_res["ms_kernel"],
                             "tflops_kernel": fp8_res["tflops_kernel"]}
            print(f"[bench] config 9 (config 2 in FP8): {rf['ms_kernel']:.3f} ms kernel, "
                  f"{rf['tflops_kernel']:.1f} TFLOP/s; quantize {rf['ms_quant']:.3f} ms",
                  file=sys.stderr, flush=True)
        if cid == 2 and r is not None:
            headline = (w, r)
        else:
            del w
        torch.cuda.empty_cache()

    decode_res = None
    if 5 in cfg_ids:
        print("[bench] config 5: generating inputs", file=sys.stderr, flush=True)
        wd = decode_workload(dev)
        r = bench_decode(ea, wd, args.steps, args.warmup)
        c = wd["cfg"]
        decode_res = {
            "workload": c["name"], "ms": round(r["ms"], 4),
            "median_ms": round(r["dist"]["median_ms"], 4), "min_ms": round(r["dist"]["min_ms"], 4),
            "p90_ms": round(r["dist"]["p90_ms"], 4),
            "algorithmic_bytes": wd["bytes"], "gbs": round(r["gbs"], 1),
            "roofline": {"bound": "hbm", "achieved": round(r["gbs"], 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(r["gbs"] / HBM_PEAK_GBS, 4),
                         "traffic": measured_traffic(c["name"]),
                         "kernels": "k_decode_split + k_decode_combine (timed together)"},
        }
        results[c["name"]] = {"ms": decode_res["ms"], "gbs": decode_res["gbs"],
                              "frac_hbm_peak": decode_res["roofline"]["frac"]}
        print(f"[bench] config 5: {r['ms']:.3f} ms, {r['gbs']:.0f} GB/s", file=sys.stderr, flush=True)
        del wd
        torch.cuda.empty_cache()

    bwd_res = None
    if 6 in cfg_ids:
        print("[bench] config 6 (backward of config 2): generating inputs", file=sys.stderr, flush=True)
        wb = fwd_workload(6, dev)
        r = bench_bwd(ea, wb, args.steps, args.warmup)
        c = wb["cfg"]
        flops = BWD_FLOP_FACTOR * wb["flops"]
        tf = flops / (r["ms"] * 1e-3) / 1e12
        bwd_res = {
            "workload": c["name"], "ms": round(r["ms"], 4),
            "median_ms": round(r["dist"]["median_ms"], 4), "min_ms": round(r["dist"]["min_ms"], 4),
            "p90_ms": round(r["dist"]["p90_ms"], 4),
            "flops": flops, "tflops": round(tf, 2),
            "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
                         "traffic": measured_traffic(c["name"]),
                         "kernels": "k_bwd_mask_kv + k_bwd_dq + k_bwd_dkdv and the "
                                    "forward block mask (one attn_bwd call, timed together)"},
        }
        results[c["name"]] = {"ms": bwd_res["ms"], "tflops": bwd_res["tflops"],
                              "frac_mfma_peak": bwd_res["roofline"]["frac"]}
        print(f"[bench] config 6: {r['ms']:.3f} ms, {tf:.1f} TFLOP/s", file=sys.stderr, flush=True)
        del wb
        torch.cuda.empty_cache()

    out = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic: seeded N(0,1) bf16 inputs (x0.5 for the headline workload)"}
    if headline is not None:
        w, r = headline
        c = w["cfg"]
        out.update({
            "value": round(r["tflops_step"], 2), "unit": "TFLOP/s",
            "ms_per_step": round(r["ms_step"], 4),
            "config": {"workload": c["name"], "B": c["B"], "Hq": c["Hq"], "Hkv": c["Hkv"],
                       "N": c["N"], "d": c["d"], "mask": "causal", "scale": w["scale"],
                       "flops_per_step": w["flops"],
                       "step": "attn_fwd building its block mask, then the forward kernel"},
            "roofline": mfma_roofline(r["tflops_kernel"], MFMA_BF16_PEAK_TFLOPS, c["name"],
                                      kernel="k_attn_fwd_d128", kernel_ms=round(r["ms_kernel"], 4)),
        })
        if not args.no_cpu_baseline:
            print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
            out["cpu_baseline"] = cpu_baseline(w)
    if decode_res is not None:
        out["decode"] = decode_res
    if bwd_res is not None:
        out["backward"] = bwd_res
    if varlen_res is not None:
        out["varlen"] = varlen_res
    if alibi_res is not None:
        out["alibi"] = alibi_res
    if fp8_res is not None:
        out["fp8"] = fp8_res
    out["configs"] = results
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
