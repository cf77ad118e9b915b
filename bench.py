#!/usr/bin/env python3
"""Benchmark: one paged decode step per iteration on one MI355X.

A step is the whole device path of a decode step for the batch: copy-on-write
block copies (when the step has any), the write of every sequence's new K/V
into its slot, then paged decode attention over each sequence's context
including that token.  The host block-manager work that produces the slots,
tables and copy pairs runs once per configuration and is timed separately.

HBM honesty: the step rotates over several independent sets of (pools,
tables, q, out) whose combined size is several times the 256 MB Infinity
Cache, so each step's KV comes from HBM.

Prints ONE JSON line (rank 0, N=1):
  value  = algorithmic KV bytes of the step / step time, in GB/s
  roofline = pa_decode's achieved algorithmic GB/s vs the 8 TB/s HBM peak,
             per-launch time measured with HIP events on the launch stream
  cpu_baseline = the fp64 oracle on the host, same algorithmic bytes
"""

from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, vendor figure
ROOT = os.path.dirname(os.path.abspath(__file__))
PROFILES = os.path.join(ROOT, "profiles")
# Sources that define the decode kernels; a traffic record is valid only for these bytes.
# What the decode kernels are built from: their sources and the headers they
# include (the compile flags are hashed beside them, see kernel_fingerprint)
KERNEL_SOURCES = ["paged_kv_cache_117_amd/csrc/decode_mfma.hip", "paged_kv_cache_117_amd/csrc/decode.hip",
                  "paged_kv_cache_117_amd/csrc/decode_api.hip", "paged_kv_cache_117_amd/csrc/decode_tile.h",
                  "paged_kv_cache_117_amd/csrc/decode_kernels.h", "paged_kv_cache_117_amd/csrc/pa_device.h"]
METRIC = "paged decode attention KV-read GB/s (% of MI355X HBM peak); seq-steps/s"
WARMUP_SECONDS = 0.2  # default warmup: GPU work before timing, for settled clocks
# Calls in each measurement pass after the timed region (the call alone, the
# unfused step, the main kernel alone): at least this many, whatever --steps
# says, so that a short timed region still gets stable per-call figures.
PASS_MIN_CALLS = 100
# Layers of the models the decode workloads are shaped after (one layer is benchmarked); used only
# to state the model's KV bytes per token next to the pages' sizing example.
MODEL_LAYERS = {"c2": 32, "c3": 40, "c4": 32, "c4b": 32, "c5": 80, "c5tp8": 80}
# Figures the source pages report, with the hardware they were measured on: context, not targets.
PAGES_CONTEXT = {
    "kv_memory_holding_tokens": "20.4-38.2% in the contiguous-slab servers profiled by the SOSP 2023 "
                                "PagedAttention paper vs 96.3% with paged blocks, on NVIDIA A100 "
                                "(PagedAttention: Virtual Memory for the KV Cache; PagedAttention and vLLM: "
                                "Paging the KV Cache Like an OS)",
    "serving_throughput": "2-4x over FasterTransformer and Orca at equal latency, NVIDIA A100 "
                          "(Batching and PagedAttention)",
    "kv_bytes_per_token_opt13b": "800 KB in FP16 (2 x 5120 hidden x 40 layers x 2 bytes); 1.6 GB for a "
                                 "2048-token request; about 30% of a 40 GB A100 left for the KV cache next to "
                                 "the 26 GB of weights (PagedAttention: Virtual Memory for the KV Cache)",
}
# partition size a workload states (positions per partition); others use the automatic split
WORKLOAD_PARTITION = {"c5": 512}  # (c5tp8: the automatic split; its partitions would be too few to balance)
WORKLOAD_NAMES = {
    "c1": "tiny paged decode fp32 (4 seqs, L in {1,5,16,37}, Hq=Hkv=2, D=64)",
    "c2": "Llama-3.1-8B decode layer bf16 (B=64, Hq=32, Hkv=8, D=128, L~U[128,4096], block 16)",
    "c3": "OPT-13B MHA decode layer fp16 (B=256, H=40, D=128, L~U[64,2048], block 16)",
    "c4": "parallel-sampling prefix share bf16 (32 prompts x 8 samples, prefix 1024, tails U[0,512])",
    "c4b": "fork step bf16 (32 prompts x 8 samples, prefix 1000, copy-on-write of the partial block)",
    "c5": "Qwen2.5-72B decode layer fp16 (B=128, Hq=64, Hkv=8, D=128, L~U[4096,8192], 512-token partitions)",
    "c5tp8": "one GPU's share of the Qwen2.5-72B decode layer at tensor parallel degree 8 fp16 (B=128, Hq=8, "
             "Hkv=1, D=128, C5's lengths, automatic split)",
}


# Chunked-prefill workloads (pa_write_kv of the chunk + pa_prefill per step)
PREFILL_METRIC = "paged chunked-prefill attention TFLOP/s (% of MI355X dense 16-bit MFMA peak); tokens/s"
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp16": 2500.0}  # MI355X dense, vendor figure
PREFILL_NAMES = {
    "p1": "Llama-3.1-8B prefill chunk layer bf16 (8 seqs x 512-token chunks, prior context U[0,3584], "
          "Hq=32, Hkv=8, D=128, block 16)",
    "p2": "Qwen2.5-72B prefill chunk layer fp16 (4 seqs x 1024-token chunks, prior context U[0,7168], "
          "Hq=64, Hkv=8, D=128, block 16)",
    "p3": "mixed chunked-prefill step bf16, Llama shapes (4 chunks of 512 + 60 single tokens)",
    "p4": "prefix-cache continuation bf16, Llama shapes (4 seqs x 64 new tokens after U[24576,32704] cached)",
    "p5": "mixed step with a long chunk bf16, Llama shapes (one 4096-token chunk + 127 single tokens after U[127,4095])",
}


# Preemption by swapping (pa_swap_blocks out to pinned host memory and back)
SWAP_METRIC = "paged KV swap-out + swap-in GB/s over the host link (pinned host pool)"
HOST_LINK_PEAK_GBPS = 64.0  # PCIe 5.0 x16, one direction, vendor figure
SWAP_NAMES = {
    "s1": "swap of 8 Llama-3.1-8B sequences x 2048 tokens, one layer bf16 (1024 blocks of 8 KV heads x 16 x 128, "
          "64 MiB K+V) to pinned host memory and back into other blocks",
}


# Host block manager with the prefix cache (no GPU work)
HOST_NAMES = {
    "h1": "prefix-cache churn: 32 prompts x 8 requests each, shared 1024-token prompt prefix + own tail "
          "U[0,512], arriving one by one (add with lookup, append with hashing), then freed",
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed warmup steps (default: at least 10, and at least %.1f s of GPU work, "
                         "so that clocks have settled)" % WARMUP_SECONDS)
    ap.add_argument("--config", default="c2",
                    choices=sorted(WORKLOAD_NAMES) + sorted(PREFILL_NAMES) + sorted(SWAP_NAMES) + sorted(HOST_NAMES))
    ap.add_argument("--partition-size", type=int, default=None,
                    help="positions per partition; 0 = automatic even split (default: the workload's, "
                         "512 for c5, automatic otherwise)")
    ap.add_argument("--sets", type=int, default=0, help="rotating buffer sets (0 = enough for >= 2 GiB)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="budget for the oracle baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--placement", choices=["shuffled", "sequential"], default="shuffled")
    ap.add_argument("--block-size", type=int, default=16,
                    help="slots per KV block for the decode workloads (8, 16, 32, 64, 128; 8 runs pa_decode through the prefill kernel)")
    ap.add_argument("--decode-kernel", choices=["auto", "valu", "partition"], default="auto",
                    help="pa_decode kernel override (PA_DECODE_KERNEL): valu = vector-ALU kernel for 16-bit KV "
                         "too, partition = matrix-core partition kernels instead of the even split")
    ap.add_argument("--no-second", action="store_true",
                    help="c2 only: skip the Qwen2.5-72B decode (c5) and Llama-3.1-8B prefill (p1) "
                         "sub-records of the default run")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run only a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--pmc-summary", nargs=4, metavar=("READ_CSV", "WRITE_CSV", "COPY_READ_CSV", "COPY_WRITE_CSV"),
                    help="turn rocprofv3 TCC counter CSVs (read and write passes of the decode bench and of "
                         "--calibrate-copy) into profiles/decode_<config>_traffic.json")
    return ap.parse_args()


def kernel_fingerprint():
    """Hash of the decode kernels' sources and the HIP compile flags: a counter
    record taken with other sources or flags no longer describes the kernel."""
    from paged_kv_cache_117_amd import build_lib

    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    # the flags without the include directories, whose absolute paths depend
    # on where the checkout lives
    flags, skip = [], False
    for f in build_lib.HIP_FLAGS:
        if skip:
            skip = False
        elif f == "-I":
            skip = True
        else:
            flags.append(f)
    h.update(" ".join(flags).encode())
    return h.hexdigest()[:16]


def traffic_record(key, partition_size):
    """The committed counter record of this workload's main kernel, while the
    kernel sources are the ones it was taken with (else None)."""
    path = os.path.join(PROFILES, f"decode_{key}_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except OSError:
        return None
    ok = (rec.get("kernel_sha") == kernel_fingerprint() and rec.get("config") == key
          and rec.get("partition_size") == partition_size and "read_scale" in rec
          and os.environ.get("PA_DECODE_KERNEL", "") in ("", "auto"))
    return rec if ok else None


def calibrate_copy():
    """A plain device copy of known size, for scaling the HBM byte counters."""
    import torch

    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": n, "copies": 5}))


def copy_bandwidth(torch, nbytes=1 << 30, reps=200):
    """The box's device-to-device copy rate: bytes read + bytes written per
    second of a plain 1 GiB copy (HIP events around `reps` copies, after two
    warm-up copies)."""
    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del src, dst
    return 2 * nbytes / (ms * 1e-3) / 1e9


READ_PROBE_GRIDS = {"sequential": (256, 512, 1024, 2048), "gather_4k": (256, 512, 1024)}


def read_ceiling(torch, nbytes=1 << 31, reps=20):
    """The box's read-only HBM ceiling from the library's read probe
    (pa_probe_read): a sequential sweep, and whole 4 KiB chunks gathered in a
    seeded random order -- the decode kernels' access shape, one KV head's
    16-slot tile per chunk.  Bytes read per second, best over a few launch
    sizes (HIP events around `reps` launches after one untimed launch)."""
    import paged_kv_cache_117_amd as pa

    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(11)
    order = torch.randperm(nbytes // 4096, device="cuda", generator=gen).to(torch.int32)
    wg_max = max(max(v) for v in READ_PROBE_GRIDS.values())
    sink = torch.empty(wg_max * 256, dtype=torch.int32, device="cuda")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    out = {}
    for mode, grids in READ_PROBE_GRIDS.items():
        best, best_wg = 0.0, 0
        for wg in grids:
            co = order if mode == "gather_4k" else None
            pa.probe_read(buf, sink, wg, co)
            e0.record()
            for _ in range(reps):
                pa.probe_read(buf, sink, wg, co)
            e1.record()
            torch.cuda.synchronize()
            gbs = nbytes / (e0.elapsed_time(e1) / reps * 1e-3) / 1e9
            if gbs > best:
                best, best_wg = gbs, wg
        out[f"{mode}_gbps"] = round(best, 1)
        out[f"{mode}_workgroups"] = best_wg
    del buf, order, sink
    return out


def _counter_means(path, kernel_pred):
    vals = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if kernel_pred(r["Kernel_Name"]):
                vals.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in vals.items()}, {k: len(v) for k, v in vals.items()}


def dominant_kernel_name(path, kernel_pred):
    with open(path) as f:
        for r in csv.DictReader(f):
            if kernel_pred(r["Kernel_Name"]):
                return r["Kernel_Name"]
    return "?"


# gfx950 L2 (TCC) -> memory fabric request counters, summed over the L2
# channels.  Read bytes = 32 n32 + 64 n64 + 128 n128 (requests by size); the
# DRAM-bound reads are also counted in 32-byte units (a 64-byte request as 2,
# 128-byte as 4).  Write bytes = 64 n64 + 32 (n - n64).
READ_COUNTERS = ["TCC_EA0_RDREQ_32B_sum", "TCC_EA0_RDREQ_64B_sum", "TCC_EA0_RDREQ_128B_sum",
                 "TCC_EA0_RDREQ_DRAM_32B_sum"]
WRITE_COUNTERS = ["TCC_EA0_WRREQ_sum", "TCC_EA0_WRREQ_64B_sum", "TCC_EA0_WRREQ_WRITE_DRAM_32B_sum"]


def _read_bytes(c):
    return 32 * c["TCC_EA0_RDREQ_32B_sum"] + 64 * c["TCC_EA0_RDREQ_64B_sum"] + 128 * c["TCC_EA0_RDREQ_128B_sum"]


def _write_bytes(c):
    return 64 * c["TCC_EA0_WRREQ_64B_sum"] + 32 * (c["TCC_EA0_WRREQ_sum"] - c["TCC_EA0_WRREQ_64B_sum"])


FUSE_MAX_KV_BYTES = 2 << 30  # pa_write_kv_decode's bound for the fused form (include/pa.h)


def write_fused_in_kernel(w):
    """Whether pa_write_kv_decode does its write inside the stream kernel for
    workload `w` (the choice include/pa.h states: 16-bit KV, up to 4096
    sequences, at most 2 GiB of K+V over num_seqs x max_context_len, no
    kernel override); otherwise a launch of its own writes first."""
    eb = {"fp32": 4, "fp16": 2, "bf16": 2}[w.dtype]
    bound = w.num_seqs * w.max_context_len * w.num_kv_heads * w.head_dim * eb * 2
    return (w.dtype != "fp32" and w.num_seqs <= 4096 and bound <= FUSE_MAX_KV_BYTES and w.block_size >= 16
            and os.environ.get("PA_DECODE_KERNEL", "") in ("", "auto"))


def main_kernel_bytes(w):
    """Algorithmic bytes of the step's main kernel: the attention's, plus the
    new rows read and written when the write runs inside it."""
    from paged_kv_cache_117_amd import metrics

    eb = metrics.ELEM_BYTES[w.dtype]
    f = metrics.write_decode_io_bytes if write_fused_in_kernel(w) else metrics.decode_io_bytes
    return f(w.context_lens, w.num_q_heads, w.num_kv_heads, w.head_dim, eb, w.block_size)


def pmc_summary(args):
    """HBM bytes per launch of the dominant decode kernel from the TCC request
    counters, each direction scaled by what the same counters read for a
    plain 1 GiB device copy (1 GiB read, 1 GiB written)."""
    from paged_kv_cache_117_amd import metrics
    from workloads import make_workload

    w = make_workload(args.config, block_size=args.block_size)
    # the step's main kernel: the stream kernel in the form the step runs
    # (the bench's other passes also run plain pa_decode)
    variant = ", true>" if write_fused_in_kernel(w) else ", false>"
    dec = lambda n: ("decode_stream<" in n and variant in n) or "decode_part" in n
    # the 1 GiB device copy itself (not the fill that creates its source)
    copy = lambda n: "copybuffer" in n.lower() or ("copy" in n.lower() and "fill" not in n.lower())
    rd, nf = _counter_means(args.pmc_summary[0], dec)
    wr, _ = _counter_means(args.pmc_summary[1], dec)
    crd, _ = _counter_means(args.pmc_summary[2], copy)
    cwr, _ = _counter_means(args.pmc_summary[3], copy)
    gib = float(1 << 30)
    r_scale = gib / _read_bytes(crd)
    w_scale = gib / _write_bytes(cwr)
    read_b = _read_bytes(rd)
    write_b = _write_bytes(wr)
    psize = args.partition_size if args.partition_size is not None else WORKLOAD_PARTITION.get(args.config, 0)
    eb = metrics.ELEM_BYTES[w.dtype]
    io = main_kernel_bytes(w)
    kv = metrics.decode_kv_bytes(w.context_lens, w.num_kv_heads, w.head_dim, eb)
    traffic = read_b * r_scale + write_b * w_scale
    rec = {
        "config": args.config,
        "partition_size": psize,
        "kernel": dominant_kernel_name(args.pmc_summary[0], dec),
        "kernel_sha": kernel_fingerprint(),
        "dispatches": nf.get("TCC_EA0_RDREQ_128B_sum", 0),
        "read_counters_per_dispatch": {k: round(rd[k], 1) for k in READ_COUNTERS},
        "write_counters_per_dispatch": {k: round(wr[k], 1) for k in WRITE_COUNTERS},
        "copy_read_counters": {k: round(crd[k], 1) for k in READ_COUNTERS},
        "copy_write_counters": {k: round(cwr[k], 1) for k in WRITE_COUNTERS},
        "read_bytes_by_size": int(read_b),
        "read_bytes_dram_32b_units": int(32 * rd["TCC_EA0_RDREQ_DRAM_32B_sum"]),
        "write_bytes_by_size": int(write_b),
        "write_bytes_dram_32b_units": int(32 * wr["TCC_EA0_WRREQ_WRITE_DRAM_32B_sum"]),
        "read_scale": round(r_scale, 4),
        "write_scale": round(w_scale, 4),
        "traffic_bytes_per_launch": int(traffic),
        "algorithmic_bytes_per_launch": io,
        "kv_bytes_per_launch": kv,
        "traffic_over_algorithmic": round(traffic / io, 4),
    }
    os.makedirs(PROFILES, exist_ok=True)
    out = os.path.join(PROFILES, f"decode_{args.config}_traffic.json")
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


def kv_utilization(bm, seq_ids, tables, block_size, num_blocks):
    """KV-cache utilisation after the host step: filled slots / slots of the
    blocks in use (a block shared by several sequences counts once, filled
    as far as its fullest holder), and blocks in use / pool blocks."""
    fill = {}
    for s, sid in enumerate(seq_ids):
        L = bm.num_tokens(int(sid))
        row = tables[s]
        for j in range(-(-L // block_size)):
            b = int(row[j])
            fill[b] = max(fill.get(b, 0), min(block_size, L - j * block_size))
    in_use = num_blocks - bm.num_free()
    return {"kv_slot_utilization": round(sum(fill.values()) / max(1, in_use * block_size), 4),
            "kv_blocks_in_use_frac": round(in_use / num_blocks, 4)}


def timing_events(torch, n, stream):
    """Per step: an event pair around the whole library call and one the
    library records around its main kernel (pa_time_next_main_kernel).  The
    second pair is recorded once here so that torch creates the events."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    kevs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for a, b in kevs:
        a.record(stream)
        b.record(stream)
    return evs, kevs


def settle_clocks(torch, seconds=0.1, nbytes=1 << 28):
    """Device copies for `seconds` of GPU time right before the warm-up
    steps.  The workload's host-side set-up leaves the GPU idle for a second
    or more, and its clocks drop; they rise again over the first tens of
    milliseconds of load, so a short explicit --warmup would time part of
    that ramp.  Not a step: the warm-up and timed steps are counted as given."""
    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    t0 = time.perf_counter()
    while True:
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= seconds:
            break
    del src, dst


class LeadIn:
    """About 0.1 ms of device copies enqueued, untimed, right before the timed
    region's start event, after the synchronize that opens it: the GPU works
    on them while the host enqueues the first timed steps, so the region
    holds the steps' GPU time and not the host's latency in launching the
    first one (tens of microseconds, 1-2% of a 20-step C2 region)."""

    def __init__(self, torch, nbytes=1 << 28):
        self.src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
        self.dst = torch.empty_like(self.src)

    def __call__(self, torch, stream):
        with torch.cuda.stream(stream):
            self.dst.copy_(self.src)


def roofline_bound(flops, nbytes, ms, peak_tflops, peak_gbps=HBM_PEAK_GBPS):
    """Roofline record of a launch of `flops` algorithmic flops and `nbytes`
    algorithmic bytes that took `ms`.  The bound is the larger of the two lower
    bounds on its time, the flops at the matrix peak and the bytes at the HBM
    peak: a launch whose arithmetic intensity (flops per byte) is below the
    ridge point peak_flops / peak_bytes (312 for 16-bit MFMA at 8 TB/s) -- a
    mixed step whose single-token rows stream most of the bytes, or a long
    continuation -- is bound by HBM, however much of its time the matrix cores
    take.  Both fractions are kept."""
    tflops = flops / (ms * 1e-3) / 1e12
    gbps = nbytes / (ms * 1e-3) / 1e9
    if flops / (peak_tflops * 1e12) >= nbytes / (peak_gbps * 1e9):
        rec = {"bound": "mfma", "achieved": round(tflops, 2), "peak": peak_tflops, "unit": "TFLOP/s",
               "frac": round(tflops / peak_tflops, 4)}
    else:
        rec = {"bound": "hbm", "achieved": round(gbps, 1), "peak": peak_gbps, "unit": "GB/s",
               "frac": round(gbps / peak_gbps, 4)}
    rec.update({"arithmetic_intensity": round(flops / nbytes, 1),
                "ridge": round(peak_tflops * 1e12 / (peak_gbps * 1e9), 1),
                "mfma_frac": round(tflops / peak_tflops, 4), "hbm_frac": round(gbps / peak_gbps, 4)})
    return rec


def warm_up(torch, step, n=None):
    """Untimed steps before the timed region: exactly `n` when given, else at
    least 10 and at least WARMUP_SECONDS of GPU work (the GPU raises its
    clocks over the first tens of milliseconds of sustained load; a short
    warmup times part of that ramp).  Returns the number of steps run.
    Either way the clocks are first settled by a pass of device copies."""
    settle_clocks(torch)
    i = 0
    if n is not None:
        for i in range(n):
            step(i)
        torch.cuda.synchronize()
        return n
    t0 = time.perf_counter()
    while True:
        step(i)
        i += 1
        if i >= 10 and i % 10 == 0:
            torch.cuda.synchronize()
            if time.perf_counter() - t0 >= WARMUP_SECONDS:
                return i


def call_pass(torch, step, steps, R, evs):
    """Durations (ms) of the library call alone over `steps` more steps of the
    same work, with an event pair around each call.  A pass of its own: an
    event recorded in the stream costs the GPU time, so the timed region
    above holds nothing but the steps."""
    torch.cuda.synchronize()
    for i in range(steps):
        step(i % R, evs[i])
    torch.cuda.synchronize()
    return np.array([a.elapsed_time(b) for a, b in evs])


def block_pass(torch, fn, steps, R, stream):
    """Mean duration (ms) of fn(i % R) over `steps` back-to-back calls between
    one event pair (after a few untimed ones), so no event sits between calls."""
    for i in range(max(5, steps // 4)):
        fn(i % R)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for i in range(steps):
        fn(i % R)
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def main_kernel_pass(torch, step, steps, R, kevs):
    """The main kernel's mean duration (ms) over `steps` more steps of the
    same work, the library handing `kevs[i]` to that kernel's launch so they
    take its own start and end (agreeing with the rocprofv3 kernel average).
    A pass of its own: events attached to a launch slow the whole call by a
    few microseconds, so the timed region above carries none."""
    torch.cuda.synchronize()
    for i in range(steps):
        step(i % R, None, kevs[i])
    torch.cuda.synchronize()
    return float(np.mean([a.elapsed_time(b) for a, b in kevs]))


def cpu_info():
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return model


def cpu_baseline(w, tables, budget_s):
    """The oracle as it stands, on whole-batch passes of the same step (or as
    many leading sequences as fit the budget), with BLAS held to one thread:
    its per-(sequence, head) loop runs on one core whatever BLAS is allowed
    (the same rate was measured with all host threads)."""
    import oracle  # test infrastructure: only this leg of the bench uses it
    from paged_kv_cache_117_amd import metrics
    from threadpoolctl import threadpool_limits

    eb = metrics.ELEM_BYTES[w.dtype]
    k, v = w.k_pool, w.v_pool
    with threadpool_limits(limits=1):
        # as many leading sequences as fit the budget (one timed probe sequence first)
        t0 = time.perf_counter()
        oracle.decode(w.q[:1], k, v, tables[:1], w.context_lens[:1], w.scale, w.dtype)
        per_tok = (time.perf_counter() - t0) / max(1, int(w.context_lens[0]))
        total_tok = int(w.context_lens.sum())
        reps = 1
        rows = w.num_seqs
        if per_tok * total_tok > budget_s:
            acc = 0
            rows = 0
            for L in w.context_lens:
                if (acc + int(L)) * per_tok > budget_s and rows > 0:
                    break
                acc += int(L)
                rows += 1
        else:
            reps = max(1, min(20, int(budget_s / max(per_tok * total_tok, 1e-9))))
        sel = slice(0, rows)
        t0 = time.perf_counter()
        for _ in range(reps):
            oracle.decode(w.q[sel], k, v, tables[sel], w.context_lens[sel], w.scale, w.dtype)
        dt = (time.perf_counter() - t0) / reps
    kvb = metrics.decode_kv_bytes(w.context_lens[sel], w.num_kv_heads, w.head_dim, eb)
    return {
        "value": round(kvb / dt / 1e9, 4),
        "unit": "GB/s",
        "cores": 1,
        "host_cores": os.cpu_count(),
        "kind": "oracle",
        "sample": (f"fp64 numpy oracle decode (gather + two-pass softmax), one thread, over the first {rows} of "
                   f"{w.num_seqs} sequences x {reps} pass(es), {dt:.3f} s per pass; "
                   f"seq-steps/s {rows / dt:.2f}; host CPU: {cpu_info()}"),
    }


def prefill_cpu_baseline(w, tables, budget_s):
    """The oracle's prefill on the first rows of the first sequence: those
    rows of the real workload, computed as a chunk of their own (same
    positions), as many as fit the budget; TFLOP/s of those rows."""
    import oracle  # test infrastructure: only this leg of the bench uses it
    from paged_kv_cache_117_amd import metrics

    from threadpoolctl import threadpool_limits

    P = int(w.prior_lens[0])

    def run(n):
        t0 = time.perf_counter()
        oracle.prefill(w.q[:n], w.k_pool, w.v_pool, tables[:1], [P + n], [0, n], w.scale, w.dtype)
        return time.perf_counter() - t0

    with threadpool_limits(limits=1):
        t1 = run(1)
        t4 = run(4)
        per_row = max((t4 - t1) / 3, 1e-6)
        n = max(1, min(int(w.chunk_lens[0]), int((budget_s - max(t1 - per_row, 0.0)) / per_row)))
        dt = run(n)
    fl = metrics.prefill_flops([P], [n], w.num_q_heads, w.head_dim)
    return {
        "value": round(fl / dt / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": 1,
        "host_cores": os.cpu_count(),
        "kind": "oracle",
        "sample": (f"fp64 numpy oracle prefill (gather + two-pass softmax per row), one thread, over the first {n} of "
                   f"{int(w.chunk_lens[0])} chunk tokens of sequence 0 (prior {P}), {dt:.3f} s; "
                   f"tokens/s {n / dt:.2f}; host CPU: {cpu_info()}"),
    }


def main_prefill(args):
    """One chunked-prefill step per iteration: write the chunk's K/V, then
    pa_prefill over every sequence's context."""
    import torch

    cpu_budget = 0.0 if args.no_cpu_baseline else args.cpu_seconds
    res = prefill_bench(torch, args.config, args, args.steps, args.warmup, cpu_budget, args.partition_size or 0)
    print(json.dumps(res), flush=True)


def prefill_bench(torch, key, args, steps, warmup, cpu_budget, pf_psize):
    """The chunked-prefill measurement of `key` (the record main_prefill prints)."""
    import paged_kv_cache_117_amd as pa
    from paged_kv_cache_117_amd import metrics
    from workloads import make_prefill_workload

    w = make_prefill_workload(key, block_size=args.block_size)
    eb = metrics.ELEM_BYTES[w.dtype]
    tdt = {"fp16": torch.float16, "bf16": torch.bfloat16}[w.dtype]
    order = w.perm if args.placement == "shuffled" else np.arange(w.num_blocks, dtype=np.int32)
    bm = pa.BlockManager(w.num_blocks, w.block_size, order)
    bm.replay(w.ops)
    t0 = time.perf_counter()
    slots = []
    for s, sid in enumerate(w.seq_ids):
        if w.chunk_lens[s]:
            slots.extend(bm.append(sid, int(w.chunk_lens[s])))
    slots = np.asarray(slots, dtype=np.int64)
    tables = bm.tables(w.seq_ids, w.max_blocks_per_seq)
    host_bm_ms = (time.perf_counter() - t0) * 1e3
    kv_util = kv_utilization(bm, w.seq_ids, tables, w.block_size, w.num_blocks)

    def dev(a, kv=False):
        a = np.ascontiguousarray(a)
        if kv and w.dtype == "bf16":
            return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(a).cuda()

    nb = w.num_blocks
    pool_bytes = 2 * nb * w.num_kv_heads * w.block_size * w.head_dim * eb
    R = args.sets or max(2, min(16, int(np.ceil(2**30 / pool_bytes))))
    k1, v1 = dev(w.k_pool, True), dev(w.v_pool, True)
    k_pool = torch.empty((R * nb,) + tuple(k1.shape[1:]), dtype=tdt, device="cuda")
    v_pool = torch.empty_like(k_pool)
    for r in range(R):
        k_pool[r * nb:(r + 1) * nb].copy_(k1)
        v_pool[r * nb:(r + 1) * nb].copy_(v1)
    del k1, v1
    q = dev(w.q, True)
    k_new, v_new = dev(w.k_new, True), dev(w.v_new, True)
    lens = dev(w.context_lens.astype(np.int32))
    qstart = dev(w.query_start.astype(np.int32))
    ws_bytes = pa.prefill_workspace_bytes(w.num_seqs, w.num_tokens, w.num_q_heads, w.num_kv_heads, w.head_dim,
                                          w.max_query_len, w.max_context_len, pf_psize)
    sets = []
    for r in range(R):
        t = np.where(tables >= 0, tables + r * nb, -1).astype(np.int32)
        sets.append(dict(tables=dev(t), slots=dev(slots + r * nb * w.block_size), out=torch.empty_like(q),
                         ws=torch.empty(max(1, ws_bytes), dtype=torch.uint8, device="cuda")))
    stream = torch.cuda.current_stream()

    def step(r, ev=None, kev=None):
        s = sets[r]
        pa.write_kv(k_pool, v_pool, k_new, v_new, s["slots"], stream=stream)
        if ev is not None:
            ev[0].record(stream)
        if kev is not None:
            pa.time_next_main_kernel(*kev)  # events around prefill_mfma alone
        pa.prefill(q, k_pool, v_pool, s["tables"], lens, qstart, w.scale, w.max_query_len, w.max_context_len,
                   out=s["out"], partition_size=pf_psize, workspace=s["ws"],
                   stream=stream)
        if ev is not None:
            ev[1].record(stream)

    warmup = warm_up(torch, lambda i: step(i % R), warmup)
    npass = max(steps, PASS_MIN_CALLS)  # the passes after the timed region
    evs, kevs = timing_events(torch, npass, stream)
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    lead = LeadIn(torch)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    lead(torch, stream)
    t_start.record(stream)
    for i in range(steps):
        step(i % R)
    t_end.record(stream)
    torch.cuda.synchronize()
    del lead
    wall = time.perf_counter() - wall0
    ms_step = t_start.elapsed_time(t_end) / steps
    pf_ms = call_pass(torch, step, npass, R, evs)
    pf_avg = float(pf_ms.mean())
    kern_avg = main_kernel_pass(torch, step, npass, R, kevs)
    flops = metrics.prefill_flops(w.prior_lens, w.chunk_lens, w.num_q_heads, w.head_dim)
    io = metrics.prefill_io_bytes(w.prior_lens, w.chunk_lens, w.num_q_heads, w.num_kv_heads, w.head_dim, eb)
    peak = MFMA_PEAK_TFLOPS[w.dtype]
    value = flops / (ms_step * 1e-3) / 1e12
    roof = roofline_bound(flops, io, kern_avg, peak)
    res = {
        "metric": PREFILL_METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {
            "workload": PREFILL_NAMES[key],
            "key": key,
            "num_seqs": w.num_seqs,
            "num_tokens": w.num_tokens,
            "flops_per_step": flops,
            "io_bytes_per_step": io,
            "block_size": w.block_size,
            "placement": args.placement,
            "rotating_sets": R,
            "partition_size": pf_psize or "auto",
            "split": bool(ws_bytes),
        },
        "mfma_peak_frac": round(value / peak, 4),
        "tokens_per_s": round(w.num_tokens / (ms_step * 1e-3), 1),
        "prefill_ms": round(pf_avg, 5),
        "prefill_ms_median": round(float(np.median(pf_ms)), 5),
        # the main kernel alone (events the library records right around it)
        "prefill_main_kernel_ms": round(kern_avg, 5),
        "prefill_call_mfma_frac": round(flops / (pf_avg * 1e-3) / 1e12 / peak, 4),
        "prefill_io_gbps": round(io / (pf_avg * 1e-3) / 1e9, 2),
        "host_block_manager_ms": round(host_bm_ms, 3),
        **kv_util,
        "wall_s": round(wall, 3),
        "roofline": {"kernel": "pa_prefill main kernel (prefill_mfma)", **roof, "traffic": None},
        "cpu_baseline": None,
    }
    if cpu_budget > 0:
        res["cpu_baseline"] = prefill_cpu_baseline(w, tables, cpu_budget)
    return res


def main_swap(args):
    """One step = swap 1024 blocks out to a pinned host pool, then back in."""
    import torch

    import paged_kv_cache_117_amd as pa
    import oracle  # test infrastructure: the cpu_baseline leg only

    nblk, hkv, D = 1024, 8, 128
    rng = np.random.default_rng(21)
    dev_blocks = 4 * nblk
    k = torch.randn(dev_blocks, hkv, 16, D, device="cuda", dtype=torch.bfloat16)
    v = torch.randn_like(k)
    hk = torch.empty((nblk, hkv, 16, D), dtype=torch.bfloat16, pin_memory=True)
    hv = torch.empty_like(hk, pin_memory=True)
    src = rng.permutation(dev_blocks)[:nblk]
    dst = rng.permutation(np.setdiff1d(np.arange(dev_blocks), src))[:nblk]
    out_pairs = torch.from_numpy(np.stack([src, rng.permutation(nblk)], 1).astype(np.int32)).cuda()
    in_pairs = torch.from_numpy(np.stack([out_pairs[:, 1].cpu().numpy(), dst], 1).astype(np.int32)).cuda()
    stream = torch.cuda.current_stream()
    moved = 2 * nblk * hkv * 16 * D * 2  # K and V bytes each way

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        pa.swap_blocks(hk, hv, k, v, out_pairs, stream=stream)
        if ev is not None:
            ev[1].record(stream)
        pa.swap_blocks(k, v, hk, hv, in_pairs, stream=stream)
        if ev is not None:
            ev[2].record(stream)

    args.warmup = warm_up(torch, lambda i: step(), args.warmup)
    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(args.steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(args.steps):
        step()
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    for i in range(args.steps):  # the two directions apart: a pass of its own (events cost GPU time)
        step(evs[i])
    torch.cuda.synchronize()
    out_ms = float(np.mean([a.elapsed_time(b) for a, b, _ in evs]))
    in_ms = float(np.mean([b.elapsed_time(c) for _, b, c in evs]))
    # reference: the DMA engines copying one contiguous buffer of the same size each way
    dbuf = torch.empty(moved // 2, dtype=torch.bfloat16, device="cuda")
    hbuf = torch.empty(moved // 2, dtype=torch.bfloat16, pin_memory=True)
    for _ in range(3):
        hbuf.copy_(dbuf, non_blocking=True)
        dbuf.copy_(hbuf, non_blocking=True)
    torch.cuda.synchronize()
    e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    e[0].record(stream)
    for _ in range(5):
        hbuf.copy_(dbuf, non_blocking=True)
    e[1].record(stream)
    for _ in range(5):
        dbuf.copy_(hbuf, non_blocking=True)
    e[2].record(stream)
    torch.cuda.synchronize()
    d2h = moved / (e[0].elapsed_time(e[1]) / 5 * 1e-3) / 1e9
    h2d = moved / (e[1].elapsed_time(e[2]) / 5 * 1e-3) / 1e9
    out_gbps = moved / (out_ms * 1e-3) / 1e9
    in_gbps = moved / (in_ms * 1e-3) / 1e9
    res = {
        "metric": SWAP_METRIC, "value": round(2 * moved / (ms * 1e-3) / 1e9, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": SWAP_NAMES[args.config], "key": args.config, "blocks": nblk,
                   "bytes_each_way": moved},
        "swap_out_gbps": round(out_gbps, 2), "swap_in_gbps": round(in_gbps, 2),
        "dma_contiguous_d2h_gbps": round(d2h, 2), "dma_contiguous_h2d_gbps": round(h2d, 2),
        "roofline": {"kernel": "pa_swap_blocks (swap-out)", "bound": "host link", "achieved": round(out_gbps, 2),
                     "peak": HOST_LINK_PEAK_GBPS, "unit": "GB/s", "frac": round(out_gbps / HOST_LINK_PEAK_GBPS, 4),
                     "traffic": None},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        hk_np = np.zeros((nblk, hkv, 16, D), np.uint16)
        k_np = rng.integers(0, 1 << 16, size=(dev_blocks // 4, hkv, 16, D), dtype=np.uint16)
        pairs = np.stack([np.arange(dev_blocks // 4), np.arange(dev_blocks // 4)], 1)
        t = time.perf_counter()
        oracle.swap_blocks(hk_np, hk_np, k_np, k_np, pairs)
        dt = time.perf_counter() - t
        res["cpu_baseline"] = {"value": round(2 * k_np.nbytes / dt / 1e9, 3), "unit": "GB/s", "cores": 1,
                               "kind": "oracle",
                               "sample": f"oracle swap_blocks of {dev_blocks // 4} blocks (K and V) between host "
                                         f"arrays, {dt:.3f} s; host CPU: {cpu_info()}"}
    print(json.dumps(res), flush=True)


def host_churn_requests(seed=31, prompts=32, per=8, prefix=1024, bs=16):
    rng = np.random.default_rng(seed)
    reqs = []
    for p in range(prompts):
        stem = rng.integers(0, 32000, size=prefix).tolist()
        for _ in range(per):
            reqs.append(stem + rng.integers(0, 32000, size=int(rng.integers(0, 513))).tolist())
    return reqs


def run_churn(bm, reqs):
    hits = 0
    for i, r in enumerate(reqs):
        n = bm.add_seq_cached(i, r)
        bm.append_tokens(i, r[n:])
        hits += n
    for i in range(len(reqs)):
        bm.free_seq(i)
    return hits


def main_host(args):
    import paged_kv_cache_117_amd as pa

    reqs = host_churn_requests()
    toks = sum(len(r) for r in reqs)
    nb = sum(-(-len(r) // 16) for r in reqs) + 16
    times = []
    for _ in range(max(1, args.steps)):
        bm = pa.BlockManager(nb, 16, prefix_cache=True)
        t = time.perf_counter()
        hits = run_churn(bm, reqs)
        times.append(time.perf_counter() - t)
    dt = float(np.median(times))
    full_blocks = sum(len(r) // 16 for r in reqs)
    res = {
        "metric": "host prefix-cache requests/s (lookup + append with chained SHA-256 block hashes)",
        "value": round(len(reqs) / dt, 1), "unit": "requests/s", "n_gpus": 0, "steps": len(times), "warmup": 0,
        "ms_per_step": round(dt * 1e3, 3), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "int32 tokens", "data": "synthetic",
        "config": {"workload": HOST_NAMES[args.config], "key": args.config, "requests": len(reqs), "tokens": toks},
        "cached_token_fraction": round(hits / toks, 4), "blocks_hashed_per_s": round(full_blocks / dt, 1),
        "roofline": None, "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        from oracle.prefix_cache import CachingBlockManager  # test infrastructure: this leg only

        sub = reqs[:64]
        t = time.perf_counter()
        run_churn(CachingBlockManager(nb, 16), sub)
        odt = time.perf_counter() - t
        res["cpu_baseline"] = {"value": round(len(sub) / odt, 1), "unit": "requests/s", "cores": 1,
                               "kind": "oracle",
                               "sample": f"oracle prefix cache (Python, hashlib) on the first {len(sub)} requests, "
                                         f"{odt:.3f} s; host CPU: {cpu_info()}"}
    print(json.dumps(res), flush=True)


def decode_bench(torch, key, args, partition_size, steps, warmup, cpu_budget):
    """One paged decode step per iteration on workload `key`: the step's
    copy-on-write copies (if any), pa_write_kv, pa_decode.  Returns the
    fields of the JSON line (timed region, per-call and main-kernel passes,
    roofline of the main kernel, the oracle baseline when cpu_budget > 0)."""
    import paged_kv_cache_117_amd as pa
    from paged_kv_cache_117_amd import metrics
    from workloads import make_workload

    w = make_workload(key, block_size=args.block_size)
    eb = metrics.ELEM_BYTES[w.dtype]
    tdt = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}[w.dtype]

    # ---- host block-manager work (H0): replay, then this step's appends --------
    order = w.perm if args.placement == "shuffled" else np.arange(w.num_blocks, dtype=np.int32)
    bm = pa.BlockManager(w.num_blocks, w.block_size, order)
    bm.replay(w.ops)
    t0 = time.perf_counter()
    slots = bm.append_batch(w.seq_ids)
    pairs = bm.take_copies_array()
    tables = bm.tables(w.seq_ids, w.max_blocks_per_seq)
    host_bm_ms = (time.perf_counter() - t0) * 1e3
    kv_util = kv_utilization(bm, w.seq_ids, tables, w.block_size, w.num_blocks)

    # ---- device buffers: R rotating sets, each a private region of one pool --------
    nb = w.num_blocks
    pool_bytes = 2 * nb * w.num_kv_heads * w.block_size * w.head_dim * eb
    R = args.sets or max(2, min(16, int(np.ceil(2 * 2**30 / pool_bytes))))

    def dev(a, dtype=None):
        a = np.ascontiguousarray(a)
        if w.dtype == "bf16" and dtype == "kv":
            return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(a).cuda()

    k1 = dev(w.k_pool, "kv")
    v1 = dev(w.v_pool, "kv")
    k_pool = torch.empty((R * nb,) + tuple(k1.shape[1:]), dtype=tdt, device="cuda")
    v_pool = torch.empty_like(k_pool)
    for r in range(R):
        k_pool[r * nb:(r + 1) * nb].copy_(k1)
        v_pool[r * nb:(r + 1) * nb].copy_(v1)
    del k1, v1
    q = dev(w.q, "kv")
    k_new = dev(w.k_new, "kv")
    v_new = dev(w.v_new, "kv")
    lens = dev(w.context_lens.astype(np.int32))
    ws_bytes = pa.decode_workspace_bytes(w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim, w.max_context_len,
                                         partition_size)
    sets = []
    for r in range(R):
        t = np.where(tables >= 0, tables + r * nb, -1).astype(np.int32)
        sets.append(dict(
            tables=dev(t),
            slots=dev(slots + r * nb * w.block_size),
            pairs=dev((pairs + r * nb).astype(np.int32)) if len(pairs) else None,
            out=torch.empty_like(q),
            ws=torch.empty(max(1, ws_bytes), dtype=torch.uint8, device="cuda"),
        ))
    stream = torch.cuda.current_stream()

    def step(r, ev=None, kev=None):
        """The step as one call: pa_write_kv_decode stores each sequence's new
        K/V at its last position and attends (after the copy-on-write copies)."""
        s = sets[r]
        if s["pairs"] is not None:
            pa.copy_blocks(k_pool, v_pool, s["pairs"], stream=stream)
        if ev is not None:
            ev[0].record(stream)
        if kev is not None:
            pa.time_next_main_kernel(*kev)  # events around the main kernel alone
        pa.write_kv_decode(q, k_pool, v_pool, k_new, v_new, s["tables"], lens, w.scale, w.max_context_len,
                           out=s["out"], partition_size=partition_size, workspace=s["ws"], stream=stream)
        if ev is not None:
            ev[1].record(stream)

    def call(r):
        """pa_write_kv_decode alone (no copies)."""
        s = sets[r]
        pa.write_kv_decode(q, k_pool, v_pool, k_new, v_new, s["tables"], lens, w.scale, w.max_context_len,
                           out=s["out"], partition_size=partition_size, workspace=s["ws"], stream=stream)

    def decode_only(r):
        """pa_decode alone (the attention of the unfused step)."""
        s = sets[r]
        pa.decode(q, k_pool, v_pool, s["tables"], lens, w.scale, w.max_context_len, out=s["out"],
                  partition_size=partition_size, workspace=s["ws"], stream=stream)

    def step_unfused(r):
        """The same step as separate calls: pa_write_kv, then pa_decode."""
        s = sets[r]
        if s["pairs"] is not None:
            pa.copy_blocks(k_pool, v_pool, s["pairs"], stream=stream)
        pa.write_kv(k_pool, v_pool, k_new, v_new, s["slots"], stream=stream)
        decode_only(r)

    warmup = warm_up(torch, lambda i: step(i % R), warmup)
    npass = max(steps, PASS_MIN_CALLS)  # the passes after the timed region
    _, kevs = timing_events(torch, npass, stream)
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    lead = LeadIn(torch)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    lead(torch, stream)
    t_start.record(stream)
    for i in range(steps):
        step(i % R)
    t_end.record(stream)
    torch.cuda.synchronize()
    del lead
    wall = time.perf_counter() - wall0
    total_ms = t_start.elapsed_time(t_end)
    ms_step = total_ms / steps
    # passes of their own after the timed region (same sets): the library
    # calls back to back, the unfused step, the main kernel alone
    call_ms = block_pass(torch, call, npass, R, stream)
    decode_only_ms = block_pass(torch, decode_only, npass, R, stream)
    ms_step_unfused = block_pass(torch, step_unfused, npass, R, stream)
    kern_avg = main_kernel_pass(torch, step, npass, R, kevs)

    kv_bytes = metrics.decode_kv_bytes(w.context_lens, w.num_kv_heads, w.head_dim, eb)
    unique_kv_bytes = metrics.decode_unique_kv_bytes(tables, w.context_lens, w.num_kv_heads, w.head_dim, eb,
                                                     w.block_size)
    io_bytes = main_kernel_bytes(w)
    call_io_bytes = metrics.write_decode_io_bytes(w.context_lens, w.num_q_heads, w.num_kv_heads, w.head_dim, eb,
                                                  w.block_size)
    dec_io_bytes = metrics.decode_io_bytes(w.context_lens, w.num_q_heads, w.num_kv_heads, w.head_dim, eb,
                                           w.block_size)
    value = kv_bytes / (ms_step * 1e-3) / 1e9
    dec_avg = call_ms
    achieved = io_bytes / (kern_avg * 1e-3) / 1e9
    res = {
        "value": round(value, 2),
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_step, 5),
        "dtype": w.dtype,
        "config": {
            "workload": WORKLOAD_NAMES[key],
            "key": key,
            "num_seqs": w.num_seqs,
            "kv_bytes_per_step": kv_bytes,
            "unique_kv_bytes_per_step": unique_kv_bytes,
            "block_size": w.block_size,
            "partition_size": partition_size or "auto (even split over all wavefronts)",
            "placement": args.placement,
            "rotating_sets": R,
            "copy_pairs": int(len(pairs)),
        },
        "hbm_peak_frac": round(value / HBM_PEAK_GBPS, 4),
        "seq_steps_per_s": round(w.num_seqs / (ms_step * 1e-3), 1),
        # the step as separate pa_write_kv + pa_decode calls (same sets, own timed region)
        "unfused_ms_per_step": round(ms_step_unfused, 5),
        "unfused_hbm_peak_frac": round(kv_bytes / (ms_step_unfused * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        # the pa_write_kv_decode call (its main kernel + the merge of cut
        # sequences; the write inside the kernel, or a launch of its own beyond
        # the fused form's size bound), back to back
        "decode_ms": round(dec_avg, 5),
        "decode_kv_gbps": round(kv_bytes / (dec_avg * 1e-3) / 1e9, 2),
        # pa_decode alone (attention only, the new tokens already in the pool), back to back
        "pa_decode_ms": round(decode_only_ms, 5),
        "pa_decode_hbm_frac": round(dec_io_bytes / (decode_only_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        # the main kernel alone (events the library records right around it;
        # the whole call adds the merge kernel and the gap before it)
        "decode_main_kernel_ms": round(kern_avg, 5),
        "decode_call_hbm_frac": round(call_io_bytes / (dec_avg * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "write_fused_in_kernel": write_fused_in_kernel(w),
        # distinct physical blocks read (shared prefix blocks once): equals the
        # logical rate unless sequences share blocks
        "decode_unique_kv_gbps": round(unique_kv_bytes / (dec_avg * 1e-3) / 1e9, 2),
        "host_block_manager_ms": round(host_bm_ms, 3),
        **kv_util,
        "kv_bytes_per_token_model": (2 * w.num_kv_heads * w.head_dim * eb * MODEL_LAYERS[key]
                                     if key in MODEL_LAYERS else None),
        "wall_s": round(wall, 3),
        "roofline": {
            "kernel": "pa_write_kv_decode main kernel (%s)" % main_kernel_label(w.dtype, w.num_seqs, w.block_size),
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": None,
        },
        "traffic_note": None,
        "algorithmic_bytes_per_launch": io_bytes,
    }
    rec = traffic_record(key, partition_size)
    if rec is not None:
        res["roofline"]["traffic"] = rec["traffic_bytes_per_launch"]
        res["traffic_note"] = ("HBM bytes per main-kernel launch from rocprofv3 TCC counters (read requests by "
                               "size + write requests by size, summed over channels), scaled by a 1 GiB copy "
                               "(read scale %.4f, write scale %.4f); %.3f x the algorithmic bytes per launch (%d)"
                               % (rec["read_scale"], rec["write_scale"], rec["traffic_bytes_per_launch"] / io_bytes,
                                  io_bytes))
    del sets, k_pool, v_pool
    torch.cuda.empty_cache()
    if cpu_budget > 0:
        res["cpu_baseline"] = cpu_baseline(w, tables, cpu_budget)
    return res


def main_kernel_label(dtype, num_seqs, block_size=16):
    kern = os.environ.get("PA_DECODE_KERNEL", "")
    if block_size == 8:
        return "prefill_mfma over one query row per sequence (blocks of 8 slots), matrix cores"
    if dtype == "fp32" or kern == "valu":
        return "decode_part_valu, vector ALU"
    if kern == "partition" or num_seqs > 4096:
        return "decode_part_wave / decode_part_mfma, matrix cores"
    return "decode_stream, the even split over all wavefronts, matrix cores"


def main():
    args = parse()
    if args.pmc_summary:
        pmc_summary(args)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); this path has no "
              "multi-GPU mode: sequences or KV heads shard across GPUs with no exchange inside "
              "attention, so run one process per GPU.", file=sys.stderr)
        sys.exit(2)
    if args.decode_kernel != "auto":
        # read by the library at each pa_decode call
        os.environ["PA_DECODE_KERNEL"] = args.decode_kernel

    if args.config in HOST_NAMES:
        main_host(args)
        return
    if args.config in SWAP_NAMES:
        import torch

        torch.cuda.set_device(0)
        main_swap(args)
        return
    if args.config in PREFILL_NAMES:
        import torch

        torch.cuda.set_device(0)
        main_prefill(args)
        return

    import torch

    import paged_kv_cache_117_amd  # noqa: F401  (fails loudly when libpa.so is missing)

    torch.cuda.set_device(0)
    if args.calibrate_copy:
        calibrate_copy()
        return
    # The box's device-copy rate first: it is reported beside the decode rate,
    # and its ~0.1 s of HBM-bound work also brings the GPU's clocks up before
    # the warm-up steps.
    cg = copy_bandwidth(torch)
    rc = read_ceiling(torch)
    psize =args.partition_size if args.partition_size is not None else WORKLOAD_PARTITION.get(args.config, 0)
    cpu_budget = 0.0 if args.no_cpu_baseline else args.cpu_seconds
    core = decode_bench(torch, args.config, args, psize, args.steps, args.warmup, cpu_budget)
    res = {
        "metric": METRIC,
        "value": core.pop("value"),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": core.pop("steps"),
        "warmup": core.pop("warmup"),
        "ms_per_step": core.pop("ms_per_step"),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": core.pop("dtype"),
        "data": "synthetic",
        "config": core.pop("config"),
    }
    cpu = core.pop("cpu_baseline", None)
    res.update(core)
    res["device_copy_gbps"] = round(cg, 1)
    res["decode_frac_of_copy"] = round(res["decode_kv_gbps"] / cg, 4)
    res["read_ceiling"] = dict(rc)
    res["read_ceiling"]["main_kernel_frac_of_gather"] = round(res["roofline"]["achieved"] / rc["gather_4k_gbps"], 4)
    res["read_ceiling"]["note"] = ("read-only probe kernels on this box (pa_probe_read): the main kernel's "
                                   "algorithmic bytes per second over the 4 KiB random-gather rate")
    res["pages_context"] = PAGES_CONTEXT
    # The second target workload (Qwen2.5-72B layer, 512-position partitions)
    # beside the headline, measured the same way in the same run.
    if args.config == "c2" and not args.no_second:
        sub = decode_bench(torch, "c5", args, WORKLOAD_PARTITION["c5"], args.steps, args.warmup, 0.0)
        res["c5"] = {k: sub[k] for k in ("value", "hbm_peak_frac", "ms_per_step", "seq_steps_per_s", "decode_ms",
                                          "decode_main_kernel_ms", "decode_call_hbm_frac", "pa_decode_ms",
                                          "pa_decode_hbm_frac", "unfused_ms_per_step", "unfused_hbm_peak_frac",
                                          "roofline", "traffic_note", "warmup", "steps", "dtype")}
        res["c5"]["workload"] = sub["config"]["workload"]
        res["c5"]["kv_bytes_per_step"] = sub["config"]["kv_bytes_per_step"]
        res["c5"]["partition_size"] = sub["config"]["partition_size"]
        res["c5"]["unit"] = "GB/s"
        res["c5"]["main_kernel_frac_of_gather"] = round(sub["roofline"]["achieved"] / rc["gather_4k_gbps"], 4)
        # and the chunked-prefill path (f1) on the Llama-3.1-8B chunk layer:
        # its own warm-up by time (the matrix-bound load after the two
        # memory-bound ones) and at least 50 timed steps
        pre = prefill_bench(torch, "p1", args, max(args.steps, 50), None, 0.0, 0)
        res["p1"] = {k: pre[k] for k in ("value", "unit", "mfma_peak_frac", "ms_per_step", "prefill_ms",
                                          "prefill_main_kernel_ms", "prefill_call_mfma_frac", "roofline",
                                          "warmup", "steps", "dtype")}
        res["p1"]["workload"] = pre["config"]["workload"]
        res["p1"]["flops_per_step"] = pre["config"]["flops_per_step"]
    res["cpu_baseline"] = cpu
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
