#!/usr/bin/env python3
"""Decode-step benchmark for the paged KV-cache library on one MI355X.

A step is one pass of the whole decode hot path over one batch, one
`paged_decode_step` call: slot mapping of the new tokens, their KV append,
and paged decode attention (context partitions, merged by log-sum-exp
inside each work-group and, for sequences longer than one chunk, by a
merge kernel).  Batches of up to 64 sequences run it as one launch (the
attention takes the new tokens from the step's input while work-groups of
the same launch store them); larger ones as an append launch that also
writes the batch's longest-first schedule, then the attention launch.
Inputs are synthetic and
resident in HBM before timing starts.

Default run: the three decode layers of the bandwidth target, one after the
other in one process -- MHA (64 sequences, 32/32 heads, lengths uniform on
[128, 2048], block size 16), GQA (256 sequences, 32/8 heads, log-normal
lengths) and long context (8 sequences, 64/8 heads, lengths uniform on
[32768, 131072], block size 32, 512-token partitions); head size 128, bf16,
shuffled block IDs.  One step of the whole job is one decode step of each
layer; `value` is the job's KV-read GB/s (the KV bytes the three attentions
must read / the sum of the three step times), and `per_config` holds each
layer's own record (step time and its spread, append and attention times,
graph replay, roofline with its counter record, CPU oracle baseline with a
full-size parity check, paged-vs-contiguous diagnostic).  The top-level
`roofline` is the dominant kernel's: the attention launch that takes
longest (the one-launch step where the step is one launch).
`--config N` runs one configuration alone and prints its record.

Prints one JSON line.  `roofline` times the attention call with HIP events
on its own stream; `cpu_baseline` times the CPU oracle on a bounded sample
of the same workloads (whole passes, about --cpu-seconds each).
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

HBM_PEAK_GBPS = 8000.0
# paged_decode_step is one launch for batches of up to this many sequences
ONE_LAUNCH_MAX_SEQS = 64

# counter records (rocprofv3 FETCH_SIZE / WRITE_SIZE of the attention launch) per configuration
TRAFFIC_RECORDS = {(2, "fp8"): "traffic_paged_decode_attention_mha_fp8.txt",
                   2: "traffic_paged_decode_attention_mha_bf16.txt",
                   3: "traffic_paged_decode_attention_gqa_bf16.txt",
                   4: "traffic_paged_decode_attention_long_context_bf16.txt",
                   5: "traffic_paged_decode_attention_shared_prefix_bf16.txt"}


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=None, choices=[1, 2, 3, 4, 5],
                    help="one decode configuration (default: configurations 2, 3 and 4 in turn, one decode step "
                         "of each per step)")
    ap.add_argument("--seed", type=int, default=None,
                    help="seed of the synthetic inputs (default: the configuration number; another seed disables "
                         "the counter record, which was taken on the default inputs)")
    ap.add_argument("--no-contiguous-diag", action="store_true",
                    help="skip the paged-vs-contiguous timing of the attention launch")
    ap.add_argument("--partition-tokens", type=int, default=None,
                    help="context partition length (default: the configuration's, else the library's choice)")
    ap.add_argument("--rotate", type=int, default=2,
                    help="independent copies of the inputs used in turn, so that no step reads what the previous "
                         "step left in the 256 MB infinity cache")
    ap.add_argument("--contiguous", action="store_true",
                    help="diagnostic: each sequence's blocks adjacent in the pool (paged vs contiguous storage)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="skip the graph-replay timing of the decode step")
    ap.add_argument("--cpu-seconds", type=float, default=8.0,
                    help="target CPU time of the oracle sample, per configuration")
    ap.add_argument("--traffic", type=str, default=None,
                    help="record of measured HBM bytes per attention launch (rocprofv3 FETCH_SIZE/WRITE_SIZE, "
                         "calibrated; default: the configuration's record under profiles/); used only when its "
                         "workload and kernel-source hash match this run")
    ap.add_argument("--kv-dtype", choices=["native", "fp8"], default="native",
                    help="pool element type: the configuration's own (bf16 or fp32), or FP8 E4M3 codes with one "
                         "scale per pool (bf16 queries)")
    ap.add_argument("--copy-blocks", type=int, default=0, metavar="PAIRS",
                    help="instead of the decode step, time pkv_copy_blocks (copy-on-write) of PAIRS random block "
                         "pairs in the configuration's pools and print its own JSON line")
    ap.add_argument("--q-len", type=int, default=0, metavar="N",
                    help="instead of the decode step, time the multi-token step (chunked prefill / speculative "
                         "decoding): the last min(N, L) tokens of every sequence are query rows, appended and then "
                         "attended causally; prints its own JSON line")
    ap.add_argument("--block-size", type=int, default=0, metavar="B",
                    help="override the configuration's block size (1, 8, 16, 32 or 64; same lengths and values)")
    ap.add_argument("--block-size-sweep", action="store_true",
                    help="instead of the decode step, time the attention launch of the configuration at every block "
                         "size 1, 8, 16, 32, 64, with shuffled and with contiguous block IDs; prints one JSON line")
    ap.add_argument("--calib-copy", type=int, default=0, metavar="MIB",
                    help="instead of the benchmark, run 20 device-to-device copies of MIB MiB (counter calibration)")
    return ap.parse_args()


def device_inputs(w, torch):
    def t(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    d = dict(q=t(w.q), kc=t(w.k_cache), vc=t(w.v_cache), bt=t(w.block_tables), sl=t(w.seq_lens),
             nk=t(w.new_k), nv=t(w.new_v))
    if w.q_start is not None:
        d["qs"] = t(w.q_start)
    return d


MFMA_BF16_PEAK_TFLOPS = 2500.0   # dense bf16 MFMA (fp8 pools are decoded to bf16 operands)
MFMA_F32_PEAK_TFLOPS = 157.3


def stream_read_ceiling(torch, pkv, nbytes: int = 2 << 30, reps: int = 20) -> dict:
    """The GPU's practical read bandwidth: the library's streaming-read probe
    over a 2 GiB buffer (best of two grid sizes, events around `reps` reads),
    reported next to the kernels' rates as the ceiling they can approach."""
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    out = torch.zeros(4, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    best = (0.0, 0)
    for wg in (2048, 8192):
        for _ in range(3):
            pkv.probe_stream_read(buf, out, wg, stream=stream)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            pkv.probe_stream_read(buf, out, wg, stream=stream)
        b.record(stream)
        torch.cuda.synchronize()
        gbps = nbytes * reps / (a.elapsed_time(b) / 1e3) / 1e9
        best = max(best, (gbps, wg))
    del buf, out
    torch.cuda.empty_cache()
    return {"gbps": round(best[0], 1), "work_groups": best[1], "bytes": nbytes}


def gather_read_ceiling(torch, pkv, w, copies, reps: int = 20):
    """The rate of the workload's paged access pattern on its own: the
    library's gather-read probe over the key and value tiles that the
    attention reads (every (sequence, KV head, block) tile of each
    sequence's first ceil(L / B) table entries, keys and values in turn, in
    batch order), every address known in advance, alternating between the
    input copies as the timed steps do (best of four grid sizes).  None when
    a tile is not a multiple of 1 KiB (B = 1)."""
    esz = {"f32": 4, "bf16": 2, "fp8": 1}[w.dtype]
    tile = w.B * w.hs * esz
    if tile % 1024:
        return None
    nblk = (w.seq_lens.astype(np.int64) + w.B - 1) // w.B
    ids, heads = [], []
    for s in range(w.S):
        row = w.block_tables[s, :nblk[s]].astype(np.int64)
        ids.append(np.tile(row, w.Hkv))
        heads.append(np.repeat(np.arange(w.Hkv, dtype=np.int64), nblk[s]))
    base = (np.concatenate(ids) * w.Hkv + np.concatenate(heads)) * tile
    offs = np.repeat(base, 2)  # key tile, then the value tile at the same place of the other pool
    t_offs = torch.from_numpy(offs).cuda()
    out = torch.zeros(4, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    nbytes = len(offs) * tile
    best = (0.0, 0)
    for wg in (4096, 8192, 16384, 32768):
        for i in range(3):
            d = copies[i % len(copies)]
            pkv.probe_gather_read(d["kc"], d["vc"], t_offs, tile, out, wg, stream=stream)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for i in range(reps):
            d = copies[i % len(copies)]
            pkv.probe_gather_read(d["kc"], d["vc"], t_offs, tile, out, wg, stream=stream)
        b.record(stream)
        torch.cuda.synchronize()
        us = a.elapsed_time(b) * 1e3 / reps
        best = max(best, (nbytes / us / 1e3, wg, us))
    del t_offs, out
    return {"gbps": round(best[0], 1), "work_groups": best[1], "us": round(best[2], 2), "bytes": int(nbytes),
            "tiles": int(len(offs)), "tile_bytes": int(tile),
            "gbps_algorithmic": round(w.kv_read_bytes() / best[2] / 1e3, 1)}


def multi_token_counts(w):
    """(KV bytes, attention flops) one multi-token step must move and do: each
    sequence's L cached tokens once per KV head (keys and values), plus the
    query and output rows; 2 * hs flops per (row, query head, visible token)
    for the scores and as many for the value sum."""
    kv = w.kv_read_bytes()
    io_elem = 4 if w.dtype == "f32" else 2
    qo = 2 * w.rows * w.Hq * w.hs * io_elem
    n = np.diff(w.q_start).astype(np.int64)
    L = w.seq_lens.astype(np.int64)
    # row i of s sees L - n + i + 1 tokens: sum over i = n (L - n) + n (n + 1) / 2
    visible = int((n * (L - n) + n * (n + 1) // 2).sum())
    return kv + qo, 4 * w.hs * w.Hq * visible


def bench_multi_token(args, w, torch, pkv) -> dict:
    """paged_multi_token_step (slot mapping, append of every query row, causal
    attention) on the configuration with the last min(q_len, L) tokens of
    each sequence as query rows; the attention launch timed with events."""
    copies = [device_inputs(w, torch) for _ in range(max(1, args.rotate))]
    d0 = copies[0]
    P = w.partition_tokens if args.partition_tokens is None else args.partition_tokens
    mql = w.max_q_len
    ws_step = pkv.alloc_multi_token_step_workspace(d0["q"], d0["kc"], d0["vc"], d0["bt"], mql, P)
    ws = pkv.alloc_multi_token_workspace(d0["q"], d0["kc"], d0["vc"], d0["bt"], mql, P)
    sched = pkv.alloc_schedule(d0["bt"])
    out = torch.empty_like(d0["q"])
    slots = torch.empty(w.rows, dtype=torch.int64, device="cuda")
    stream = torch.cuda.current_stream()
    sc = dict(k_scale=w.k_scale, v_scale=w.v_scale)
    turn = [0]

    def step():
        d = copies[turn[0] % len(copies)]
        turn[0] += 1
        pkv.paged_multi_token_step(d["q"], d["nk"], d["nv"], d["kc"], d["vc"], d["qs"], mql, d["bt"], d["sl"],
                                   w.scale, out=out, slot_mapping=slots, workspace=ws_step, partition_tokens=P,
                                   stream=stream, **sc)

    def step_timed(ev):
        # the same step through its three entry points (the slot mapping
        # also writes the longest-first schedule), events around the attention
        d = copies[turn[0] % len(copies)]
        turn[0] += 1
        pkv.multi_token_slot_mapping(d["bt"], d["sl"], d["qs"], w.rows, mql, w.B, out=slots, schedule=sched,
                                     stream=stream)
        pkv.multi_token_append(d["nk"], d["nv"], d["qs"], mql, d["bt"], d["sl"], d["kc"], d["vc"], stream=stream, **sc)
        ev[0].record(stream)
        pkv.paged_multi_token_attention(d["q"], d["qs"], mql, d["kc"], d["vc"], d["bt"], d["sl"], w.scale, out=out,
                                        workspace=ws, partition_tokens=P, schedule=sched, stream=stream, **sc)
        ev[1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(args.steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(end) / args.steps
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for e in evs:
        step_timed(e)
    torch.cuda.synchronize()
    attn_ms = np.array([a.elapsed_time(b) for a, b in evs])
    t = float(attn_ms.mean()) / 1e3
    nbytes, flops = multi_token_counts(w)
    peak_tf = MFMA_F32_PEAK_TFLOPS if w.dtype == "f32" else MFMA_BF16_PEAK_TFLOPS
    ridge = peak_tf * 1e12 / (HBM_PEAK_GBPS * 1e9)  # flop per byte where the two roofs meet
    if flops / nbytes < ridge:
        roof = {"bound": "hbm", "achieved": round(nbytes / t / 1e9, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(nbytes / t / 1e9 / HBM_PEAK_GBPS, 4)}
    else:
        roof = {"bound": "mfma", "achieved": round(flops / t / 1e12, 2), "peak": peak_tf, "unit": "TFLOP/s",
                "frac": round(flops / t / 1e12 / peak_tf, 4)}
    which = pkv.multi_token_kernel(d0["q"], d0["kc"], d0["vc"], d0["bt"], mql, P)
    roof.update({"traffic": None, "kernel": "paged_multi_token_attention: " + (
                     "unpartitioned kernel (128 rows per work-group, whole visible context)" if which == "unpartitioned"
                     else "partition kernel (16-row causal tiles)" + (" + chunk merge kernel" if ws is not None else "")),
                 "algorithmic_bytes_per_launch": nbytes, "algorithmic_flops_per_launch": flops,
                 "arithmetic_intensity": round(flops / nbytes, 2), "ridge_flop_per_byte": round(ridge, 1),
                 "attained_tflops": round(flops / t / 1e12, 2), "attained_gbps": round(nbytes / t / 1e9, 1),
                 "launch_us": {"mean": round(t * 1e6, 2), "median": round(float(np.median(attn_ms)) * 1e3, 2)}})
    if roof["bound"] == "hbm":
        sr = stream_read_ceiling(torch, pkv)
        roof.update({"stream_read": sr, "frac_of_stream_read": round(nbytes / t / 1e9 / sr["gbps"], 4)})
    return {"metric": "multi-token paged attention query tokens/s (chunked prefill / speculative decoding step)",
            "value": round(w.rows / (ms_step / 1e3), 1), "unit": "query tokens/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None,
            "dtype": {"f32": "f32", "bf16": "bf16", "fp8": "fp8-e4m3 pools, bf16 q/out"}[w.dtype],
            "data": "synthetic (seeded N(0,1) q/K/V, shuffled block IDs; no dataset)",
            "config": {"workload": f"{w.description}; last min({args.q_len}, L) tokens of each sequence are query "
                                   f"rows", "q_len": args.q_len, "query_rows": w.rows, "max_q_len": mql,
                       "partition_tokens": P, "kv_bytes_per_step": w.kv_read_bytes()},
            "kv_read_gbps_step": round(w.kv_read_bytes() / (ms_step / 1e3) / 1e9, 1),
            "roofline": roof,
            "cpu_baseline": None if args.no_cpu_baseline else cpu_baseline_multi_token(w, args.cpu_seconds)}


def cpu_baseline_multi_token(w, target_s: float) -> dict:
    """The CPU oracle's causal attention on whole sequences of the workload,
    one at a time in batch order, until about target_s seconds have passed;
    query rows per second."""
    import oracle

    log("timing the CPU oracle sample")
    rows = 0
    done = 0
    t0 = time.perf_counter()
    for s in range(w.S):
        a, b = int(w.q_start[s]), int(w.q_start[s + 1])
        if a == b:
            continue
        oracle.paged_multi_token_attention(w.q[a:b], np.array([0, b - a], np.int32), w.k_cache, w.v_cache,
                                           w.block_tables[s:s + 1], w.seq_lens[s:s + 1], w.scale,
                                           k_scale=w.k_scale, v_scale=w.v_scale)
        rows += b - a
        done += 1
        if time.perf_counter() - t0 >= target_s:
            break
    el = time.perf_counter() - t0
    return {"value": round(rows / el, 2), "unit": "query tokens/s", "cores": int(oracle.max_threads()),
            "kind": "oracle", "sample": f"causal attention of the first {done} sequences' {rows} query rows (all "
                                        f"{w.Hq} heads), fp64 C oracle with OpenMP, {el:.1f} s wall"}


def calib_copy(mib: int) -> None:
    import torch

    n = mib * (1 << 20)
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    for _ in range(20):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calib_copy_bytes": n, "launches": 20}))


def bench_copy_blocks(args, w, torch, pkv) -> dict:
    """pkv_copy_blocks of args.copy_blocks (src, dst) pairs (distinct dsts, none a src) drawn from the pool:
    algorithmic bytes per launch = pairs x 2 pools x block bytes x 2 (read and write)."""
    copies = [device_inputs(w, torch) for _ in range(max(1, args.rotate))]
    n = args.copy_blocks
    if 2 * n > w.num_blocks:
        raise SystemExit(f"--copy-blocks {n}: the pool has only {w.num_blocks} blocks")
    perm = np.random.default_rng(12345).permutation(w.num_blocks)
    pairs = torch.tensor(np.stack([perm[:n], perm[n:2 * n]], axis=1).astype(np.int32), device="cuda")
    stream = torch.cuda.current_stream()
    elem = w.elem_bytes
    block_bytes = w.Hkv * w.B * w.hs * elem
    moved = n * 2 * block_bytes * 2
    turn = [0]

    def once():
        d = copies[turn[0] % len(copies)]
        turn[0] += 1
        pkv.copy_blocks(pairs, d["kc"], d["vc"], stream=stream)

    for _ in range(args.warmup):
        once()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    for a, b in evs:
        a.record(stream)
        once()
        b.record(stream)
    torch.cuda.synchronize()
    ms = np.array([a.elapsed_time(b) for a, b in evs])
    t = float(ms.mean()) / 1e3
    gbps = moved / t / 1e9
    # ceiling: a plain device-to-device copy of the same bytes (half read, half written) in the same run
    half = moved // 2
    csrc = torch.empty(half, dtype=torch.uint8, device="cuda")
    cdst = torch.empty_like(csrc)
    csrc.fill_(1)
    for _ in range(3):
        cdst.copy_(csrc)
    cev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(20)]
    torch.cuda.synchronize()
    for a, b in cev:
        a.record(stream)
        cdst.copy_(csrc)
        b.record(stream)
    torch.cuda.synchronize()
    copy_gbps = moved / (float(np.mean([a.elapsed_time(b) for a, b in cev])) / 1e3) / 1e9
    del csrc, cdst
    return {"metric": "block copy GB/s (bytes read + written by pkv_copy_blocks)", "value": round(gbps, 1),
            "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(t * 1e3, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": {"f32": "f32", "bf16": "bf16", "fp8": "fp8-e4m3 pools, bf16 q/out"}[w.dtype], "data": "synthetic",
            "config": {"workload": f"block copy in the pool of: {w.description}", "pairs": n,
                       "block_bytes_per_pool": block_bytes},
            "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": None,
                         "device_copy": round(copy_gbps, 1), "frac_of_device_copy": round(gbps / copy_gbps, 4),
                         "kernel": "copy_blocks_kernel", "algorithmic_bytes_per_launch": moved,
                         "launch_us": {"mean": round(t * 1e6, 2), "median": round(float(np.median(ms)) * 1e3, 2)}},
            "cpu_baseline": None}


SWEEP_BLOCK_SIZES = (1, 8, 16, 32, 64)


def time_attention(w, torch, pkv, steps: int, warmup: int, rotate: int) -> np.ndarray:
    """Per-launch microseconds of paged_decode_attention on the workload
    (after its decode append with the longest-first schedule), bracketed by
    events on the launch stream."""
    copies = [device_inputs(w, torch) for _ in range(max(1, rotate))]
    d0 = copies[0]
    P = w.partition_tokens
    ws = pkv.alloc_workspace(d0["q"], d0["kc"], d0["vc"], d0["bt"], P)
    sched = pkv.alloc_schedule(d0["bt"])
    out = torch.empty_like(d0["q"])
    slots = torch.empty(w.S, dtype=torch.int64, device="cuda")
    stream = torch.cuda.current_stream()
    sc = dict(k_scale=w.k_scale, v_scale=w.v_scale)

    def one(i, ev=None):
        d = copies[i % len(copies)]
        pkv.decode_append(d["nk"], d["nv"], d["bt"], d["sl"], d["kc"], d["vc"], slot_mapping=slots, schedule=sched,
                          stream=stream, **sc)
        if ev:
            ev[0].record(stream)
        pkv.paged_decode_attention(d["q"], d["kc"], d["vc"], d["bt"], d["sl"], w.scale, out=out, workspace=ws,
                                   partition_tokens=P, schedule=sched, stream=stream, **sc)
        if ev:
            ev[1].record(stream)

    for i in range(warmup):
        one(i)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    for i, e in enumerate(evs):
        one(i, e)
    torch.cuda.synchronize()
    us = np.array([a.elapsed_time(b) * 1e3 for a, b in evs])
    del copies
    torch.cuda.empty_cache()
    return us


def bench_block_size_sweep(args, torch, pkv, pi) -> dict:
    """The configuration's attention at each block size: KV-read GB/s with
    shuffled block IDs (paged) and with each sequence's blocks adjacent
    (contiguous), plus the share of allocated slots that hold tokens."""
    rows = []
    cfg = args.config if args.config is not None else 3
    for B in SWEEP_BLOCK_SIZES:
        row = {"block_size": B}
        for layout in ("paged", "contiguous"):
            w = pi.make_workload(cfg, mode="timing", B=B, contiguous=(layout == "contiguous"))
            us = time_attention(w, torch, pkv, args.steps, args.warmup, args.rotate)
            gbps = w.kv_read_bytes() / (us.mean() * 1e-6) / 1e9
            row[layout] = {"attention_us": round(float(us.mean()), 2), "median_us": round(float(np.median(us)), 2),
                           "kv_read_gbps": round(gbps, 1), "frac_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4)}
            log(f"B={B} {layout}: {us.mean():.1f} us, {gbps:.0f} GB/s")
            if layout == "paged":
                nblk = -(-w.seq_lens.astype(np.int64) // B)
                row["slot_utilisation"] = round(float(w.seq_lens.sum() / (nblk.sum() * B)), 5)
                row["partition_tokens"] = int(pkv.decode_partition_tokens(w.S, w.Hq, w.Hkv, w.hs, w.M, B, 0))
                desc = w.description
                kvb = w.kv_read_bytes()
            del w
        row["paged_over_contiguous"] = round(row["paged"]["attention_us"] / row["contiguous"]["attention_us"], 4)
        rows.append(row)
    best = max(rows, key=lambda r: r["paged"]["kv_read_gbps"])
    return {"metric": "paged decode attention KV-read GB/s per block size (block-size trade-off)",
            "value": best["paged"]["kv_read_gbps"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(best["paged"]["attention_us"] / 1e3, 5),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic (seeded N(0,1) q/K/V; no dataset)",
            "config": {"workload": f"{desc}, block size swept", "block_sizes": list(SWEEP_BLOCK_SIZES),
                       "kv_bytes_per_launch": kvb, "best_block_size": best["block_size"]},
            "sweep": rows, "roofline": {"bound": "hbm", "achieved": best["paged"]["kv_read_gbps"],
                                        "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                                        "frac": best["paged"]["frac_hbm_peak"], "traffic": None,
                                        "kernel": "paged_decode_attention at the best block size"},
            "cpu_baseline": None}


def kernel_sources_sha256(paths) -> str:
    import hashlib

    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(path, config: int, partition_tokens: int, contiguous: bool, kv_dtype: str = "native"):
    """HBM bytes per attention launch from a counter record, or None when the
    record is missing or was taken on another workload (configuration, pool
    dtype, partition length) or another version of the kernel sources."""
    if not path or not os.path.isfile(path) or contiguous:
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("config") != config or rec.get("partition_tokens") != partition_tokens:
        return None
    if rec.get("kv_dtype", "native") != kv_dtype:
        return None
    if rec.get("kernel_sources_sha256") != kernel_sources_sha256(rec.get("kernel_sources", [])):
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(w, target_s: float, gpu=None) -> dict:
    """Time the CPU oracle (fp64, as it stands) on the workload's attention:
    whole passes over every (sequence, query head), repeated until about
    target_s seconds of wall time have passed.  gpu: (out, k_cache, v_cache)
    of the timed GPU run on the same inputs; its output is then compared with
    the last pass's and its pools with the oracle's appended pools, byte for
    byte (returned under "parity")."""
    import oracle

    slots = oracle.decode_slot_mapping(w.block_tables, w.seq_lens, w.B)
    kp, vp = w.k_cache.copy(), w.v_cache.copy()
    if w.dtype == "fp8":
        oracle.kv_append_fp8(w.new_k, w.new_v, slots, kp, vp, oracle.fp8_inv_scale(w.k_scale),
                             oracle.fp8_inv_scale(w.v_scale))
    else:
        oracle.kv_append(w.new_k, w.new_v, slots, kp, vp)
    passes = 0
    used = oracle.max_threads()
    t0 = time.perf_counter()
    while True:
        if w.dtype == "fp8":
            ref = oracle.paged_attention_fp8(w.q, kp, vp, w.block_tables, w.seq_lens, w.scale, w.k_scale, w.v_scale)
        else:
            ref, used = oracle.paged_attention(w.q, kp, vp, w.block_tables, w.seq_lens, w.scale,
                                               return_threads=True)
        passes += 1
        if time.perf_counter() - t0 >= target_s:
            break
    el = time.perf_counter() - t0
    bytes_read = passes * w.kv_read_bytes()
    res = {"value": round(bytes_read / el / 1e9, 4), "unit": "GB/s", "cores": int(used), "kind": "oracle",
           "sample": f"{passes} full passes of the workload's attention (all {w.S} sequences x {w.Hq} query "
                     f"heads), fp64 C oracle with OpenMP, {el:.1f} s wall on {used} threads; "
                     f"same KV-byte accounting as value"}
    if gpu is not None:
        import torch

        out, kc, vc = gpu

        def host_bytes(t):
            return (t.view(torch.int16) if t.dtype == torch.bfloat16 else t).cpu().numpy().tobytes()

        err = float(np.abs(out.float().cpu().numpy().astype(np.float64) - ref).max())
        tol = 1e-5 if w.dtype == "f32" else 2e-3
        res["parity"] = {
            "max_abs_err": err, "tolerance": tol, "within_tolerance": err <= tol,
            "append_bit_exact": host_bytes(kc) == np.ascontiguousarray(kp).tobytes()
            and host_bytes(vc) == np.ascontiguousarray(vp).tobytes(),
            "checked": "the timed run's output (every sequence and query head) against the last oracle pass, "
                       "and both pools of its first input copy byte for byte against the oracle's append"}
    return res


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo; lscpu is not always there)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform

    return platform.processor() or "unknown"


def single_thread_passes(pi, seed_of) -> dict:
    """One whole pass of the oracle's attention on one host thread, for the
    tiny fp32 configuration and the MHA configuration (the CPU baseline's
    per-core figure, beside its all-thread rate)."""
    import oracle

    res = {}
    for c in (1, 2):
        w = pi.make_workload(c, mode="timing", seed=seed_of(c))
        t0 = time.perf_counter()
        oracle.paged_attention(w.q, w.k_cache, w.v_cache, w.block_tables, w.seq_lens, w.scale, threads=1)
        el = time.perf_counter() - t0
        res[f"config{c}"] = {"pass_s": round(el, 4), "kv_gbps": round(w.kv_read_bytes() / el / 1e9, 4),
                             "decode_tokens_per_s": round(w.S / el, 1)}
        del w
    return res


def contiguous_tables(w) -> np.ndarray:
    """The workload's block tables with each sequence's blocks renumbered to
    adjacent IDs (sequence after sequence from block 0): the same kernel and
    sizes on contiguous storage, for the paged-vs-contiguous diagnostic (the
    timing does not depend on the values the blocks hold).  None when the
    pool cannot hold every sequence's blocks apart (shared blocks)."""
    nblk = -(-np.clip(w.seq_lens.astype(np.int64), 0, None) // w.B)
    if int(nblk.sum()) > w.num_blocks:
        return None
    base = np.concatenate([[0], np.cumsum(nblk)[:-1]])
    t = np.full_like(w.block_tables, w.block_tables[0, 0])
    for s in range(w.S):
        t[s, :nblk[s]] = base[s] + np.arange(nblk[s])
    return t.astype(np.int32)


def bench_decode(args, config: int, torch, pkv, pi, sr: dict, seed: int) -> dict:
    """The decode step of one configuration: K timed steps (an event after
    each, for the per-step spread), the same steps through the append and
    attention entry points with events around each launch, a graph replay,
    the roofline of the attention call, the CPU oracle baseline with a
    full-size parity check of the timed run, and the paged-vs-contiguous
    diagnostic.  Returns the configuration's record."""
    t0 = time.perf_counter()
    kvdt = "fp8" if args.kv_dtype == "fp8" else None
    bkw = {"B": args.block_size} if args.block_size else {}
    w = pi.make_workload(config, mode="timing", contiguous=args.contiguous, dtype=kvdt, seed=seed, **bkw)
    sc = dict(k_scale=w.k_scale, v_scale=w.v_scale)
    log(f"generated config {config} ({w.description}) in {time.perf_counter() - t0:.1f} s")
    P = w.partition_tokens if args.partition_tokens is None else args.partition_tokens
    copies = [device_inputs(w, torch) for _ in range(max(1, args.rotate))]
    d0 = copies[0]
    ws_step = pkv.alloc_step_workspace(d0["q"], d0["kc"], d0["vc"], d0["bt"], P)
    ws = pkv.alloc_workspace(d0["q"], d0["kc"], d0["vc"], d0["bt"], P)
    sched = pkv.alloc_schedule(d0["bt"])
    out = torch.empty_like(d0["q"])
    slots = torch.empty(w.S, dtype=torch.int64, device="cuda")
    stream = torch.cuda.current_stream()
    P_used = pkv.decode_partition_tokens(w.S, w.Hq, w.Hkv, w.hs, w.M, w.B, P)
    turn = [0]

    # batches of up to ONE_LAUNCH_MAX_SEQS sequences: the step is one launch
    # (attention plus the stores of the new tokens; a chunk merge launch
    # where the sequences are split)
    one_launch = w.S <= ONE_LAUNCH_MAX_SEQS

    def step():
        # one decode step: slot of each sequence's new token (from its block
        # table) and the append of its K/V, and the attention (plus the chunk
        # merge where needed); larger batches: the append launch also writes
        # the longest-first schedule, then the attention launch
        d = copies[turn[0] % len(copies)]
        turn[0] += 1
        pkv.paged_decode_step(d["q"], d["nk"], d["nv"], d["kc"], d["vc"], d["bt"], d["sl"], w.scale, out=out,
                              slot_mapping=slots, workspace=ws_step, partition_tokens=P, stream=stream, **sc)

    def step_timed(ev, tables=None):
        # the same step with events around its launches: a one-launch step
        # whole (ev[0] .. ev[1], no separate append), else through the two
        # entry points it is made of, with events around the append launch
        # and around the attention launch
        d = copies[turn[0] % len(copies)]
        turn[0] += 1
        bt = d["bt"] if tables is None else tables
        if one_launch:
            ev[2].record(stream)
            ev[0].record(stream)
            pkv.paged_decode_step(d["q"], d["nk"], d["nv"], d["kc"], d["vc"], bt, d["sl"], w.scale, out=out,
                                  slot_mapping=slots, workspace=ws_step, partition_tokens=P, stream=stream, **sc)
            ev[1].record(stream)
            return
        ev[2].record(stream)
        pkv.decode_append(d["nk"], d["nv"], bt, d["sl"], d["kc"], d["vc"], slot_mapping=slots, schedule=sched,
                          stream=stream, **sc)
        ev[0].record(stream)
        pkv.paged_decode_attention(d["q"], d["kc"], d["vc"], bt, d["sl"], w.scale, out=out, workspace=ws,
                                   partition_tokens=P, schedule=sched, stream=stream, **sc)
        ev[1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: K whole steps, an event before the first and after each
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    marks[0].record(stream)
    for i in range(args.steps):
        step()
        marks[i + 1].record(stream)
    torch.cuda.synchronize()
    ms_step = marks[0].elapsed_time(marks[-1]) / args.steps
    step_ms = np.array([marks[i].elapsed_time(marks[i + 1]) for i in range(args.steps)])

    # the attention call alone, bracketed by events on the same stream
    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    for e in evs:
        step_timed(e)
    torch.cuda.synchronize()
    attn_ms = np.array([e[0].elapsed_time(e[1]) for e in evs])
    append_ms = np.array([e[2].elapsed_time(e[0]) for e in evs])
    log(f"config {config}: {args.steps} steps, {ms_step * 1e3:.1f} us/step, attention median "
        f"{np.median(attn_ms) * 1e3:.1f} us")

    # the same steps replayed from a HIP graph (one step per input copy),
    # as a serving loop would run them: reported beside the eager figure
    graph_info = None
    if not args.no_graph:
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                for d in copies:
                    pkv.paged_decode_step(d["q"], d["nk"], d["nv"], d["kc"], d["vc"], d["bt"], d["sl"], w.scale,
                                          out=out, slot_mapping=slots, workspace=ws_step, partition_tokens=P,
                                          stream=side, **sc)
        torch.cuda.synchronize()
        reps = max(1, args.steps // len(copies))
        for _ in range(2):
            g.replay()
        # replay() launches on the current stream: time it there
        ga, gb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        ga.record(stream)
        for _ in range(reps):
            g.replay()
        gb.record(stream)
        torch.cuda.synchronize()
        g_ms = ga.elapsed_time(gb) / (reps * len(copies))
        graph_info = {"ms_per_step": round(g_ms, 5), "kv_read_gbps": round(w.kv_read_bytes() / (g_ms / 1e3) / 1e9, 1),
                      "steps": reps * len(copies)}
        del g
        log(f"config {config}: graph replay {g_ms * 1e3:.1f} us/step")

    kv_bytes = w.kv_read_bytes()
    attn_avg_s = float(attn_ms.mean()) / 1e3
    achieved = kv_bytes / attn_avg_s / 1e9
    record = TRAFFIC_RECORDS.get((config, "fp8") if w.dtype == "fp8" else config, "")
    traffic_path = args.traffic or os.path.join(ROOT, "profiles", record)
    traffic = None if (args.block_size or seed != config) else measured_traffic(
        traffic_path, config, P_used, args.contiguous, "fp8" if w.dtype == "fp8" else "native")
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                "kernel": (("paged_decode_step in one launch: paged_decode_partition_kernel with the new tokens' "
                            "stores" + (" (one chunk per sequence, no merge launch)" if ws is None else
                                        " + chunk merge kernel"))
                           if one_launch else
                           "paged_decode_attention with the step's longest-first schedule: "
                           "paged_decode_partition_kernel alone (one chunk per sequence, no merge launch)"
                           if ws is None else
                           "paged_decode_attention with the step's longest-first schedule: partition kernel + "
                           "chunk merge kernel"),
                "algorithmic_bytes_per_launch": kv_bytes,
                "launch_us": {"mean": round(attn_avg_s * 1e6, 2), "median": round(float(np.median(attn_ms)) * 1e3, 2),
                              "p10": round(float(np.percentile(attn_ms, 10)) * 1e3, 2),
                              "p90": round(float(np.percentile(attn_ms, 90)) * 1e3, 2)}}
    # shared blocks (a shared prefix): the distinct bytes read, beside the logical ones
    unique = w.unique_kv_bytes()
    if unique < kv_bytes:
        roofline.update({"unique_bytes_per_launch": unique,
                         "achieved_unique_gbps": round(unique / attn_avg_s / 1e9, 1)})
    roofline.update({"stream_read": sr, "frac_of_stream_read": round(achieved / sr["gbps"], 4)})
    # the same tiles read by the gather-read probe alone: the ceiling of this
    # access pattern (frac = the probe's time over the launch's time).  Not
    # for shared blocks: the probe reads each branch's copy of the prefix at
    # another time, so it gets less from the caches than the attention does
    gr = None if (args.contiguous or unique < kv_bytes) else gather_read_ceiling(torch, pkv, w, copies)
    if gr is not None:
        roofline.update({"gather_read": gr, "frac_of_gather_read": round(achieved / gr["gbps_algorithmic"], 4)})
        log(f"config {config}: gather-read probe {gr['gbps']} GB/s over {gr['tiles']} tiles ({gr['us']} us)")
    cpu = None
    if not args.no_cpu_baseline:
        log(f"config {config}: timing the CPU oracle sample")
        cpu = cpu_baseline(w, args.cpu_seconds, gpu=(out, copies[0]["kc"], copies[0]["vc"]))
        log(f"config {config}: CPU oracle {cpu['value']} GB/s; parity {cpu.get('parity', {}).get('max_abs_err')}")

    # paged vs contiguous storage: the same attention launch with each
    # sequence's blocks renumbered adjacent (after the parity check, since
    # the appends through these tables write other slots)
    contig = None
    ct_host = None if (args.contiguous or args.no_contiguous_diag) else contiguous_tables(w)
    if ct_host is None and not (args.contiguous or args.no_contiguous_diag):
        contig = {"skipped": "the tables share blocks: their blocks cannot all be laid out apart in this pool"}
    if ct_host is not None:
        ct = torch.from_numpy(ct_host).cuda()
        cevs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(args.steps)]
        for _ in range(max(2, args.warmup)):
            step_timed(tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)), ct)
        torch.cuda.synchronize()
        for e in cevs:
            step_timed(e, ct)
        torch.cuda.synchronize()
        c_ms = np.array([e[0].elapsed_time(e[1]) for e in cevs])
        contig = {"contiguous_attention_us": round(float(c_ms.mean()) * 1e3, 2),
                  "paged_attention_us": round(attn_avg_s * 1e6, 2),
                  "paged_over_contiguous": round(attn_avg_s * 1e3 / float(c_ms.mean()), 4)}
        del ct

    value = kv_bytes / (ms_step / 1e3) / 1e9
    rec = {
        "value": round(value, 1),
        "ms_per_step": round(ms_step, 5),
        "step_us": {"p10": round(float(np.percentile(step_ms, 10)) * 1e3, 2),
                    "median": round(float(np.median(step_ms)) * 1e3, 2),
                    "p90": round(float(np.percentile(step_ms, 90)) * 1e3, 2)},
        "dtype": {"f32": "f32", "bf16": "bf16", "fp8": "fp8-e4m3 pools, bf16 q/out"}[w.dtype],
        "config": {"workload": w.description + (" [contiguous block order]" if args.contiguous else ""),
                   "config": config, "seed": w.seed, "num_seqs": w.S, "input_copies": len(copies),
                   "q_heads": w.Hq, "kv_heads": w.Hkv, "head_size": w.hs, "block_size": w.B,
                   "pool_blocks": w.num_blocks, "sum_seq_len": int(w.seq_lens.sum()),
                   "partition_tokens": P_used, "kv_bytes_per_step": kv_bytes},
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "decode_tokens_per_s": round(w.S / (ms_step / 1e3), 1),
        "attention_calls_per_s": round(1.0 / attn_avg_s, 1),
        "append_us": ("inside the attention launch" if one_launch else
                      {"mean": round(float(append_ms.mean()) * 1e3, 2),
                       "median": round(float(np.median(append_ms)) * 1e3, 2)}),
        "graph_replay": graph_info,
        "paged_vs_contiguous": contig,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    del copies, d0, ws_step, ws, sched, out, slots, w
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return rec


METRIC = "paged decode attention KV-read GB/s (% of HBM peak) + decode tokens/s, 1 GPU"
DATA = "synthetic (seeded N(0,1) q/K/V, shuffled block IDs; no dataset)"
# the default run: one decode step of each of the three layers the >= 70 %
# bandwidth target names (MHA, GQA, long context)
DEFAULT_CONFIGS = (2, 3, 4)


def main() -> int:
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); this build has no multi-GPU path",
              file=sys.stderr)
        return 2
    import torch

    if args.calib_copy:
        calib_copy(args.calib_copy)
        return 0

    import paged_kv_cache_35_amd as pkv
    import pkv_inputs as pi

    pkv.library()
    torch.cuda.set_device(0)
    t0 = time.perf_counter()
    kvdt = "fp8" if args.kv_dtype == "fp8" else None
    seed_of = (lambda c: c) if args.seed is None else (lambda c: args.seed)
    if args.block_size_sweep:
        print(json.dumps(bench_block_size_sweep(args, torch, pkv, pi)), flush=True)
        return 0
    bkw = {"B": args.block_size} if args.block_size else {}
    single = args.config if args.config is not None else (None if not (args.q_len or args.copy_blocks) else 2)
    if args.q_len:
        base = pi.make_workload(single, mode="timing", contiguous=args.contiguous, dtype=kvdt, seed=seed_of(single),
                                **bkw)
        q_lens = np.minimum(args.q_len, base.seq_lens)
        del base
        w = pi.make_workload(single, mode="timing", contiguous=args.contiguous, dtype=kvdt, q_lens=q_lens,
                             seed=seed_of(single), **bkw)
        log(f"generated config {single} with {w.rows} query rows in {time.perf_counter() - t0:.1f} s")
        print(json.dumps(bench_multi_token(args, w, torch, pkv)), flush=True)
        return 0
    if args.copy_blocks:
        w = pi.make_workload(single, mode="timing", dtype=kvdt, seed=seed_of(single), **bkw)
        print(json.dumps(bench_copy_blocks(args, w, torch, pkv)), flush=True)
        return 0

    # the measured read ceiling of this GPU, beside the 8 TB/s peak (once)
    sr = stream_read_ceiling(torch, pkv)
    log(f"streaming-read ceiling {sr['gbps']} GB/s")
    configs = [single] if single is not None else list(DEFAULT_CONFIGS)
    recs = {c: bench_decode(args, c, torch, pkv, pi, sr, seed_of(c)) for c in configs}
    common = {"metric": METRIC, "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
              "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "data": DATA}
    if single is not None:
        r = recs[single]
        out = {"metric": METRIC, "value": r["value"], **{k: v for k, v in common.items() if k != "metric"}}
        out.update({k: v for k, v in r.items() if k != "value"})
        if out["cpu_baseline"] is not None:
            out["cpu_baseline"]["cpu_model"] = cpu_model()
        print(json.dumps(out), flush=True)
        return 0

    # one step = one decode step of each configuration, in turn: the whole
    # job's KV bytes over the sum of the step times
    kv_total = sum(r["config"]["kv_bytes_per_step"] for r in recs.values())
    ms_total = sum(r["ms_per_step"] for r in recs.values())
    value = kv_total / (ms_total / 1e3) / 1e9
    # the dominant kernel: the attention call that takes longest
    dom = max(configs, key=lambda c: recs[c]["roofline"]["launch_us"]["mean"])
    roof = dict(recs[dom]["roofline"])
    roof["kernel"] = f"configuration {dom}: " + roof["kernel"]
    roof["config"] = dom
    cpu = None
    if not args.no_cpu_baseline:
        cb = [recs[c]["cpu_baseline"] for c in configs]
        # seconds per oracle pass of each configuration, summed like the GPU steps
        sec = sum(recs[c]["config"]["kv_bytes_per_step"] / (cb[i]["value"] * 1e9) for i, c in enumerate(configs))
        cpu = {"value": round(kv_total / sec / 1e9, 4), "unit": "GB/s", "cores": cb[0]["cores"], "kind": "oracle",
               "sample": "whole oracle passes over every sequence and query head of each configuration (about "
                         f"{args.cpu_seconds:.0f} s of wall time each), fp64 C oracle with OpenMP; the rate of one "
                         "pass of each configuration in turn, in the same KV-byte accounting as value",
               "cpu_model": cpu_model(),
               "per_config": {str(c): {"value": cb[i]["value"], "sample": cb[i]["sample"]}
                              for i, c in enumerate(configs)},
               "parity": {str(c): cb[i].get("parity") for i, c in enumerate(configs)}}
        log("timing single-thread oracle passes (configurations 1 and 2)")
        cpu["single_thread"] = single_thread_passes(pi, seed_of)
    names = {2: "MHA", 3: "GQA", 4: "long-context"}
    step_p = {k: round(sum(recs[c]["step_us"][k] for c in configs), 2) for k in ("p10", "median", "p90")}
    out = {"metric": METRIC, "value": round(value, 1), **{k: v for k, v in common.items() if k != "metric"},
           "ms_per_step": round(ms_total, 5),
           "dtype": recs[configs[0]]["dtype"],
           "config": {"workload": "one decode step (append + paged attention) of each of three layers in turn: "
                                  + "; ".join(f"{names.get(c, c)} {recs[c]['config']['workload']}" for c in configs),
                      "configs": configs, "seeds": [recs[c]["config"]["seed"] for c in configs],
                      "kv_bytes_per_step": kv_total},
           "pct_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
           "step_us_sum_of_percentiles": step_p,
           "decode_tokens_per_s": {str(c): recs[c]["decode_tokens_per_s"] for c in configs},
           "roofline": roof,
           "cpu_baseline": cpu,
           "per_config": {str(c): recs[c] for c in configs}}
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
