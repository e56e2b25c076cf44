#!/usr/bin/env python3
"""Benchmark of the paged-attention library on one MI355X.

Default workload: the Llama-3-8B-shaped decode batch -- 64 sequences, 32 query heads on 8 KV
heads (head_dim 128), block size 16, bf16, context lengths uniform in [512, 4096], physical
blocks shuffled over a pool 10% larger than needed. One step is one pass of the hot path over
that batch: kv_cache_write of the 64 new tokens' K/V, then paged_attention_decode (partition
kernel, plus the reduce kernel when the context is split).

    python bench.py [--steps K] [--warmup W] [--workload decode-8b|decode-70b|shared-prefix|prefill-chunk]
    python bench.py --workload cow-fork|block-copy|swap-out|swap-in      # block copies

Prints ONE JSON line on stdout. Inputs are resident in HBM before timing starts. Steps rotate
over --replicas copies of the pools (so no step re-reads what the previous step left in the
256 MB Infinity Cache); every copy holds the same data. The dominant kernel's average duration
is measured live with the library's own HIP events, recorded on the stream each kernel runs on,
over the timed region. The CPU baseline times the oracle (float64 NumPy, one thread) on a
bounded sample of the same batch.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
COPY_BYTES = 256 << 20          # calibration copy: reads and writes this many bytes
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak

WORKLOADS = {
    "decode-8b": 2,
    "decode-70b": 3,
    "shared-prefix": 4,
    "prefill-chunk": 5,
    # the same decode batches with E4M3 (one byte per element) pools, per-pool scale 1/16
    "decode-8b-fp8": 2,
    "decode-70b-fp8": 3,
    # the shared-prefix batch through the prefix-aware decode (prefix read once per KV head)
    "shared-prefix-grouped": 4,
    "shared-prefix-grouped-fp8": 4,
    # the decode batches through the fused write-and-decode call (one launch per step)
    "decode-8b-fused": 2,
    "decode-70b-fused": 3,
    # one GPU's share of the 70B-shaped batch split by KV head over 8 GPUs: 1 KV head, 8 query
    # heads, the same sequences (what each GPU runs under 8-way tensor parallelism)
    "decode-70b-tp8": 3,
}
# Block-copy workloads, all on the decode-8b pool: copy-on-write of one block per sequence (a
# fork of every sequence), a device-to-device migration of the blocks of half the sequences,
# and the swap-out / swap-in of those blocks to / from pinned host memory.
BLOCK_WORKLOADS = ("cow-fork", "block-copy", "swap-out", "swap-in")
PCIE_PEAK_GBS = 64.0           # PCIe 5.0 x16, one direction (32 GT/s x 16 lanes)


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# ------------------------------------------------------------------------- algorithmic work

def _pool_esz(w):
    return {"fp8": 1, "bf16": 2, "f32": 4}[w.pool_dtype]


def decode_bytes(w):
    """Bytes the decode method must move: every context token's K and V row for every KV head,
    q read, out written, one block id per (sequence, block), one context length per sequence."""
    esz = 2 if w.dtype == "bf16" else 4
    n = w.context_lens.astype("int64")
    kv = int(n.sum()) * 2 * w.num_kv_heads * w.head_dim * _pool_esz(w)
    q = w.num_seqs * w.num_q_heads * w.head_dim * esz
    ids = int(((n + w.block_size - 1) // w.block_size).sum()) * 4
    return {"kv": kv, "q": q, "out": q, "ids": ids, "ctx": 4 * w.num_seqs}


def unique_decode_kv_bytes(w):
    """KV bytes counting the shared-prefix blocks once (what HBM must deliver at least)."""
    n = w.context_lens.astype("int64")
    per_tok = 2 * w.num_kv_heads * w.head_dim * _pool_esz(w)
    if not w.prefix_tokens:
        return int(n.sum()) * per_tok
    return (w.prefix_tokens + int((n - w.prefix_tokens).sum())) * per_tok


def write_bytes(w):
    """New rows read (input dtype) and written (pool dtype), K and V, plus the slot list."""
    esz = 2 if w.dtype == "bf16" else 4
    t = int((w.slot_mapping >= 0).sum())
    return 2 * t * w.num_kv_heads * w.head_dim * (esz + _pool_esz(w)) + 4 * len(w.slot_mapping)


def prefill_flops(w):
    """4*D flops (QK^T and PV) per visible (query row, key) pair and query head."""
    total = 0
    for s in range(w.num_seqs):
        c = int(w.cu_q_lens[s + 1] - w.cu_q_lens[s])
        r = int(w.context_lens[s]) - c
        total += c * r + c * (c + 1) // 2
    return 4 * w.head_dim * w.num_q_heads * total


def prefill_bytes(w):
    esz = 2 if w.dtype == "bf16" else 4
    kv = int(w.context_lens.astype("int64").sum()) * 2 * w.num_kv_heads * w.head_dim * esz
    qo = 2 * w.total_q * w.num_q_heads * w.head_dim * esz
    return kv + qo


# ---------------------------------------------------------------------------- device side

def block_sources(w, workload):
    """Source blocks of a block-copy workload: each sequence's last block for cow-fork (the one
    a forked child writes next), else every block of the first half of the sequences."""
    import numpy as np
    b = w.block_size
    nblk = (w.context_lens.astype(np.int64) + b - 1) // b
    if workload == "cow-fork":
        return np.asarray([w.block_table[s, nblk[s] - 1] for s in range(w.num_seqs)], np.int32)
    half = w.num_seqs // 2
    return np.concatenate([w.block_table[s, :nblk[s]] for s in range(half)]).astype(np.int32)


def run_blocks(args, w):
    """Time kv_cache_copy_blocks on the decode-8b pool (see BLOCK_WORKLOADS)."""
    import numpy as np
    import torch

    from paged_kv_cache_190_amd import binding as bd

    dev = torch.device("cuda:0")
    k0, v0 = to_dev(w.k_pool), to_dev(w.v_pool)
    b = w.block_size
    src = block_sources(w, args.workload)
    n = len(src)
    block_bytes = 2 * w.num_kv_heads * b * w.head_dim * 2  # K and V of one block, bf16
    host = args.workload in ("swap-out", "swap-in")
    shape_k = (n, w.num_kv_heads, b, w.head_dim)
    shape_v = (n, w.num_kv_heads, w.head_dim, b)
    if args.workload == "cow-fork":
        free = np.setdiff1d(np.arange(w.num_blocks), w.block_table[w.block_table >= 0])
        pairs = np.stack([src, free[:n].astype(np.int32)], 1)
        ends = (k0, v0, k0, v0)
    else:
        ok = torch.empty(shape_k, dtype=torch.bfloat16, device="cpu" if host else dev,
                         pin_memory=host)
        ov = torch.empty(shape_v, dtype=torch.bfloat16, device="cpu" if host else dev,
                         pin_memory=host)
        out_pairs = np.stack([src, np.arange(n, dtype=np.int32)], 1)
        if args.workload == "swap-in":
            bd.kv_cache_copy_blocks(k0, v0, ok, ov, to_dev(out_pairs))
            pairs, ends = out_pairs[:, ::-1].copy(), (ok, ov, k0, v0)
        else:
            pairs, ends = out_pairs, (k0, v0, ok, ov)
    tp = to_dev(np.ascontiguousarray(pairs))
    log(f"workload {args.workload}: {n} blocks of {block_bytes} B ({n * block_bytes / 1e6:.1f} MB)")

    def step():
        bd.kv_cache_copy_blocks(*ends, tp)

    if args.calibrate_copy:
        calibration_copies(dev)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    def timed(instrument):
        bd.profile_enable(instrument)
        start = torch.cuda.Event(enable_timing=True)
        stop = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record()
        for _ in range(args.steps):
            step()
        stop.record()
        torch.cuda.synchronize()
        ms, cnt = bd.profile_read("copy_blocks") if instrument else (0.0, 0)
        bd.profile_enable(False)
        return start.elapsed_time(stop) / args.steps, (1e3 * ms / cnt if cnt else None)

    ms_per_step, _ = timed(False)
    _, kern_us = timed(True)
    moved = n * block_bytes
    result = {"ms_per_step": round(ms_per_step, 4),
              "kernels": {"copy_blocks": {"avg_us": round(kern_us, 2), "launches": args.steps}},
              "blocks_per_step": n, "bytes_per_block": block_bytes}
    if host:
        # context: the DMA engines copying one contiguous buffer of the same size
        dsrc = torch.empty(moved, dtype=torch.uint8, device=dev)
        hbuf = torch.empty(moved, dtype=torch.uint8, pin_memory=True)
        a, bb = (dsrc, hbuf) if args.workload == "swap-out" else (hbuf, dsrc)
        bb.copy_(a, non_blocking=True)
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(5):
            bb.copy_(a, non_blocking=True)
        t1.record()
        torch.cuda.synchronize()
        result["contiguous_dma_copy_GBs"] = round(5 * moved / (t0.elapsed_time(t1) * 1e-3) / 1e9, 1)
        achieved = moved / (kern_us * 1e-6) / 1e9
        result["roofline"] = {"bound": "pcie", "achieved": round(achieved, 1),
                              "peak": PCIE_PEAK_GBS, "unit": "GB/s",
                              "frac": round(achieved / PCIE_PEAK_GBS, 4), "traffic": None,
                              "kernel": "copy_blocks", "avg_us": round(kern_us, 2),
                              "algorithmic_bytes_per_launch": moved}
        result.update(metric=f"{args.workload} of KV blocks over the host link, GB/s",
                      value=round(moved / (ms_per_step * 1e-3) / 1e9, 2), unit="GB/s")
    else:
        hbm = 2 * moved + 8 * n  # read + write every block, plus the pair list
        achieved = hbm / (kern_us * 1e-6) / 1e9
        result["roofline"] = {"bound": "hbm", "achieved": round(achieved, 1),
                              "peak": HBM_PEAK_GBS, "unit": "GB/s",
                              "frac": round(achieved / HBM_PEAK_GBS, 4),
                              "traffic": traffic_from_profile(args.workload, hbm),
                              "kernel": "copy_blocks", "avg_us": round(kern_us, 2),
                              "algorithmic_bytes_per_launch": hbm}
        result.update(metric=f"{args.workload}: KV block copy HBM GB/s (read + write)",
                      value=round(hbm / (ms_per_step * 1e-3) / 1e9, 1), unit="GB/s")
    return result


def cpu_baseline_blocks(w, src, budget_s):
    """The oracle's block copy timed on the host (one thread), over growing prefixes of the
    same source blocks, copied into a host pool of their own."""
    import numpy as np

    from oracle import paged_attention as orc
    dk = np.empty((len(src),) + w.k_pool.shape[1:], w.k_pool.dtype)
    dv = np.empty((len(src),) + w.v_pool.shape[1:], w.v_pool.dtype)
    local = np.stack([src, np.arange(len(src), dtype=np.int32)], 1)
    t0 = time.perf_counter()
    done = 0
    while done < len(local) and time.perf_counter() - t0 < budget_s:
        orc.kv_cache_copy_blocks(w.k_pool, w.v_pool, dk, dv, local[done:done + 256])
        done = min(done + 256, len(local))
    dt = time.perf_counter() - t0
    per = 2 * w.k_pool[0].nbytes
    return {"value": round(done * per / dt / 1e9, 3), "unit": "GB/s", "cores": 1,
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"oracle block copy of {done} of {len(src)} blocks in calls of 256 "
                      f"({dt:.2f} s, NumPy, one thread); bytes of the blocks copied / time"}

def calibration_copies(dev):
    """Plain device copies of known size, for scaling rocprofv3's byte counters."""
    import torch
    src = torch.ones(COPY_BYTES, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def to_dev(a):
    import numpy as np
    import torch
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


class Replica:
    def __init__(self, w, k_pool, v_pool):
        self.k_pool = k_pool
        self.v_pool = v_pool


def make_workload(args):
    """The seeded synthetic inputs of --workload (host arrays; no GPU involved)."""
    from paged_kv_cache_190_amd import workloads as wl
    if args.workload in BLOCK_WORKLOADS:
        return wl.make_config(WORKLOADS["decode-8b"])
    cfg = WORKLOADS[args.workload]
    fp8 = args.workload.endswith("-fp8")
    tp = 8 if args.workload.endswith("-tp8") else 1
    w = wl.make_config(cfg, kv_dtype="fp8" if fp8 else "", tp=tp)
    log(f"workload {args.workload} ({wl.CONFIG_NAMES[cfg]}): S={w.num_seqs} "
        f"sum(n)={int(w.context_lens.sum())} NB={w.num_blocks}")
    return w


def _percentiles(us):
    import numpy as np
    a = np.asarray(us, dtype=np.float64)
    return {"median": round(float(np.median(a)), 2), "p10": round(float(np.percentile(a, 10)), 2),
            "p90": round(float(np.percentile(a, 90)), 2), "n": int(a.size)}


def run(args, w):
    import numpy as np
    import torch

    from paged_kv_cache_190_amd import binding as bd

    fp8 = args.workload.endswith("-fp8")
    grouped = args.workload.startswith("shared-prefix-grouped")
    fused = args.workload.endswith("-fused")
    dev = torch.device("cuda:0")
    q = to_dev(w.q)
    k_new, v_new = to_dev(w.k_new), to_dev(w.v_new)
    slots, bt, ctx = to_dev(w.slot_mapping), to_dev(w.block_table), to_dev(w.context_lens)
    cu = to_dev(w.cu_q_lens) if w.cu_q_lens is not None else None
    pool_bytes = w.k_pool.nbytes * 2
    replicas = max(1, args.replicas if args.replicas else math.ceil(2e9 / pool_bytes))
    k0, v0 = to_dev(w.k_pool), to_dev(w.v_pool)
    reps = [Replica(w, k0, v0)] + [Replica(w, k0.clone(), v0.clone())
                                   for _ in range(replicas - 1)]
    out = torch.empty(q.shape, dtype=q.dtype, device=dev)
    P = args.partition_size
    if w.kind == "decode":
        code = bd.PKV_BF16 if w.dtype == "bf16" else bd.PKV_F32
        if fp8:
            code = bd.PKV_FP8_E4M3
        need = bd.decode_workspace_size(w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim,
                                        w.max_context_len, P, code)
        if grouped:
            need = bd.decode_shared_prefix_workspace_size(
                w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim, w.max_context_len,
                w.prefix_tokens, code)
            gstart = to_dev(np.asarray([0, w.num_seqs], np.int32))
            gpre = to_dev(np.asarray([w.prefix_tokens], np.int32))
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
        P_eff = 0 if (fp8 or grouped or fused) else bd.decode_partition_size(
            P, w.num_seqs, w.num_kv_heads, w.max_context_len, code)

    nw = args.waves

    def step(i):
        r = reps[i % replicas]
        if fused:
            bd.kv_cache_write_and_decode(out, q, k_new, v_new, slots, r.k_pool, r.v_pool, bt, ctx,
                                         w.scale, max_context_len=w.max_context_len,
                                         workspace=ws, num_waves=nw)
            return
        if grouped:
            if fp8:
                bd.kv_cache_write_fp8(k_new, v_new, r.k_pool, r.v_pool, slots, w.k_scale,
                                      w.v_scale)
            else:
                bd.kv_cache_write(k_new, v_new, r.k_pool, r.v_pool, slots)
            bd.paged_attention_decode_shared_prefix(
                out, q, r.k_pool, r.v_pool, bt, ctx, gstart, gpre, w.scale, w.num_seqs,
                w.prefix_tokens, k_scale=w.k_scale, v_scale=w.v_scale,
                max_context_len=w.max_context_len, workspace=ws, num_waves=nw)
            return
        if fp8:
            bd.kv_cache_write_fp8(k_new, v_new, r.k_pool, r.v_pool, slots, w.k_scale, w.v_scale)
            bd.paged_attention_decode_fp8(out, q, r.k_pool, r.v_pool, bt, ctx, w.scale,
                                          w.k_scale, w.v_scale,
                                          max_context_len=w.max_context_len, workspace=ws,
                                          num_waves=nw)
            return
        bd.kv_cache_write(k_new, v_new, r.k_pool, r.v_pool, slots)
        if w.kind == "decode":
            bd.paged_attention_decode(out, q, r.k_pool, r.v_pool, bt, ctx, w.scale,
                                      max_context_len=w.max_context_len, partition_size=P,
                                      workspace=ws, num_waves=nw)
        else:
            bd.paged_attention_prefill_chunk(out, q, cu, ctx, r.k_pool, r.v_pool, bt, w.scale,
                                             max_q_len=w.max_q_len,
                                             max_context_len=w.max_context_len)

    if args.calibrate_copy:
        calibration_copies(dev)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    log(f"warmup done ({args.warmup} steps, {replicas} pool copies of {pool_bytes / 1e6:.0f} MB)")

    def timed(first, instrument):
        """K steps bracketed by synchronisations and torch events on the launch stream; with
        `instrument`, the library also times each of its kernels with HIP events recorded by
        the kernel dispatches themselves."""
        bd.profile_enable(instrument)
        start = torch.cuda.Event(enable_timing=True)
        stop = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record()
        for i in range(args.steps):
            step(first + i)
        stop.record()
        torch.cuda.synchronize()
        kern = {}
        if instrument:
            for name in bd.KERNEL_NAMES:
                ms, cnt = bd.profile_read(name)
                if cnt:
                    kern[name] = {"avg_us": 1e3 * ms / cnt, "launches": cnt}
        bd.profile_enable(False)
        return start.elapsed_time(stop) / args.steps, kern

    def per_step(first):
        """Each step between its own pair of torch events on the launch stream (median, p10,
        p90 of the step times)."""
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(evs):
            a.record()
            step(first + i)
            b.record()
        torch.cuda.synchronize()
        return _percentiles([1e3 * a.elapsed_time(b) for a, b in evs])

    # Pass 1 gives the throughput; pass 2 (same steps, kernels timed) the per-kernel durations;
    # pass 3 the distribution of single-step times.
    ms_per_step, _ = timed(args.warmup, False)
    ms_instr, kern = timed(args.warmup + args.steps, True)
    step_dist = per_step(args.warmup + 2 * args.steps)
    log(f"timed {args.steps} steps: {ms_per_step * 1e3:.1f} us/step "
        f"({ms_instr * 1e3:.1f} us/step with kernel timing); kernels: {kern}; "
        f"single steps: {step_dist}")

    probe = None
    if (w.kind == "decode" and w.dtype == "bf16" and not (fp8 or grouped or fused)
            and P == 0):
        # The read probe: the decode's waves reading exactly its tiles without the arithmetic,
        # over the same rotation of pool copies, timed the same way as the kernels above.
        sink = torch.empty(bd.lib().pkv_decode_read_probe_sink_size(
            w.num_seqs, w.num_q_heads, w.num_kv_heads, w.max_context_len, nw) // 4,
            dtype=torch.int32, device=dev)
        for i in range(args.warmup):
            r = reps[i % replicas]
            bd.decode_read_probe(r.k_pool, r.v_pool, bt, ctx, w.num_q_heads,
                                 max_context_len=w.max_context_len, num_waves=nw, sink=sink)
        bd.profile_enable(True, kernels=["read_probe"])
        torch.cuda.synchronize()
        for i in range(args.steps):
            r = reps[i % replicas]
            bd.decode_read_probe(r.k_pool, r.v_pool, bt, ctx, w.num_q_heads,
                                 max_context_len=w.max_context_len, num_waves=nw, sink=sink)
        torch.cuda.synchronize()
        pms, pcnt = bd.profile_read("read_probe")
        bd.profile_enable(False)
        probe = {"avg_us": 1e3 * pms / pcnt, "launches": pcnt}
        log(f"read probe: {probe['avg_us']:.1f} us per launch")

    result = {}
    if w.kind == "decode":
        b = decode_bytes(w)
        step_bytes = sum(b.values()) + write_bytes(w)
        value = step_bytes / (ms_per_step * 1e-3) / 1e9
        dom = "decode_partition"
        dom_bytes = b["kv"] + b["q"] + b["ids"] + b["ctx"] + (0 if "decode_reduce" in kern
                                                              else b["out"])
        if fused:  # the one kernel also stores the new tokens
            dom_bytes += write_bytes(w)
        if w.prefix_tokens:
            # HBM has to deliver each shared prefix block once; the plain decode reads it once
            # per sequence, mostly from cache, the prefix-aware one once per KV head
            logical_bytes = dom_bytes
            dom_bytes += unique_decode_kv_bytes(w) - b["kv"]
        dom_us = kern[dom]["avg_us"]
        achieved = dom_bytes / (dom_us * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": traffic_from_profile(args.workload, dom_bytes),
                "kernel": dom, "avg_us": round(dom_us, 2),
                "algorithmic_bytes_per_launch": dom_bytes}
        shape = {"decode-8b": "8B-shaped", "decode-70b": "70B-shaped",
                 "shared-prefix": "shared-prefix, 8B-shaped", "decode-8b-fp8": "8B-shaped, fp8 KV",
                 "decode-70b-fp8": "70B-shaped, fp8 KV",
                 "shared-prefix-grouped": "shared-prefix, prefix-aware, 8B-shaped",
                 "shared-prefix-grouped-fp8": "shared-prefix, prefix-aware, 8B-shaped, fp8 KV",
                 "decode-8b-fused": "8B-shaped, fused write+decode",
                 "decode-70b-fused": "70B-shaped, fused write+decode",
                 "decode-70b-tp8": "70B-shaped, one GPU's share under 8-way tensor parallelism",
                 }[args.workload]
        result.update(
            metric=f"paged decode KV HBM GB/s (% of peak) and decode tokens/sec/GPU, {shape}",
            value=round(value, 1), unit="GB/s", higher_is_better=True,
            pct_of_hbm_peak=round(100 * value / HBM_PEAK_GBS, 2),
            tokens_per_s_per_layer=round(w.num_seqs / (ms_per_step * 1e-3), 1),
            tokens_per_s_32_layers=round(w.num_seqs / (32 * ms_per_step * 1e-3), 1),
            step_bytes=step_bytes,
            decode_split="balanced" if P_eff == 0 else f"fixed partitions of {P_eff} tokens")
        if w.prefix_tokens:
            roof["logical_bytes_per_launch"] = logical_bytes
            roof["logical_achieved"] = round(logical_bytes / (dom_us * 1e-6) / 1e9, 1)
        # The decode call as the method defines it: the partition kernel plus the merge (both
        # event-timed per launch), over the call's algorithmic bytes (q, K/V, ids, out).
        call_us = dom_us + kern.get("decode_reduce", {}).get("avg_us", 0.0)
        call_bytes = dom_bytes if "decode_reduce" not in kern else dom_bytes + b["out"]
        result["decode_call"] = {
            "avg_us": round(call_us, 2), "achieved": round(call_bytes / (call_us * 1e-6) / 1e9, 1),
            "frac": round(call_bytes / (call_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "kernels": [k for k in ("decode_partition", "decode_reduce") if k in kern]}
        if probe is not None:
            pgbs = dom_bytes / (probe["avg_us"] * 1e-6) / 1e9
            result["read_probe"] = {
                "avg_us": round(probe["avg_us"], 2), "achieved": round(pgbs, 1),
                "frac_of_peak": round(pgbs / HBM_PEAK_GBS, 4),
                "decode_pct_of_probe": round(100 * probe["avg_us"] / dom_us, 2),
                "what": "the decode's waves reading exactly its K/V tiles with its loads, "
                        "no attention arithmetic (pkv_decode_read_probe)"}
    else:
        flops = prefill_flops(w)
        dom = "prefill_chunk"
        dom_us = kern[dom]["avg_us"]
        achieved = flops / (dom_us * 1e-6) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                "traffic": traffic_from_profile(args.workload, prefill_bytes(w)),
                "kernel": dom, "avg_us": round(dom_us, 2), "algorithmic_flops_per_launch": flops}
        value = flops / (ms_per_step * 1e-3) / 1e12
        result.update(metric="chunked prefill attention TFLOP/s (MFMA bf16 % of peak)",
                      value=round(value, 1), unit="TFLOP/s", higher_is_better=True,
                      tokens_per_s=round(w.total_q / (ms_per_step * 1e-3), 1))
    result["kernels"] = {k: {"avg_us": round(v["avg_us"], 2), "launches": v["launches"]}
                         for k, v in kern.items()}
    result["roofline"] = roof
    result["ms_per_step"] = round(ms_per_step, 4)
    result["ms_per_step_kernel_timing_on"] = round(ms_instr, 4)
    result["step_us"] = step_dist
    return result


def traffic_from_profile(workload, algorithmic):
    """HBM bytes per launch measured by rocprofv3 counters, read from the committed summary in
    profiles/ -- only if the kernel sources are the ones the counters were taken on."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"kernel_sources_sha256:\s*([0-9a-f]{64})", text)
    t = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m or not t or m.group(1) != kernel_sources_sha(workload):
        return None
    return float(t.group(1))


def kernel_sources(workload):
    """The sources that decide what the workload's dominant kernel does: the kernel's own file,
    the shared device headers, and the host code that plans its launch (api.cpp)."""
    if workload in BLOCK_WORKLOADS:
        return ["blocks.hip", "common.hpp", "launch.hpp", "api.cpp"]
    main = "prefill.hip" if workload == "prefill-chunk" else "decode.hip"
    return [main, "common.hpp", "lds_tile.hpp", "launch.hpp", "api.cpp"]


def kernel_sources_sha(workload):
    """SHA-256 of the code of kernel_sources(workload): comments dropped and whitespace
    collapsed, so that editing a comment does not disown counters taken on the same code."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "paged_kv_cache_190_amd", "csrc")
    for f in sorted(kernel_sources(workload)):
        text = open(os.path.join(csrc, f)).read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(f.encode() + b"\0" + " ".join(text.split()).encode())
    return h.hexdigest()


# ------------------------------------------------------------------------------ CPU baseline

def cpu_model():
    """The host CPU's model name from /proc/cpuinfo (None where there is none)."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def host_cores():
    """Cores this process may use: its CPU affinity, capped by OMP_NUM_THREADS when that is set
    (the share of the host a GPU job is given)."""
    n = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS", "")
    return max(1, min(n, int(env))) if env.isdigit() and int(env) > 0 else n


# State shared with the oracle's worker processes: set before the pool forks, so each worker
# sees the same arrays without copying them.
_CPU = {}


def _cpu_decode_worker(args):
    """One worker of the all-cores leg: whole sequences of the batch (its share, in turn) until
    the deadline; returns (KV bytes attended, sequences done, seconds)."""
    from threadpoolctl import threadpool_limits

    from oracle import paged_attention as orc
    widx, nworkers, deadline = args
    w, kp, vp = _CPU["w"], _CPU["kp"], _CPU["vp"]
    per_tok = 2 * w.num_kv_heads * w.head_dim * _pool_esz(w)
    work = done = 0
    t0 = time.perf_counter()
    with threadpool_limits(limits=1):
        s = widx
        while time.time() < deadline:
            sq = s % w.num_seqs
            orc.decode(w.q[sq:sq + 1], kp, vp, w.block_table[sq:sq + 1],
                       w.context_lens[sq:sq + 1], w.scale, w.dtype,
                       kv_dtype=w.kv_dtype or None, k_scale=w.k_scale, v_scale=w.v_scale)
            work += int(w.context_lens[sq]) * per_tok
            done += 1
            s += nworkers
    return work, done, time.perf_counter() - t0


def _cpu_prefill_worker(args):
    """All-cores leg of the prefill: this worker's share of the shuffled (row, head) outputs
    until the deadline; returns (flops, outputs done, seconds)."""
    from threadpoolctl import threadpool_limits

    from oracle import paged_attention as orc
    widx, nworkers, deadline = args
    w, kp, vp, rows, pos = _CPU["w"], _CPU["kp"], _CPU["vp"], _CPU["rows"], _CPU["pos"]
    flops = done = 0
    t0 = time.perf_counter()
    with threadpool_limits(limits=1):
        for t, h in rows[widx::nworkers]:
            if time.time() >= deadline:
                break
            orc.prefill_chunk(w.q, w.cu_q_lens, w.context_lens, kp, vp, w.block_table, w.scale,
                              w.dtype, rows=[(t, h)])
            flops += 4 * w.head_dim * pos[t]
            done += 1
    return flops, done, time.perf_counter() - t0


def cpu_baseline(w, budget_s):
    """The oracle, unchanged, timed on the host on a bounded sample of the same batch, twice:
    with BLAS limited to one thread (one core), and as a pool of single-threaded worker processes
    over the host's cores (all cores), each for about budget_s seconds. Scaled to GB/s (decode)
    or TFLOP/s (prefill) with the GPU's algorithmic byte / flop counts. Runs before the process
    touches the GPU, so the pool forks a process with no GPU state."""
    import multiprocessing as mp
    import random

    from oracle import paged_attention as orc
    if w.pool_dtype == "fp8":
        kp, vp = orc.kv_cache_write_fp8(w.k_pool, w.v_pool, w.k_new, w.v_new, w.slot_mapping,
                                        w.block_size, w.dtype, w.k_scale, w.v_scale)
    else:
        kp, vp = orc.kv_cache_write(w.k_pool, w.v_pool, w.k_new, w.v_new, w.slot_mapping,
                                    w.block_size)
    _CPU.update(w=w, kp=kp, vp=vp)
    cores = host_cores()
    model = cpu_model()
    if w.kind == "decode":
        one = _cpu_decode_worker((0, 1, time.time() + budget_s))
        unit, scale = "GB/s", 1e9
        what = (f"oracle decode of whole sequences, all {w.num_q_heads} query heads, passes over "
                f"the {w.num_seqs}-sequence batch (float64 NumPy); KV bytes of the sample / time")
    else:
        rows = [(t, h) for t in range(w.total_q) for h in range(w.num_q_heads)]
        random.Random(0).shuffle(rows)
        pos = {}
        for s in range(w.num_seqs):
            for t in range(int(w.cu_q_lens[s]), int(w.cu_q_lens[s + 1])):
                pos[t] = int(w.context_lens[s]) - int(w.cu_q_lens[s + 1]) + t + 1
        _CPU.update(rows=rows, pos=pos)
        one = _cpu_prefill_worker((0, 1, time.time() + budget_s))
        unit, scale = "TFLOP/s", 1e12
        what = ("oracle prefill of random (row, head) outputs, one at a time (float64 NumPy); "
                "flops of the sample / time")
    t0 = time.perf_counter()
    ctx = mp.get_context("fork")
    worker = _cpu_decode_worker if w.kind == "decode" else _cpu_prefill_worker
    deadline = time.time() + budget_s
    with ctx.Pool(cores) as pool:
        parts = pool.map(worker, [(i, cores, deadline) for i in range(cores)])
    wall = time.perf_counter() - t0
    all_work = sum(p[0] for p in parts)
    all_done = sum(p[1] for p in parts)
    digits = 4 if unit == "GB/s" else 6
    return {"value": round(all_work / wall / scale, digits), "unit": unit, "cores": cores,
            "kind": "oracle", "cpu_model": model,
            "sample": f"{what}; all cores: {cores} single-threaded processes, {all_done} items in "
                      f"{wall:.1f} s",
            "one_core": {"value": round(one[0] / one[2] / scale, digits), "unit": unit,
                         "cores": 1, "sample": f"{one[1]} items in {one[2]:.1f} s, BLAS "
                                               f"limited to one thread"}}


# ------------------------------------------------------------------- rocprofv3 summaries

# Traced runs warm up for TRACE_WARMUP steps: compute-bound kernels run slower until the GPU's
# clocks have ramped up (the chunked prefill from about 420 down to 340 us over its first few
# dozen launches), so the summary also averages only the dispatches after the warmup.
TRACE_WARMUP = 100
TRACE_CMD = ("rocprofv3 --kernel-trace --stats -f csv -d {d} -o run -- "
             "python3 bench.py --workload {w} --steps 20 --warmup " + str(TRACE_WARMUP) +
             " --no-cpu-baseline")
PMC_CMD = ("rocprofv3 --pmc {c} -f csv -d {d} -o run -- python3 bench.py "
           "--workload {w} --steps 10 --warmup 2 --no-cpu-baseline --calibrate-copy")


def _csv(path):
    import csv
    return list(csv.DictReader(open(path)))


def _find(d, suffix):
    for root, _, files in os.walk(d):
        for f in files:
            if f.endswith(suffix):
                return os.path.join(root, f)
    raise FileNotFoundError(f"no *{suffix} under {d}")


def _short(name):
    return name.split("(")[0].replace("void ", "").replace("pkv::", "")


def _rel(d):
    """The output directory as the recorded command names it (relative to the repository root
    when it lies inside it)."""
    a = os.path.abspath(d)
    return os.path.relpath(a, ROOT) if a.startswith(ROOT + os.sep) else a


def summarize_trace(d, workload):
    rows = _csv(_find(d, "kernel_stats.csv"))
    launches = {}
    for r in _csv(_find(d, "kernel_trace.csv")):  # dispatch order
        launches.setdefault(_short(r["Kernel_Name"]), []).append(
            (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    cmd = TRACE_CMD.format(w=workload, d=_rel(d))
    out = [f"# Kernel durations, workload {workload}", "",
           "rocprofv3 kernel trace of `bench.py` on one MI355X (gfx950).", "",
           f"Command (from the repository root): `{cmd}`", "",
           "Columns 2-6 are rocprofv3's statistics over every dispatch; the last column averages "
           f"the same trace's dispatches after the first {TRACE_WARMUP} of each kernel (the "
           "bench's warmup steps).", "",
           "| kernel | calls | average us | min us | max us | share of GPU time | "
           "average us after warmup |",
           "|---|---|---|---|---|---|---|"]
    for r in rows:
        k = _short(r["Name"])
        after = launches.get(k, [])[TRACE_WARMUP:]
        steady = f"{sum(after) / len(after):.2f} ({len(after)})" if after else "-"
        out.append(f"| `{k}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} "
                   f"| {float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                   f"{float(r['Percentage']):.1f}% | {steady} |")
    out += ["", "`__amd_rocclr_copyBuffer` is the set-up copies of the inputs to the device "
            "(not timed by the bench)."]
    path = os.path.join(ROOT, "profiles", f"kernels_{workload}.md")
    open(path, "w").write("\n".join(out) + "\n")
    return path


def _dispatches(path):
    """{dispatch id: (kernel name, counter value)} from a rocprofv3 counter_collection.csv."""
    return {int(r["Dispatch_Id"]): (_short(r["Kernel_Name"]), float(r["Counter_Value"]))
            for r in _csv(path)}


def summarize_pmc(fetch_dir, write_dir, workload, dominant):
    """Both runs execute the same program, so dispatch ids match across them. The calibration
    copies are the device copies whose WRITE_SIZE is the copy size."""
    fetch = _dispatches(_find(fetch_dir, "counter_collection.csv"))
    write = _dispatches(_find(write_dir, "counter_collection.csv"))
    copy_kib = COPY_BYTES / 1024
    calib = [i for i, (k, v) in write.items()
             if "copy" in k.lower() and abs(v - copy_kib) < 1e-3 * copy_kib and i in fetch]
    if not calib:
        raise RuntimeError("no calibration copy found (run bench.py with --calibrate-copy)")
    f_scale = copy_kib / (sum(fetch[i][1] for i in calib) / len(calib))
    w_scale = copy_kib / (sum(write[i][1] for i in calib) / len(calib))
    per = {}
    for i, (k, fv) in fetch.items():
        wv = write.get(i, (k, 0.0))[1]
        per.setdefault(k, []).append((fv, wv))
    out = [f"# HBM traffic per dispatch, workload {workload}", "",
           "rocprofv3 counters on one MI355X (gfx950), one run per counter:", "",
           f"- `{PMC_CMD.format(c='FETCH_SIZE', w=workload, d=_rel(fetch_dir))}`",
           f"- `{PMC_CMD.format(c='WRITE_SIZE', w=workload, d=_rel(write_dir))}`", "",
           f"Scale: the {len(calib)} calibration copies of {COPY_BYTES >> 20} MiB (device to "
           f"device) read {copy_kib / f_scale:.0f} KiB and write {copy_kib / w_scale:.0f} KiB each "
           f"by these counters, so FETCH_SIZE is multiplied by {f_scale:.4f} and WRITE_SIZE by "
           f"{w_scale:.4f}.", "",
           "| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled bytes |",
           "|---|---|---|---|---|"]
    avg = {}
    for k, v in per.items():
        fv = sum(x for x, _ in v) / len(v)
        wv = sum(y for _, y in v) / len(v)
        avg[k] = (fv * f_scale + wv * w_scale) * 1024
        out.append(f"| `{k}` | {len(v)} | {fv:.0f} | {wv:.0f} | {avg[k]:.4g} |")
    dom = next(k for k in per if k.startswith(dominant))
    out += ["", "(`__amd_rocclr_copyBuffer` rows mix the input set-up copies and the calibration "
            "copies.)", "", f"dominant kernel: `{dom}`",
            f"traffic_bytes_per_launch: {avg[dom]:.6g}",
            f"kernel_sources_sha256: {kernel_sources_sha(workload)}"]
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.md")
    open(path, "w").write("\n".join(out) + "\n")
    return path


MFMA_CMD = ("rocprofv3 --pmc SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_VALU_MFMA_BUSY_CYCLES "
            "GRBM_GUI_ACTIVE -f csv -d {d} -o run -- python3 bench.py "
            "--workload {w} --steps 10 --warmup 2 --no-cpu-baseline")


def summarize_mfma(d, workload):
    """MFMA utilisation = busy cycles / (GUI-active cycles of one XCD x 1024 SIMDs); the
    GRBM_GUI_ACTIVE value rocprofv3 reports is summed over the 8 XCDs."""
    rows = _csv(_find(d, "counter_collection.csv"))
    per = {}
    for r in rows:
        k = _short(r["Kernel_Name"])
        per.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    out = [f"# MFMA utilisation, workload {workload}", "",
           f"Command (from the repository root): `{MFMA_CMD.format(w=workload, d=_rel(d))}`", "",
           "| kernel | dispatches | MFMA bf16 MOPs (x512 flops) | busy cycles | GUI active "
           "(sum of 8 XCDs) | MFMA busy % | bf16 flops per dispatch |",
           "|---|---|---|---|---|---|---|"]
    for k, c in per.items():
        mops = sum(c["SQ_INSTS_VALU_MFMA_MOPS_BF16"]) / len(c["SQ_INSTS_VALU_MFMA_MOPS_BF16"])
        if mops == 0:
            continue
        busy = sum(c["SQ_VALU_MFMA_BUSY_CYCLES"]) / len(c["SQ_VALU_MFMA_BUSY_CYCLES"])
        gui = sum(c["GRBM_GUI_ACTIVE"]) / len(c["GRBM_GUI_ACTIVE"])
        util = 100 * busy / ((gui / 8) * 1024)
        out.append(f"| `{k}` | {len(c['GRBM_GUI_ACTIVE'])} | {mops:.4g} | {busy:.4g} | "
                   f"{gui:.4g} | {util:.1f} | {mops * 512:.4g} |")
    path = os.path.join(ROOT, "profiles", f"mfma_{workload}.md")
    open(path, "w").write("\n".join(out) + "\n")
    return path


# Instruction and stall counters of the dominant kernel, one rocprofv3 pass per set (each set
# within one pass's hardware limits).
COUNTER_SETS = (
    "SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_WAIT_INST_LDS "
    "SQ_ACTIVE_INST_LDS SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_ANY",
    "SQ_LDS_IDX_ACTIVE SQ_LDS_DATA_FIFO_FULL SQ_LDS_CMD_FIFO_FULL SQ_LDS_BANK_CONFLICT "
    "SQ_INSTS_LDS_LOAD_BANDWIDTH SQ_VALU_MFMA_BUSY_CYCLES SQ_VALU_MFMA_COEXEC_CYCLES "
    "SQ_INST_LEVEL_LDS GRBM_GUI_ACTIVE",
    "SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS SQ_INSTS_SALU SQ_INSTS_VALU_TRANS_F32 "
    "SQ_ACTIVE_INST_MISC SQ_ACTIVE_INST_SCA SQ_WAVES GRBM_GUI_ACTIVE",
)
COUNTERS_CMD = ("rocprofv3 --pmc {c} -f csv -d {d} -o run -- python3 bench.py --workload {w} "
                "--steps 10 --warmup 60 --no-cpu-baseline")


def summarize_counters(dirs, workload, dominant):
    """Per-dispatch averages of the COUNTER_SETS passes for the dominant kernel, with the ratios
    they give (shares of wave cycles, MFMA busy and co-issue shares, instructions per MFMA)."""
    vals = {}
    kernel = None
    for d in dirs:
        per = {}
        for r in _csv(_find(d, "counter_collection.csv")):
            k = _short(r["Kernel_Name"])
            if k.startswith(dominant):
                kernel = k
                per.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
        for c, v in per.items():
            vals.setdefault(c, sum(v) / len(v))
    out = [f"# Instruction and stall counters, workload {workload}", "",
           "Commands (from the repository root), one pass per counter set:", ""]
    for c, d in zip(COUNTER_SETS, dirs):
        out.append(f"- `{COUNTERS_CMD.format(c=c, d=_rel(d), w=workload)}`")
    out += ["", f"Kernel: `{kernel}`; per-dispatch averages (each counter summed over the GPU).",
            "", "| counter | per dispatch |", "|---|---|"]
    for c in sorted(vals):
        out.append(f"| {c} | {vals[c]:.4g} |")
    def ratio(a, b):
        return vals[a] / vals[b] if a in vals and b in vals and vals[b] else float("nan")
    gui = vals.get("GRBM_GUI_ACTIVE", float("nan"))
    derived = [
        ("wave cycles issuing any instruction", ratio("SQ_ACTIVE_INST_ANY", "SQ_WAVE_CYCLES")),
        ("wave cycles issuing VALU", ratio("SQ_ACTIVE_INST_VALU", "SQ_WAVE_CYCLES")),
        ("wave cycles waiting (any)", ratio("SQ_WAIT_ANY", "SQ_WAVE_CYCLES")),
        ("wave cycles waiting on LDS", ratio("SQ_WAIT_INST_LDS", "SQ_WAVE_CYCLES")),
        ("MFMA busy (of 1024 SIMDs x GUI-active cycles of one XCD)",
         vals.get("SQ_VALU_MFMA_BUSY_CYCLES", float("nan")) / (gui / 8 * 1024)),
        ("MFMA-busy cycles co-issuing VALU",
         ratio("SQ_VALU_MFMA_COEXEC_CYCLES", "SQ_VALU_MFMA_BUSY_CYCLES")),
        ("VALU instructions per MFMA instruction (as counted)",
         ratio("SQ_INSTS_VALU", "SQ_INSTS_MFMA")),
        ("transcendental per MFMA", ratio("SQ_INSTS_VALU_TRANS_F32", "SQ_INSTS_MFMA")),
        ("SALU per MFMA", ratio("SQ_INSTS_SALU", "SQ_INSTS_MFMA")),
        ("LDS instructions per MFMA", ratio("SQ_INSTS_LDS", "SQ_INSTS_MFMA")),
        ("LDS bank conflicts per LDS-active cycle",
         ratio("SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE")),
    ]
    out += ["", "| derived | value |", "|---|---|"]
    out += [f"| {name} | {v:.3f} |" for name, v in derived]
    path = os.path.join(ROOT, "profiles", f"counters_{workload}.md")
    open(path, "w").write("\n".join(out) + "\n")
    return path


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", choices=sorted(WORKLOADS) + list(BLOCK_WORKLOADS),
                    default="decode-8b")
    ap.add_argument("--replicas", type=int, default=0,
                    help="pool copies the steps rotate over (0: enough for 2 GB)")
    ap.add_argument("--partition-size", type=int, default=0)
    ap.add_argument("--waves", type=int, default=0,
                    help="waves of the balanced decode split (0: the library's default)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run a 256 MiB device copy first (scale for rocprofv3 byte counters)")
    ap.add_argument("--summarize-trace", metavar="DIR",
                    help="write profiles/kernels_<workload>.md from a rocprofv3 kernel trace")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/traffic_<workload>.md from FETCH_SIZE / WRITE_SIZE runs")
    ap.add_argument("--summarize-mfma", metavar="DIR",
                    help="write profiles/mfma_<workload>.md from an MFMA counter run")
    ap.add_argument("--summarize-counters", nargs=len(COUNTER_SETS), metavar="DIR",
                    help="write profiles/counters_<workload>.md from the COUNTER_SETS passes")
    args = ap.parse_args()
    if args.summarize_mfma:
        print(summarize_mfma(args.summarize_mfma, args.workload))
    if args.summarize_counters:
        dom = "prefill" if args.workload == "prefill-chunk" else "decode"
        print(summarize_counters(args.summarize_counters, args.workload, dom))
        return
    if args.summarize_trace or args.summarize_pmc:
        if args.summarize_trace:
            print(summarize_trace(args.summarize_trace, args.workload))
        if args.summarize_pmc:
            dom = ("prefill" if args.workload == "prefill-chunk" else
                   "decode_prefix" if args.workload.startswith("shared-prefix-grouped") else
                   "copy_blocks" if args.workload in BLOCK_WORKLOADS else "decode_balanced")
            print(summarize_pmc(*args.summarize_pmc, args.workload, dom))
    if args.summarize_trace or args.summarize_pmc or args.summarize_mfma:
        return
    if args.gpus != 1:
        print(f"bench.py: the library runs on one GPU; --gpus {args.gpus} is not supported "
              "(the paged-attention kernels shard by sequence or KV head without any exchange; "
              "multi-GPU runs are out of scope here)", file=sys.stderr)
        sys.exit(2)

    # Inputs and the CPU baseline first: the oracle's worker pool forks before this process
    # touches the GPU.
    from paged_kv_cache_190_amd.workloads import CONFIG_NAMES
    blocks = args.workload in BLOCK_WORKLOADS
    w = make_workload(args)
    cpu = None
    if not args.no_cpu_baseline:
        log("timing the oracle on the host ...")
        cpu = (cpu_baseline_blocks(w, block_sources(w, args.workload), args.cpu_seconds)
               if blocks else cpu_baseline(w, args.cpu_seconds))
        log(f"oracle: {cpu}")

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    res = run_blocks(args, w) if blocks else run(args, w)
    base = "decode-8b" if blocks else args.workload
    desc = CONFIG_NAMES[WORKLOADS[base]]
    if args.workload.endswith("-tp8"):
        desc += f"; one GPU's share under 8-way KV-head split ({w.num_q_heads}/{w.num_kv_heads} heads)"
    cfg = {"workload": f"{args.workload}: {desc}",
           "num_seqs": w.num_seqs, "num_q_heads": w.num_q_heads,
           "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim, "block_size": w.block_size,
           "sum_context_tokens": int(w.context_lens.sum()), "seed": WORKLOADS[base]}
    if args.waves:
        cfg["num_waves"] = args.waves
    line = {"metric": res.pop("metric"), "value": res.pop("value"), "unit": res.pop("unit"),
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": res.pop("ms_per_step"), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": w.dtype, "data": "synthetic", "config": cfg}
    if w.kv_dtype:
        line["kv_dtype"] = w.kv_dtype
    line["roofline"] = res.pop("roofline")
    line["cpu_baseline"] = cpu
    line.update(res)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
