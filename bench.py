#!/usr/bin/env python3
"""Paged decode attention bench on one MI355X.

One step is one decode step of the whole batch through every stage of the
path: the host allocator appends one token to each sequence (taking a new
block where a block fills up), the block tables, context lengths and slot
mapping are rebuilt in pinned host memory and copied to the GPU in one
transfer, reshape_and_cache writes the batch's new K/V into their slots, the
partition kernel computes attention over every sequence's paged cache, and
the log-sum-exp merge combines the partitions.  Inputs are resident in HBM
before the timed region; the new tokens' K/V for every step are generated up
front.

Prints one JSON line: KV bytes read per second (algorithmic: each KV head's
cached K and V once per sequence, real tokens only, scales included) as
`value`, tokens/s, the roofline of the partition kernel measured with HIP
events, and the CPU oracle timed on the host for comparison.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

METRIC = "paged decode attn: KV GB/s (% of HBM peak) + tokens/s, Llama-3-8B shape"
HBM_PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="c2", choices=["c2", "c3", "c4", "c5"])
    ap.add_argument("--partition", type=int, default=None,
                    help="tokens per split-K partition (0 = library's choice, -1 = one pass)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cold-iters", type=int, default=20,
                    help="decode launches timed after a cache flush (0 to skip)")
    return ap.parse_args()


def kv_bytes_per_token(wl) -> int:
    """Algorithmic bytes of one token's K and V over all KV heads."""
    D, H = wl.D, wl.Hkv
    per = {"f16": 2 * D, "bf16": 2 * D, "fp8_e4m3": D + 4, "int4_asym_g32": D // 2 + (D // 32) * 4}
    return 2 * H * per[wl.kv_dtype]


def unique_tokens(lengths: np.ndarray, wl) -> int:
    """Distinct cached tokens: a shared prefix counts once."""
    tot = int(lengths.sum())
    if wl.shared_prefix:
        k, pre = wl.shared_prefix
        tot -= (k - 1) * pre
    return tot


def log(msg):
    sys.stderr.write(f"[bench] {msg}\n")
    sys.stderr.flush()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the decode path "
              "shards by sequence or KV head with no exchange, see the design notes.",
              file=sys.stderr)
        sys.exit(2)
    import torch

    if not torch.cuda.is_available():
        print("no GPU visible: the bench needs an MI355X", file=sys.stderr)
        sys.exit(3)
    import paged_kv_cache_250_amd as pkv
    import workloads

    wl = workloads.get(args.workload)
    partition = wl.partition if args.partition is None else args.partition
    total_steps = args.warmup + args.steps
    log(f"workload {wl.name}: {wl.description}")
    gen = workloads.generate(wl)
    B, Hq, Hkv, D, p = wl.B, wl.Hq, wl.Hkv, wl.D, wl.p
    io = wl.io_dtype
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16}[io]

    # ---- allocator state, pools, prefill (untimed)
    pool = pkv.BlockPool(gen.num_blocks, p, gen.free_order)
    pool.run_ops(gen.ops)
    W = -(-(int(gen.lengths.max()) + total_steps) // p)
    seq_ids = np.arange(B, dtype=np.int64)
    desc = pkv.cache_desc(wl.kv_dtype, io, Hkv, D, p, gen.num_blocks)
    pool_bytes, meta_bytes = pkv.pkv_cache_bytes(desc)
    k_pool = torch.empty(pool_bytes, dtype=torch.uint8, device="cuda")
    v_pool = torch.empty(pool_bytes, dtype=torch.uint8, device="cuda")
    k_meta = torch.empty(meta_bytes, dtype=torch.uint8, device="cuda") if meta_bytes else None
    v_meta = torch.empty(meta_bytes, dtype=torch.uint8, device="cuda") if meta_bytes else None
    seq, pos, rows = gen.token_positions()
    slots_all = pool.slot_mapping(seq, pos)
    chunk = 1 << 18
    for s in range(0, len(rows), chunk):
        r = rows[s:s + chunk]
        kk = torch.from_numpy(gen.k_bits[r].view(np.int16)).cuda().view(tdt)
        vv = torch.from_numpy(gen.v_bits[r].view(np.int16)).cuda().view(tdt)
        ss = torch.from_numpy(slots_all[s:s + chunk]).cuda()
        pkv.pkv_reshape_and_cache(desc, kk, vv, ss, k_pool, v_pool, k_meta, v_meta)
    torch.cuda.synchronize()
    q = torch.from_numpy(gen.q_bits.view(np.int16)).cuda().view(tdt)
    out = torch.empty((B, Hq, D), dtype=tdt, device="cuda")
    # new tokens of every step, drawn from their own seeded stream
    rng = np.random.default_rng(wl.seed + 7919)
    newk = rng.standard_normal((total_steps, B, Hkv, D), dtype=np.float32)
    newv = rng.standard_normal((total_steps, B, Hkv, D), dtype=np.float32)
    new_k = torch.from_numpy(newk).to(tdt).cuda()
    new_v = torch.from_numpy(newv).to(tdt).cuda()
    del newk, newv
    max_ctx_final = int(gen.lengths.max()) + total_steps
    ws_bytes = pkv.pkv_decode_workspace_bytes(desc, B, Hq, max_ctx_final, partition)
    ws = torch.empty(ws_bytes // 4 + 4, dtype=torch.float32, device="cuda") if ws_bytes else None
    resolved = pkv.pkv_decode_partition(desc, B, Hq, max_ctx_final, partition)
    scale = float(np.float32(1.0 / math.sqrt(D)))

    # ---- per-step metadata: slots (int64) | ctx_lens | tables, one pinned buffer per parity
    n_i32 = 2 * B + B + B * W
    pinned = [torch.empty(n_i32, dtype=torch.int32).pin_memory() for _ in range(2)]
    dev_meta = torch.empty(n_i32, dtype=torch.int32, device="cuda")
    copy_done = [torch.cuda.Event(), torch.cuda.Event()]
    slots_dev = dev_meta[:2 * B].view(torch.int64)
    ctx_dev = dev_meta[2 * B:3 * B]
    tables_dev = dev_meta[3 * B:].view(B, W)
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    bytes_per_tok = kv_bytes_per_token(wl)
    lengths = gen.lengths.copy()
    step_bytes, step_tokens = [], []

    def step(i: int, timed_idx: int | None):
        buf = pinned[i % 2]
        if i >= 2:
            copy_done[i % 2].synchronize()  # the copy that last read this buffer is done
        host = buf.numpy()
        slots_h = host[:2 * B].view(np.int64)
        pool.append_batch(seq_ids, 1, slots_h)                   # allocator: one token each
        pool.block_tables(seq_ids, W, host[3 * B:].reshape(B, W), host[2 * B:3 * B])
        dev_meta.copy_(buf, non_blocking=True)                    # one H2D transfer
        copy_done[i % 2].record(stream)
        pkv.pkv_reshape_and_cache(desc, new_k[i], new_v[i], slots_dev, k_pool, v_pool, k_meta,
                                  v_meta)
        max_ctx = int(lengths.max()) + i + 1
        a = pkv.decode_args(out, q, k_pool, v_pool, k_meta, v_meta, tables_dev, ctx_dev,
                            max_ctx, scale, partition, ws, flags=pkv.PKV_DECODE_SKIP_MERGE)
        if timed_idx is not None:
            ev[timed_idx][0].record(stream)
        pkv.pkv_paged_decode(desc, a)
        if timed_idx is not None:
            ev[timed_idx][1].record(stream)
        pkv.pkv_lse_reduce(desc, a)
        return unique_tokens(lengths + i + 1, wl)

    log(f"pool {gen.num_blocks} blocks, table width {W}, partition {resolved}, "
        f"workspace {ws_bytes} B; warmup {args.warmup}, steps {args.steps}")
    for i in range(args.warmup):
        step(i, None)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        ntok = step(args.warmup + k, k)
        step_tokens.append(ntok)
        step_bytes.append(ntok * bytes_per_tok)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    elapsed = t1 - t0
    kern_ms = [a.elapsed_time(b) for a, b in ev]
    kern_avg_s = float(np.mean(kern_ms)) / 1e3
    total_bytes = float(sum(step_bytes))
    value = total_bytes / elapsed / 1e9
    tokens_per_s = B * args.steps / elapsed
    achieved = float(np.mean(step_bytes)) / kern_avg_s / 1e9
    log(f"step {elapsed / args.steps * 1e3:.4f} ms, partition kernel avg {kern_avg_s * 1e6:.2f} us "
        f"(min {min(kern_ms) * 1e3:.2f}, max {max(kern_ms) * 1e3:.2f}), {achieved:.1f} GB/s")

    # ---- cold-cache timing of the decode call (flush >= 1 GiB between launches)
    cold = None
    if args.cold_iters > 0:
        flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        a = pkv.decode_args(out, q, k_pool, v_pool, k_meta, v_meta, tables_dev, ctx_dev,
                            int(lengths.max()) + total_steps, scale, partition, ws,
                            flags=pkv.PKV_DECODE_SKIP_MERGE)
        times = []
        for _ in range(args.cold_iters):
            pkv.pkv_bench_flush(flush)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            pkv.pkv_paged_decode(desc, a)
            e1.record(stream)
            e1.synchronize()
            times.append(e0.elapsed_time(e1) / 1e3)
        cold_bytes = unique_tokens(lengths + total_steps, wl) * bytes_per_tok
        cold = {"median_us": float(np.median(times) * 1e6),
                "gbs": float(cold_bytes / np.median(times) / 1e9)}
        # streaming-read ceiling on the same GPU
        sink = torch.empty(8192, dtype=torch.int32, device="cuda")
        buf = torch.empty(2 << 30, dtype=torch.uint8, device="cuda")
        pkv.pkv_bench_flush(buf)
        rt = []
        for _ in range(5):
            pkv.pkv_bench_flush(flush)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            pkv.pkv_bench_stream_read(buf, sink)
            e1.record(stream)
            e1.synchronize()
            rt.append(e0.elapsed_time(e1) / 1e3)
        cold["stream_read_gbs"] = float(buf.numel() / np.median(rt) / 1e9)
        del flush, buf
        log(f"cold decode {cold['median_us']:.1f} us = {cold['gbs']:.1f} GB/s; "
            f"streaming read {cold['stream_read_gbs']:.1f} GB/s")

    # ---- CPU oracle on the host cores (bounded sample of the same workload)
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(gen, wl, bytes_per_tok)

    dtype = {"bf16": "bf16", "f16": "f16"}[io]
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic (seeded N(0,1) Q/K/V, random block placement)",
        "config": {
            "workload": f"{wl.name}: {wl.description}",
            "batch": B, "q_heads": Hq, "kv_heads": Hkv, "head_dim": D, "block_size": p,
            "kv_dtype": wl.kv_dtype, "partition_tokens": resolved,
            "context_tokens_first_step": int(step_tokens[0]) if step_tokens else 0,
        },
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "tokens_per_s": round(tokens_per_s, 1),
        "roofline": {
            "bound": "hbm",
            "kernel": "paged_decode_kernel",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": None,
            "avg_us": round(kern_avg_s * 1e6, 3),
            "bytes_per_launch": int(np.mean(step_bytes)),
        },
        "cold": cold,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line))
    pool.close()


def cpu_baseline(gen, wl, bytes_per_tok):
    """Time the fp64 oracle's paged attention over the workload's sequences."""
    import oracle
    from oracle.state import oracle_state

    log("cpu baseline: building oracle pools")
    d, pools, bt, cl, _ = oracle_state(gen)
    # bounded sample: the first sequences up to ~5 M (token, query head) pairs,
    # about 10 s of single-core work (the whole Llama-3-8B-shaped batch)
    budget = 5_000_000
    mask = np.zeros(wl.B, np.uint8)
    acc = 0
    for b in range(wl.B):
        mask[b] = 1
        acc += int(gen.lengths[b]) * wl.Hq
        if acc >= budget:
            break
    ntok = int(gen.lengths[mask.astype(bool)].sum())
    times = []
    for _ in range(3):
        t0 = time.perf_counter()
        oracle.paged_attention(d, gen.q_bits, pools, bt, cl, float(np.float32(1 / math.sqrt(wl.D))),
                               seq_mask=mask)
        times.append(time.perf_counter() - t0)
    t = float(np.median(times))
    cores = oracle.num_threads()
    log(f"cpu baseline: {int(mask.sum())} sequences, {ntok} tokens, {t:.3f} s on {cores} threads")
    return {"value": round(ntok * bytes_per_tok / t / 1e9, 4), "unit": "GB/s", "cores": cores,
            "kind": "oracle",
            "sample": f"first {int(mask.sum())} of {wl.B} sequences ({ntok} tokens), one decode "
                      f"step, median of 3 runs ({t:.3f} s)",
            "tokens_per_s": round(int(mask.sum()) / t, 3)}


if __name__ == "__main__":
    main()
