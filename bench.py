#!/usr/bin/env python3
"""Paged decode attention bench on one MI355X.

One step is one decode step of the whole batch through every stage of the
path, over a stack of `--layers` attention layers that share one block table
(each layer has its own K/V pools, as in a model):

  host   the block pool appends one token to every sequence (taking a new
         block when one fills up); block tables, context lengths and the slot
         mapping are rebuilt in pinned memory (a ring of buffers, so the host
         prepares the next steps while the GPU works) and uploaded by a copy
         kernel in the launching stream that reads the pinned buffer directly;
  GPU    per layer: reshape_and_cache writes the batch's new K/V into their
         slots, the decode kernel computes attention over every
         sequence's paged cache, and the log-sum-exp merge combines the
         parts of the runs it split.

With four layers of the Llama-3-8B-shaped batch the KV read per step is
about 2.6 GB, ten times the 256 MB Infinity Cache, so every layer's KV comes
from HBM as it would in a full model.  Inputs are resident in HBM before the
timed region; the new tokens' K/V of every step are generated up front.

Prints one JSON line: KV bytes read per second (algorithmic: each KV head's
cached K and V once per sequence, real tokens only, FP8/INT4 scales
included) over the whole timed steps as `value` (wall-clock between
synchronisations, nothing timed inside), tokens/s, and the roofline of the
decode kernel.  The roofline comes from a separate pass after the steps:
`--launches` decode launches, each with its merge, timed one by one with HIP
events on the launching stream after a 1 GiB streaming read of another
buffer (cold caches), then as many back to back (warm).  The CPU oracle is
timed on the host for comparison.
"""
from __future__ import annotations

import argparse
import ctypes
import csv
import glob
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

METRIC = "paged decode attn: KV GB/s (% of HBM peak) + tokens/s, Llama-3-8B shape"
HBM_PEAK_GBS = 8000.0


def parse(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="c2", choices=["c2", "c3", "c4", "c5"])
    ap.add_argument("--layers", type=int, default=4,
                    help="attention layers per step sharing one block table")
    ap.add_argument("--partition", type=int, default=None,
                    help="tokens per split-K partition (0 = library's choice, -1 = one pass)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--upload", default="kernel", choices=["kernel", "dma"],
                    help="how each step's slots, lengths and tables reach the GPU: a copy "
                         "kernel reading the pinned buffer (default) or a DMA copy")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run the 1 GiB copy kernel (for scaling HBM byte counters)")
    ap.add_argument("--summarize-profiles", nargs=5, metavar=("STATS", "FETCH", "WRITE",
                                                              "COPY_FETCH", "COPY_WRITE"),
                    help="write the profile summary of --workload from rocprofv3 output "
                         "folders (kernel trace, FETCH_SIZE, WRITE_SIZE of the bench, then "
                         "FETCH_SIZE and WRITE_SIZE of --copy-calibration)")
    ap.add_argument("--command", default="",
                    help="with --summarize-profiles: the commands that made the folders")
    ap.add_argument("--placement", default="random", choices=["random", "identity"],
                    help="initial free-list order: seeded permutation (the workload's) or "
                         "0..N-1, which leaves every sequence's blocks contiguous")
    ap.add_argument("--block-size", type=int, default=None,
                    help="override the workload's block size (16 or 32)")
    ap.add_argument("--kv-dtype", default=None,
                    choices=["f16", "bf16", "fp8_e4m3", "fp8_e5m2", "fp8_e4m3_block",
                             "int4_asym_g32"],
                    help="override the workload's cache type")
    ap.add_argument("--copy-blocks", action="store_true",
                    help="time pkv_copy_blocks instead: the copy-on-write copies of one "
                         "beam-search step over the workload's batch, then a large copy")
    ap.add_argument("--beams", type=int, default=4,
                    help="with --copy-blocks: beams per sequence")
    ap.add_argument("--copy-case", default="both", choices=["both", "beam", "large"],
                    help="with --copy-blocks: which copies to time (profiles take one)")
    ap.add_argument("--swap", action="store_true",
                    help="time swapping instead: half of the batch's sequences out to pinned "
                         "host memory and back")
    ap.add_argument("--prefix-cache", action="store_true",
                    help="time the host prefix cache instead: RAG-style prompts with a "
                         "common prefix allocated, freed and re-requested")
    ap.add_argument("--kernel", default=None,
                    help="with --summarize-profiles: kernel to summarise (default: the "
                         "decode kernel of --workload)")
    ap.add_argument("--summarize-counters", nargs="+", metavar="FOLDER",
                    help="write the hardware-counter summary of the decode kernel of "
                         "--workload from rocprofv3 --pmc output folders (one pass each)")
    ap.add_argument("--launches", type=int, default=60,
                    help="decode launches timed one by one after the stepped run (cold, "
                         "then as many warm)")
    ap.add_argument("--counters-name", default="counters",
                    help="with --summarize-counters: suffix of the summary file")
    return ap.parse_args(argv)


def kv_bytes_per_token(wl) -> int:
    """Algorithmic bytes of one token's K and V over all KV heads of a layer."""
    D, H = wl.D, wl.Hkv
    per = {"f16": 2 * D, "bf16": 2 * D, "fp8_e4m3": D + 4, "fp8_e5m2": D + 4,
           "fp8_e4m3_block": D + 4,
           "int4_asym_g32": D // 2 + (D // 32) * 4}
    return 2 * H * per[wl.kv_dtype]


def unique_tokens(lengths: np.ndarray, wl) -> int:
    """Distinct cached tokens: a shared prefix counts once."""
    tot = int(lengths.sum())
    if wl.shared_prefix:
        k, pre = wl.shared_prefix
        tot -= (k - 1) * pre
    return tot


def _hip_runtime():
    """The HIP runtime library this process has loaded."""
    with open("/proc/self/maps") as f:
        for line in f:
            if "libamdhip64.so" in line:
                return ctypes.CDLL(line.split()[-1])
    return ctypes.CDLL("libamdhip64.so")


def pinned_device_address(t) -> int:
    """Device address of a pinned host tensor (hipHostGetDevicePointer), for
    kernels that read the buffer directly."""
    dev = ctypes.c_void_p()
    rc = _hip_runtime().hipHostGetDevicePointer(ctypes.byref(dev), ctypes.c_void_p(t.data_ptr()),
                                                ctypes.c_uint(0))
    if rc != 0 or not dev.value or dev.value % 16:
        raise RuntimeError(f"no 16-byte aligned device address for a pinned buffer (HIP error {rc})")
    return dev.value


# host ring of per-step metadata buffers, and how often an upload is marked
# with an event (a mark is needed until PINNED_RING steps after it, so
# MARK_EVENTS * MARK_EVERY must exceed PINNED_RING)
PINNED_RING, MARK_EVERY, MARK_EVENTS = 8, 4, 3


def log(msg):
    sys.stderr.write(f"[bench] {msg}\n")
    sys.stderr.flush()


class Bench:
    """Device state of one workload: allocator, shared tables, per-layer pools."""

    def __init__(self, wl, layers: int, max_steps: int, placement: str = "random",
                 upload: str = "kernel"):
        import torch

        import paged_kv_cache_250_amd as pkv
        import workloads

        self.torch, self.pkv, self.wl = torch, pkv, wl
        self.layers = layers
        gen = workloads.generate(wl)
        if placement == "identity":
            # blocks taken in id order: every sequence's blocks are contiguous
            gen.free_order = np.arange(gen.num_blocks, dtype=np.int32)
        self.gen = gen
        B, Hq, Hkv, D, p = wl.B, wl.Hq, wl.Hkv, wl.D, wl.p
        io = wl.io_dtype
        tdt = {"bf16": torch.bfloat16, "f16": torch.float16}[io]
        self.pool = pkv.BlockPool(gen.num_blocks, p, gen.free_order)
        self.pool.run_ops(gen.ops)
        self.W = -(-(int(gen.lengths.max()) + max_steps) // p)
        self.seq_ids = np.arange(B, dtype=np.int64)
        self.desc = pkv.cache_desc(wl.kv_dtype, io, Hkv, D, p, gen.num_blocks)
        pool_bytes, meta_bytes = pkv.pkv_cache_bytes(self.desc)
        self.pools = []
        seq, pos, rows = gen.token_positions()
        slots_all = self.pool.slot_mapping(seq, pos)
        chunk = 1 << 18
        # a block-scaled FP8 cache takes one token per block per call: the
        # prompts are written in rounds of one offset
        rounds = [np.arange(len(rows))] if wl.kv_dtype != "fp8_e4m3_block" else \
            [np.nonzero(slots_all % p == o)[0] for o in range(p)]
        for layer in range(layers):
            kp = torch.empty(pool_bytes, dtype=torch.uint8, device="cuda")
            vp = torch.empty(pool_bytes, dtype=torch.uint8, device="cuda")
            km = torch.empty(meta_bytes, dtype=torch.uint8, device="cuda") if meta_bytes else None
            vm = torch.empty(meta_bytes, dtype=torch.uint8, device="cuda") if meta_bytes else None
            for sel in rounds:
                for s in range(0, len(sel), chunk):
                    i = sel[s:s + chunk]
                    r = rows[i]
                    kk = torch.from_numpy(gen.k_bits[r].view(np.int16)).cuda().view(tdt)
                    vv = torch.from_numpy(gen.v_bits[r].view(np.int16)).cuda().view(tdt)
                    ss = torch.from_numpy(slots_all[i]).cuda()
                    pkv.pkv_reshape_and_cache(self.desc, kk, vv, ss, kp, vp, km, vm)
            self.pools.append((kp, vp, km, vm))
        torch.cuda.synchronize()
        self.pool_bytes = pool_bytes
        self.q = torch.from_numpy(gen.q_bits.view(np.int16)).cuda().view(tdt)
        self.out = torch.empty((B, Hq, D), dtype=tdt, device="cuda")
        # new tokens of every step and layer, from their own seeded stream
        rng = np.random.default_rng(wl.seed + 7919)
        shape = (max_steps, layers, B, Hkv, D)
        self.new_k = torch.from_numpy(rng.standard_normal(shape, dtype=np.float32)).to(tdt).cuda()
        self.new_v = torch.from_numpy(rng.standard_normal(shape, dtype=np.float32)).to(tdt).cuda()
        self.max_steps = max_steps
        self.steps_done = 0
        self.host_s = 0.0  # allocator and table building, summed over steps
        self.lengths0 = gen.lengths.copy()
        self.scale = float(np.float32(1.0 / math.sqrt(D)))
        self.bytes_per_tok = kv_bytes_per_token(wl)
        # Per-step metadata (slots as int64 | context lengths | block tables) is
        # built in pinned host memory and sent with one upload per step to one
        # of two device buffers (the stream orders a step's upload after the
        # kernels of the step before the last, which read the same buffer).
        # The host buffers form a ring of PINNED_RING, so that the host can
        # run ahead of the GPU; before it refills a buffer it waits for an
        # event recorded after a later upload, one event every MARK_EVERY
        # steps (each recorded event costs the stream a few microseconds).
        n_i32 = -(-(3 * B + B * self.W) // 4) * 4  # whole 16-byte vectors
        self.pinned = [torch.empty(n_i32, dtype=torch.int32).pin_memory()
                       for _ in range(PINNED_RING)]
        self.dev_meta = [torch.empty(n_i32, dtype=torch.int32, device="cuda") for _ in range(2)]
        self.marks = [torch.cuda.Event() for _ in range(MARK_EVENTS)]
        # The upload is a copy kernel in the launching stream that reads the
        # pinned buffer through its device address ("kernel"), or a DMA copy
        # (hipMemcpyAsync, "dma").  A DMA copy hands the stream over to a copy
        # engine and back: in a kernel trace of the c2 step it takes 6.6 us
        # with about 9 us before it and 15 us after it in which no kernel runs.
        self.upload = upload
        self.meta_bytes = n_i32 * 4
        self.pinned_dev = [pinned_device_address(t) for t in self.pinned] \
            if upload == "kernel" else None
        self.meta_views = [(m[:2 * B].view(torch.int64), m[2 * B:3 * B],
                            m[3 * B:3 * B + B * self.W].view(B, self.W)) for m in self.dev_meta]
        # an upper bound of every step's context lengths (the decode only reads
        # it as a bound)
        self.max_ctx = int(self.lengths0.max()) + max_steps
        self.args, self.args_key = None, None

    def workspace(self, partition):
        wl = self.wl
        nbytes = self.pkv.pkv_decode_workspace_bytes(self.desc, wl.B, wl.Hq, self.max_ctx,
                                                     partition)
        ws = self.torch.empty(nbytes // 4 + 4, dtype=self.torch.float32, device="cuda") \
            if nbytes else None
        return ws, self.pkv.pkv_decode_partition(self.desc, wl.B, wl.Hq, self.max_ctx, partition)

    def prepare(self, partition, ws):
        """Argument structs of every (metadata buffer, layer), built once."""
        pkv = self.pkv
        self.stream = self.torch.cuda.current_stream().cuda_stream
        # the merge runs as its own call so that the timed launch is the
        # decode kernel alone
        flags = pkv.PKV_DECODE_SKIP_MERGE
        self.args = [[pkv.decode_args(self.desc, self.out, self.q, kp, vp, km, vm, self.meta_views[k][2],
                                      self.meta_views[k][1], self.max_ctx, self.scale, partition,
                                      ws, flags=flags)
                      for (kp, vp, km, vm) in self.pools] for k in range(2)]
        ptr = lambda t: None if t is None else t.data_ptr()  # noqa: E731
        self.pool_ptrs = [tuple(ptr(t) for t in pools) for pools in self.pools]
        self.slot_ptrs = [ptr(self.meta_views[k][0]) for k in range(2)]
        self.new_ptrs = (self.new_k.data_ptr(), self.new_v.data_ptr(),
                         self.new_k[0, 0].numel() * self.new_k.element_size())

    def step(self, partition, ws):
        """One decode step over all layers; returns the step's KV bytes."""
        pkv, wl, B = self.pkv, self.wl, self.wl.B
        lib, desc = pkv._lib, ctypes.byref(self.desc)
        if self.args is None or self.args_key != (partition, None if ws is None else ws.data_ptr()):
            self.prepare(partition, ws)
            self.args_key = (partition, None if ws is None else ws.data_ptr())
        i = self.steps_done
        assert i < self.max_steps
        k = i % 2
        slot = i % PINNED_RING
        buf = self.pinned[slot]
        if i >= PINNED_RING:
            # the upload that last read this buffer (step i - PINNED_RING) is
            # done once the first marked upload at or after it is
            e = -(-(i - PINNED_RING) // MARK_EVERY) * MARK_EVERY
            self.marks[(e // MARK_EVERY) % MARK_EVENTS].synchronize()
        host = buf.numpy()
        t0 = time.perf_counter()
        self.pool.append_batch(self.seq_ids, 1, host[:2 * B].view(np.int64))
        self.pool.block_tables(self.seq_ids, self.W,
                               host[3 * B:3 * B + B * self.W].reshape(B, self.W), host[2 * B:3 * B])
        self.host_s += time.perf_counter() - t0
        if self.upload == "kernel":
            pkv._check(lib.pkv_bench_copy(ctypes.c_void_p(self.dev_meta[k].data_ptr()),
                                          ctypes.c_void_p(self.pinned_dev[slot]),
                                          ctypes.c_size_t(self.meta_bytes),
                                          ctypes.c_void_p(self.stream)))
        else:
            self.dev_meta[k].copy_(buf, non_blocking=True)
        if i % MARK_EVERY == 0:
            self.marks[(i // MARK_EVERY) % MARK_EVENTS].record()
        kbase, vbase, row = self.new_ptrs
        for layer in range(self.layers):
            kp, vp, km, vm = self.pool_ptrs[layer]
            off = (i * self.layers + layer) * row
            pkv._check(lib.pkv_reshape_and_cache(desc, kbase + off, vbase + off, B,
                                                 self.slot_ptrs[k], kp, vp, km, vm, self.stream))
            a = ctypes.byref(self.args[k][layer])
            pkv._check(lib.pkv_paged_decode(desc, a, self.stream))
            pkv._check(lib.pkv_lse_reduce(desc, a, self.stream))
        self.steps_done += 1
        return unique_tokens(self.lengths0 + i + 1, wl) * self.bytes_per_tok * self.layers

    def run(self, partition, warmup, steps, launches=60):
        """The stepped run (wall-clock, no events inside it), then a separate
        pass timing `launches` decode launches with their merges."""
        torch = self.torch
        ws, resolved = self.workspace(partition)
        for _ in range(warmup):
            self.step(partition, ws)
        step_bytes = []
        torch.cuda.synchronize()
        self.host_s = 0.0
        t0 = time.perf_counter()
        for k in range(steps):
            step_bytes.append(self.step(partition, ws))
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        last = self.steps_done - 1
        if not torch.equal(self.dev_meta[last % 2].cpu(), self.pinned[last % PINNED_RING]):
            raise RuntimeError("the last step's uploaded tables differ from the host's")
        # the last step's tables and context lengths stay in place: every
        # launch of the pass reads the same cache state
        last_bytes = unique_tokens(self.lengths0 + self.steps_done, self.wl) * self.bytes_per_tok
        cold = self.launch_pass(launches, flush=True)
        warm = self.launch_pass(launches, flush=False)
        return {"elapsed": elapsed, "steps": steps, "partition": resolved,
                "step_bytes": step_bytes, "launch_bytes": float(last_bytes),
                "value": float(sum(step_bytes)) / elapsed / 1e9,
                "host_us": self.host_s / steps * 1e6,
                "tokens_per_s": self.wl.B * steps / elapsed, "cold": cold, "warm": warm}

    def launch_pass(self, launches, flush):
        """HIP events on the launching stream around each decode launch and
        each merge launch, `launches` times (after 5 untimed), rotating over
        the layers.  With `flush`, a 1 GiB streaming read of another buffer
        runs before each launch, outside the events, so the pools come from
        HBM (cold); without it the same layer is decoded back to back (warm:
        whatever the 256 MiB Infinity Cache still holds)."""
        torch, pkv = self.torch, self.pkv
        lib, desc = pkv._lib, ctypes.byref(self.desc)
        if not hasattr(self, "_flush"):
            self._flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
            self._sink = torch.empty(8192, dtype=torch.int32, device="cuda")
            pkv.pkv_bench_flush(self._flush)
        k = (self.steps_done - 1) % 2  # the metadata buffers of the last step
        stream = torch.cuda.current_stream()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)]
              for _ in range(launches + 5)]
        for i, (e0, e1, e2) in enumerate(ev):
            layer = i % self.layers if flush else 0
            a = ctypes.byref(self.args[k][layer])
            if flush:
                pkv.pkv_bench_stream_read(self._flush, self._sink)
            e0.record(stream)
            pkv._check(lib.pkv_paged_decode(desc, a, self.stream))
            e1.record(stream)
            pkv._check(lib.pkv_lse_reduce(desc, a, self.stream))
            e2.record(stream)
        torch.cuda.synchronize()
        dec = np.array([a.elapsed_time(b) for a, b, _ in ev[5:]]) * 1e3
        mrg = np.array([b.elapsed_time(c) for _, b, c in ev[5:]]) * 1e3
        tot = dec + mrg
        pct = lambda x: [round(float(np.percentile(x, q)), 3) for q in (10, 50, 90)]  # noqa: E731
        return {"launches": launches, "decode_avg_us": float(dec.mean()),
                "decode_p10_median_p90_us": pct(dec), "merge_avg_us": float(mrg.mean()),
                "decode_merge_avg_us": float(tot.mean()),
                "decode_merge_p10_median_p90_us": pct(tot)}

    def stream_read_ceiling(self):
        """Achievable streaming-read bandwidth: 2 GiB read with 128-bit loads,
        each wave over its own range of 1 KB runs, four loads in flight."""
        torch, pkv = self.torch, self.pkv
        sink = torch.empty(8192, dtype=torch.int32, device="cuda")
        buf = torch.empty(2 << 30, dtype=torch.uint8, device="cuda")
        pkv.pkv_bench_flush(buf)
        stream = torch.cuda.current_stream()
        rt = []
        for _ in range(6):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            pkv.pkv_bench_stream_read(buf, sink)
            e1.record(stream)
            e1.synchronize()
            rt.append(e0.elapsed_time(e1) / 1e3)
        del buf
        return float((2 << 30) / np.median(rt[1:]) / 1e9)


def copy_blocks_bench(args, wl):
    """pkv_copy_blocks on (1) the copy-on-write copies of one beam-search
    step: every sequence of the batch is forked into `beams` beams at its
    full length, then every beam appends one token, so each partly filled
    last block is copied by all but its last holder; and (2) a large copy of
    half the pool onto the other half.  Each launch is timed with HIP events
    on the launching stream after a 1 GiB streaming read of another buffer,
    so sources come from HBM and no dirty lines are left to write back (as
    after the decode kernels, which only read the pools)."""
    import torch
    import paged_kv_cache_250_amd as pkv

    bench = Bench(wl, 1, 2, args.placement)
    pool, gen = bench.pool, bench.gen
    kp, vp, km, vm = bench.pools[0]
    beams = []
    nxt = wl.B
    for b in range(wl.B):
        beams.append(b)
        for _ in range(args.beams - 1):
            pool.fork(b, nxt, int(gen.lengths[b]))
            beams.append(nxt)
            nxt += 1
    pool.append_batch(np.asarray(beams, np.int64), 1)
    beam_pairs = pool.take_copies()
    pool_bytes, meta_bytes = pkv.pkv_cache_bytes(bench.desc)
    block_bytes = 2 * (pool_bytes + meta_bytes) // gen.num_blocks  # K and V, all heads
    flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    pkv.pkv_bench_flush(flush)
    sink = torch.empty(8192, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()

    def timed(pairs_host, reps):
        pairs = torch.from_numpy(np.ascontiguousarray(pairs_host, np.int32)).cuda()
        times = []
        for _ in range(reps + 2):
            pkv.pkv_bench_stream_read(flush, sink)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            pkv.pkv_copy_blocks(bench.desc, pairs, kp, vp, km, vm)
            e1.record(stream)
            e1.synchronize()
            times.append(e0.elapsed_time(e1) / 1e3)
        t = float(np.mean(times[2:]))
        moved = 2 * len(pairs_host) * block_bytes  # read + written
        return {"pairs": int(len(pairs_host)), "bytes_per_launch": int(moved),
                "avg_us": round(t * 1e6, 3), "min_us": round(min(times[2:]) * 1e6, 3),
                "achieved": round(moved / t / 1e9, 2)}

    beam = timed(beam_pairs, args.steps) if args.copy_case in ("both", "beam") else None
    perm = np.random.default_rng(wl.seed + 31).permutation(gen.num_blocks).astype(np.int32)
    half = gen.num_blocks // 2
    large = timed(np.stack([perm[:half], perm[half:2 * half]], 1), args.steps) \
        if args.copy_case in ("both", "large") else beam
    line = {
        "metric": "copy_blocks: bytes read + written per second (copy-on-write)",
        "value": large["achieved"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "higher_is_better": True, "dtype": "u8", "data": "synthetic",
        "config": {"workload": f"{wl.name}: {wl.description}", "beams": args.beams,
                   "block_bytes_k_and_v": int(block_bytes)},
        "roofline": {"bound": "hbm", "kernel": "copy_blocks_kernel",
                     "achieved": large["achieved"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(large["achieved"] / HBM_PEAK_GBS, 4),
                     "traffic": (traffic_from_profile(wl, "copy_blocks_kernel")
                                 if args.copy_case != "beam" else None),
                     "avg_us": large["avg_us"], "bytes_per_launch": large["bytes_per_launch"]},
        "large_copy": large,
        "beam_step": beam,
    }
    print(json.dumps(line))
    pool.close()


PCIE_PEAK_GBS = 64.0  # PCIe Gen5 x16, one direction


def swap_bench(args, wl):
    """pkv_swap_blocks moving the first half of the batch's sequences to a
    pinned host pool and back (64 MiB staging), after the allocator's
    swap-out / swap-in; each direction timed with HIP events on the
    launching stream, `--steps` times."""
    import torch
    import paged_kv_cache_250_amd as pkv

    bench = Bench(wl, 1, 2, args.placement)
    pool, gen = bench.pool, bench.gen
    kp, vp, km, vm = bench.pools[0]
    half = list(range(wl.B // 2))
    need = sum(-(-int(gen.lengths[b]) // wl.p) for b in half)
    pool.set_host_blocks(need)
    bb = pkv.pkv_swap_block_bytes(bench.desc)
    host = torch.empty(need * bb, dtype=torch.uint8).pin_memory()
    staging = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    t_out, t_in = [], []
    for it in range(args.steps + 1):
        out_pairs = np.concatenate([pool.swap_out(b) for b in half])
        e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        e0.record(stream)
        pkv.pkv_swap_blocks(bench.desc, out_pairs, True, kp, vp, km, vm, host, need, staging)
        e1.record(stream)
        in_pairs = np.concatenate([pool.swap_in(b) for b in half])
        torch.cuda.synchronize()
        e1b = torch.cuda.Event(enable_timing=True)
        e1b.record(stream)
        pkv.pkv_swap_blocks(bench.desc, in_pairs, False, kp, vp, km, vm, host, need, staging)
        e2.record(stream)
        e2.synchronize()
        if it:
            t_out.append(e0.elapsed_time(e1) / 1e3)
            t_in.append(e1b.elapsed_time(e2) / 1e3)
    moved = len(out_pairs) * bb
    out_gbs = moved / float(np.mean(t_out)) / 1e9
    in_gbs = moved / float(np.mean(t_in)) / 1e9
    line = {
        "metric": "swap: KV bytes moved per second between HBM and pinned host memory",
        "value": round(out_gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "higher_is_better": True, "dtype": "u8", "data": "synthetic",
        "config": {"workload": f"{wl.name}: {wl.description}", "sequences": len(half),
                   "blocks": int(len(out_pairs)), "block_bytes": int(bb),
                   "staging_bytes": 64 << 20},
        "roofline": {"bound": "pcie", "achieved": round(out_gbs, 2), "peak": PCIE_PEAK_GBS,
                     "unit": "GB/s", "frac": round(out_gbs / PCIE_PEAK_GBS, 4), "traffic": None,
                     "avg_us": round(float(np.mean(t_out)) * 1e6, 1),
                     "bytes_per_launch": int(moved)},
        "to_host_gbs": round(out_gbs, 2), "to_device_gbs": round(in_gbs, 2),
        "to_device_us": round(float(np.mean(t_in)) * 1e6, 1),
    }
    print(json.dumps(line))
    pool.close()


def prefix_cache_bench(args, wl):
    """Host cost and memory effect of the prefix cache on a RAG-like load
    with the workload's block size: every request is an 800-token shared
    context (one of 4 documents after one system prompt) plus 20 tokens of
    its own; `--steps` rounds of wl.B requests, the oldest half of the
    requests freed after each round (their cached blocks become evictable).
    Token ids are seeded; the allocator runs in the library."""
    import paged_kv_cache_250_amd as pkv

    rng = np.random.default_rng(wl.seed + 101)
    p = wl.p
    system = rng.integers(0, 32000, 200).astype(np.int32)
    docs = [rng.integers(0, 32000, 600).astype(np.int32) for _ in range(4)]
    rounds = max(args.steps, 2)
    prompts = [np.concatenate([system, docs[int(rng.integers(0, 4))],
                               rng.integers(0, 32000, 20).astype(np.int32)])
               for _ in range(rounds * wl.B)]
    need = -(-len(prompts[0]) // p)
    num_blocks = need * wl.B  # room for one round without sharing
    pool = pkv.BlockPool(num_blocks, p)
    live, seq, cached, t_alloc, t_free, n_free = [], 0, 0, 0.0, 0.0, 0
    peak_used = 0
    for r in range(rounds):
        for i in range(wl.B):
            t0 = time.perf_counter()
            cached += pool.allocate_cached(seq, prompts[seq])
            t_alloc += time.perf_counter() - t0
            live.append(seq)
            seq += 1
        peak_used = max(peak_used, pool.stats()[1])
        t0 = time.perf_counter()
        for s_ in live[: len(live) // 2]:
            pool.free(s_)
        t_free += time.perf_counter() - t0
        n_free += len(live) // 2
        live = live[len(live) // 2:]
    total = sum(len(x) for x in prompts)
    cblocks, evictable, hits, queries = pool.cache_stats()
    line = {
        "metric": "prefix cache: host us per cached allocation, KV tokens reused",
        "value": round(t_alloc / seq * 1e6, 3), "unit": "us", "higher_is_better": False,
        "n_gpus": 1, "steps": rounds, "data": "synthetic token ids (seeded)",
        "config": {"workload": f"RAG-like prompts, block size {p}", "requests": seq,
                   "prompt_tokens": int(len(prompts[0])), "pool_blocks": num_blocks},
        "tokens_reused": int(cached), "tokens_total": int(total),
        "compute_saved_frac": round(cached / total, 4),
        "blocks_per_request_peak": round(peak_used / wl.B, 2),
        "blocks_per_request_unshared": need,
        "block_hit_rate": round(hits / max(queries, 1), 4),
        "free_us_per_request": round(t_free / max(n_free, 1) * 1e6, 3),
        "cached_blocks": cblocks, "evictable_blocks": evictable,
    }
    print(json.dumps(line))
    pool.close()


# ------------------------------------------------------------- profiles

HERE = os.path.dirname(os.path.abspath(__file__))
PROFILES = os.path.join(HERE, "profiles")
COPY_BYTES = 1 << 30
COUNTER_STEPS = 4  # --warmup 1 --steps 3 in the profiling commands
KERNEL_SOURCES = ("paged_kv_cache_250_amd/csrc/pkv_decode.hip",
                  "paged_kv_cache_250_amd/csrc/pkv_device.h",
                  "paged_kv_cache_250_amd/csrc/pkv_internal.h",
                  "paged_kv_cache_250_amd/build.py")
COPY_KERNEL_SOURCES = ("paged_kv_cache_250_amd/csrc/pkv_cache.hip",
                       "paged_kv_cache_250_amd/csrc/pkv_internal.h",
                       "paged_kv_cache_250_amd/build.py")


def kernel_source_hash(kernel: str = "") -> str:
    """sha256 over a kernel's sources and build flags."""
    h = hashlib.sha256()
    for rel in (COPY_KERNEL_SOURCES if kernel == "copy_blocks_kernel" else KERNEL_SOURCES):
        with open(os.path.join(HERE, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def decode_kernel_name(wl, resolved_partition: int) -> str:
    """The kernel a decode call launches: one pass per (sequence, KV head)
    for partition -1; otherwise the unit stream (balanced split or fixed
    partitions), or one workgroup per partition item beyond 4096 sequences."""
    if resolved_partition == -1:
        return "paged_decode_kernel"
    return "streamk_decode_kernel" if wl.B <= 4096 else "partition_decode_kernel"


def profile_path(wl, kernel: str) -> str:
    return os.path.join(PROFILES, f"{kernel}_{wl.name}.txt")


def read_profile(path: str) -> dict:
    out = {}
    if not os.path.exists(path):
        return out
    with open(path) as f:
        for line in f:
            if line.startswith("#") or ":" not in line:
                continue
            k, v = line.split(":", 1)
            out[k.strip()] = v.strip()
    return out


def traffic_from_profile(wl, kernel: str):
    """HBM bytes per launch from the committed counters, or None when they
    were taken on other kernel sources."""
    prof = read_profile(profile_path(wl, kernel))
    if not prof or prof.get("source_sha256") != kernel_source_hash(kernel):
        return None
    return float(prof["traffic_bytes_per_launch"])


def traffic_ratio_from_profile(wl, kernel: str):
    """Counter traffic over the algorithmic bytes of the same (counter) runs."""
    prof = read_profile(profile_path(wl, kernel))
    if not prof or prof.get("source_sha256") != kernel_source_hash(kernel) \
            or "traffic_ratio" not in prof:
        return None
    return float(prof["traffic_ratio"])


def copy_calibration():
    import torch

    import paged_kv_cache_250_amd as pkv

    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    pkv.pkv_bench_flush(src)
    torch.cuda.synchronize()
    for _ in range(5):
        pkv.pkv_bench_copy(dst, src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "launches": 5}))


def _csv_rows(folder: str, suffix: str):
    paths = glob.glob(os.path.join(folder, "**", "*" + suffix), recursive=True)
    if not paths:
        raise SystemExit(f"no *{suffix} under {folder}")
    rows = []
    for path in paths:
        with open(path) as f:
            rows += list(csv.DictReader(f))
    return rows


def _counter_mean(folder: str, counter: str, kernel_part: str):
    vals = [float(r["Counter_Value"]) for r in _csv_rows(folder, "counter_collection.csv")
            if r["Counter_Name"] == counter and kernel_part in r["Kernel_Name"]]
    if not vals:
        raise SystemExit(f"no {counter} rows for {kernel_part} in {folder}")
    return float(np.mean(vals)), len(vals)


def summarize_profiles(args, wl):
    stats_dir, fetch_dir, write_dir, cfetch_dir, cwrite_dir = args.summarize_profiles
    kernel = args.kernel or decode_kernel_name(
        wl, wl.partition if args.partition is None else args.partition)
    tag = f"::{kernel}<" if kernel != "copy_blocks_kernel" else f"::{kernel}("
    stats = [r for r in _csv_rows(stats_dir, "kernel_stats.csv")]
    mine = [r for r in stats if tag in r["Name"]]
    if len(mine) != 1:
        raise SystemExit(f"expected one {kernel} instantiation in the stats, got {len(mine)}")
    k = mine[0]
    fetch, nf = _counter_mean(fetch_dir, "FETCH_SIZE", tag)
    write, nw = _counter_mean(write_dir, "WRITE_SIZE", tag)
    cfetch, _ = _counter_mean(cfetch_dir, "FETCH_SIZE", "copy_kernel")
    cwrite, _ = _counter_mean(cwrite_dir, "WRITE_SIZE", "copy_kernel")
    fscale = COPY_BYTES / 1024.0 / cfetch
    wscale = COPY_BYTES / 1024.0 / cwrite
    traffic = (fetch * fscale + write * wscale) * 1024.0
    # the counter runs take COUNTER_STEPS steps: their launches read the
    # workload's lengths plus that many tokens
    import workloads
    alg = None if kernel == "copy_blocks_kernel" else \
        unique_tokens(workloads.plan(wl).lengths + COUNTER_STEPS, wl) * kv_bytes_per_token(wl)
    lines = [
        f"# rocprofv3 summary: {kernel}, workload {wl.name} ({wl.description})",
        "# commands (run from the repository root):",
        *[f"#   {c}" for c in args.command.split(";;") if c.strip()],
        "# FETCH_SIZE and WRITE_SIZE are KiB per dispatch; each is scaled by what it reads",
        f"# for the copy kernel moving {COPY_BYTES} bytes (read and written once).",
        f"kernel: {k['Name']}",
        f"source_sha256: {kernel_source_hash(kernel)}",
        f"calls: {k['Calls']}",
        f"avg_ns: {float(k['AverageNs']):.1f}",
        f"min_ns: {float(k['MinNs']):.1f}",
        f"max_ns: {float(k['MaxNs']):.1f}",
        f"fetch_kib_per_dispatch: {fetch:.1f}  (mean of {nf})",
        f"write_kib_per_dispatch: {write:.1f}  (mean of {nw})",
        f"copy_fetch_kib: {cfetch:.1f}",
        f"copy_write_kib: {cwrite:.1f}",
        f"fetch_scale: {fscale:.4f}",
        f"write_scale: {wscale:.4f}",
        f"traffic_bytes_per_launch: {traffic:.0f}",
        *([] if alg is None else [
            f"counter_run_steps: {COUNTER_STEPS}",
            f"algorithmic_bytes_per_launch: {alg}  (the counter runs' launches)",
            f"traffic_ratio: {traffic / alg:.4f}"]),
        "# all kernels of the traced run (kernel_stats.csv):",
    ]
    for r in sorted(stats, key=lambda r: -float(r["TotalDurationNs"])):
        name = r["Name"] if len(r["Name"]) < 90 else r["Name"][:87] + "..."
        lines.append(f"#   {name:90s} calls {int(r['Calls']):5d}  avg {float(r['AverageNs']) / 1e3:9.2f} us"
                     f"  total {float(r['Percentage']):6.2f}%")
    os.makedirs(PROFILES, exist_ok=True)
    out = profile_path(wl, kernel)
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(out)


SIMDS = 256 * 4       # MI355X: 256 compute units of 4 SIMDs
CLOCK_HZ = 2.4e9      # peak engine clock
VALU_CYCLES = 4       # a wave64 VALU instruction occupies a 16-lane SIMD for 4 cycles


def units_per_launch(wl, lengths: np.ndarray) -> int:
    """16-token units one decode launch processes: ceil(n / 16) per (sequence,
    KV head), a shared prefix counted for every sequence that reads it."""
    return int(np.sum(-(-np.asarray(lengths, np.int64) // 16))) * wl.Hkv


def summarize_counters(args, wl):
    """Per-dispatch means of every counter in the --pmc folders for the
    decode kernel of the workload, and the same per 16-token unit (each unit
    is processed by one wave)."""
    import workloads

    kernel = args.kernel or decode_kernel_name(
        wl, wl.partition if args.partition is None else args.partition)
    tag = f"::{kernel}<"
    vals = {}
    for folder in args.summarize_counters:
        for r in _csv_rows(folder, "counter_collection.csv"):
            if tag in r["Kernel_Name"]:
                key = r["Counter_Name"]
                vals.setdefault(key, {}).setdefault(r.get("Dispatch_Id", len(vals)), 0.0)
                vals[key][r.get("Dispatch_Id", len(vals))] += float(r["Counter_Value"])
    if not vals:
        raise SystemExit(f"no counters for {kernel} in {args.summarize_counters}")
    lengths = workloads.plan(wl).lengths + COUNTER_STEPS
    units = units_per_launch(wl, lengths)
    mean = {k: float(np.mean(list(v.values()))) for k, v in vals.items()}
    lines = [
        f"# rocprofv3 hardware counters: {kernel}, workload {wl.name} ({wl.description})",
        "# commands (run from the repository root):",
        *[f"#   {c}" for c in args.command.split(";;") if c.strip()],
        "# values are means per dispatch of the decode kernel; 'per unit' divides by the",
        "# 16-token units one launch processes (ceil(n/16) per sequence and KV head).",
        f"kernel: {kernel}",
        f"source_sha256: {kernel_source_hash(kernel)}",
        f"units_per_launch: {units}",
    ]
    for k in sorted(mean):
        lines.append(f"{k}: {mean[k]:.1f}  (dispatches {len(vals[k])}; per unit "
                     f"{mean[k] / units:.2f})")
    if "SQ_INSTS_VALU" in mean:
        t = mean["SQ_INSTS_VALU"] * VALU_CYCLES / (SIMDS * CLOCK_HZ)
        lines.append(f"valu_issue_us: {t * 1e6:.1f}  (VALU instructions x {VALU_CYCLES} cycles "
                     f"spread over {SIMDS} SIMDs at {CLOCK_HZ / 1e9:.1f} GHz)")
    if "SQ_WAIT_INST_ANY" in mean and "SQ_WAVE_CYCLES" in mean:
        lines.append(f"wait_inst_any_frac: {mean['SQ_WAIT_INST_ANY'] / mean['SQ_WAVE_CYCLES']:.3f}"
                     "  (wave cycles waiting for a dependency)")
    if "SQ_ACTIVE_INST_VALU" in mean and "SQ_WAVE_CYCLES" in mean:
        lines.append(f"active_valu_frac: "
                     f"{mean['SQ_ACTIVE_INST_VALU'] / mean['SQ_WAVE_CYCLES']:.3f}"
                     "  (wave cycles issuing VALU)")
    os.makedirs(PROFILES, exist_ok=True)
    out = os.path.join(PROFILES, f"{kernel}_{wl.name}_{args.counters_name}.txt")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(out)


def arithmetic_dtype(wl) -> str:
    """The cache's storage type and the matrix-core operand type the decode
    computes its products in (fp32 accumulation throughout)."""
    product = {"f16": "f16", "bf16": "bf16", "fp8_e4m3": wl.io_dtype, "fp8_e5m2": wl.io_dtype,
               "fp8_e4m3_block": wl.io_dtype, "int4_asym_g32": "f16"}[wl.kv_dtype]
    return wl.kv_dtype if wl.kv_dtype == product else f"{wl.kv_dtype}/{product}"


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(gen, wl, bytes_per_tok):
    """Time the fp64 oracle's paged attention over the workload's sequences."""
    import oracle
    from oracle.state import oracle_state

    log("cpu baseline: building oracle pools")
    d, pools, bt, cl, _ = oracle_state(gen)
    # bounded sample: the first sequences up to ~5 M (token, query head) pairs
    # (the whole Llama-3-8B-shaped batch)
    budget = 5_000_000
    mask = np.zeros(wl.B, np.uint8)
    acc = 0
    for b in range(wl.B):
        mask[b] = 1
        acc += int(gen.lengths[b]) * wl.Hq
        if acc >= budget:
            break
    ntok = int(gen.lengths[mask.astype(bool)].sum())
    scale = float(np.float32(1 / math.sqrt(wl.D)))
    # repeat the sample until about 10 s of wall-clock have passed
    runs, t0 = 0, time.perf_counter()
    while True:
        oracle.paged_attention(d, gen.q_bits, pools, bt, cl, scale, seq_mask=mask)
        runs += 1
        total = time.perf_counter() - t0
        if total >= 10.0 or runs >= 200:
            break
    t = total / runs
    cores = oracle.num_threads()
    log(f"cpu baseline: {int(mask.sum())} sequences, {ntok} tokens, {runs} runs, {t:.3f} s each "
        f"on {cores} threads")
    return {"value": round(ntok * bytes_per_tok / t / 1e9, 4), "unit": "GB/s", "cores": cores,
            "cpu_model": cpu_model(), "host_cpus": len(os.sched_getaffinity(0)),
            "kind": "oracle",
            "sample": f"one decode step of one layer over the first {int(mask.sum())} of "
                      f"{wl.B} sequences ({ntok} tokens), repeated {runs} times in "
                      f"{total:.1f} s ({t:.3f} s each)",
            "tokens_per_s": round(int(mask.sum()) / t, 3)}


def main(argv=None):
    args = parse(argv)
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): it "
              "measures one GPU's share; the decode shards by sequence or KV head without "
              "any exchange.", file=sys.stderr)
        sys.exit(2)
    import workloads

    if args.summarize_profiles:
        summarize_profiles(args, workloads.get(args.workload))
        return
    if args.summarize_counters:
        summarize_counters(args, workloads.get(args.workload))
        return
    import torch

    if args.prefix_cache:  # host only
        wl = workloads.get(args.workload)
        if args.block_size is not None:
            wl = wl.replace(p=args.block_size)
        prefix_cache_bench(args, wl)
        return
    if not torch.cuda.is_available():
        print("no GPU visible: the bench needs an MI355X", file=sys.stderr)
        sys.exit(3)
    if args.copy_calibration:
        copy_calibration()
        return
    wl = workloads.get(args.workload)
    if args.block_size is not None and args.block_size != wl.p:
        wl = wl.replace(name=f"{wl.name}-p{args.block_size}", p=args.block_size,
                        description=f"{wl.description}; block size {args.block_size}")
    if args.kv_dtype is not None and args.kv_dtype != wl.kv_dtype:
        wl = wl.replace(name=f"{wl.name}-{args.kv_dtype}", kv_dtype=args.kv_dtype,
                        description=f"{wl.description}; {args.kv_dtype} cache")
    if args.copy_blocks:
        copy_blocks_bench(args, wl)
        return
    if args.swap:
        swap_bench(args, wl)
        return

    partition = wl.partition if args.partition is None else args.partition
    log(f"workload {wl.name}: {wl.description}; {args.layers} layers per step; "
        f"{args.placement} placement")
    bench = Bench(wl, args.layers, args.warmup + args.steps, args.placement, upload=args.upload)
    r = bench.run(partition, args.warmup, args.steps, args.launches)
    cold, warm = r["cold"], r["warm"]
    achieved = r["launch_bytes"] / cold["decode_avg_us"] / 1e3
    attention = r["launch_bytes"] / cold["decode_merge_avg_us"] / 1e3
    log(f"step {r['elapsed'] / args.steps * 1e3:.4f} ms, whole step {r['value']:.1f} GB/s; "
        f"decode kernel (cold, {cold['launches']} launches) avg {cold['decode_avg_us']:.2f} us "
        f"= {achieved:.1f} GB/s, with its merge {cold['decode_merge_avg_us']:.2f} us = "
        f"{attention:.1f} GB/s; warm decode {warm['decode_avg_us']:.2f} us")
    ceiling = bench.stream_read_ceiling()
    log(f"streaming-read ceiling {ceiling:.1f} GB/s")
    cpu = None if args.no_cpu else cpu_baseline(bench.gen, wl, bench.bytes_per_tok)
    kernel = decode_kernel_name(wl, r["partition"])
    # the committed counters were taken on the workload's own placement and split
    same_run = args.placement == "random" and partition == wl.partition
    traffic = traffic_from_profile(wl, kernel) if same_run else None
    if traffic is not None:
        traffic = round(traffic, 0)
    line = {
        "metric": METRIC,
        "value": round(r["value"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["elapsed"] / args.steps * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": arithmetic_dtype(wl),
        "data": f"synthetic (seeded N(0,1) Q/K/V, {args.placement} block placement)",
        "config": {
            "workload": f"{wl.name}: {wl.description}",
            "batch": wl.B, "q_heads": wl.Hq, "kv_heads": wl.Hkv, "head_dim": wl.D,
            "block_size": wl.p, "kv_dtype": wl.kv_dtype, "layers_per_step": args.layers,
            "partition_tokens": r["partition"],
            "context_tokens_first_step": int(r["step_bytes"][0] // bench.bytes_per_tok
                                             // args.layers),
        },
        "pct_hbm_peak": round(100.0 * r["value"] / HBM_PEAK_GBS, 2),
        "tokens_per_s": round(r["tokens_per_s"], 1),
        "tokens_per_s_per_layer": round(r["tokens_per_s"] * args.layers, 1),
        "host_us_per_step": round(r["host_us"], 2),
        "roofline": {
            "bound": "hbm",
            "kernel": kernel,
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            # traffic over the algorithmic bytes of the counter runs themselves
            # (they take fewer steps, so their contexts are a little shorter)
            "traffic_ratio": traffic_ratio_from_profile(wl, kernel) if same_run else None,
            "avg_us": round(cold["decode_avg_us"], 3),
            "p10_median_p90_us": cold["decode_p10_median_p90_us"],
            "launches_timed": cold["launches"],
            "bytes_per_launch": int(r["launch_bytes"]),
            "cache": "cold: a 1 GiB streaming read of another buffer before each launch",
            "attention_avg_us": round(cold["decode_merge_avg_us"], 3),
            "attention_p10_median_p90_us": cold["decode_merge_p10_median_p90_us"],
            "attention_frac": round(attention / HBM_PEAK_GBS, 4),
            "merge_avg_us": round(cold["merge_avg_us"], 3),
            "warm": {"avg_us": round(warm["decode_avg_us"], 3),
                     "p10_median_p90_us": warm["decode_p10_median_p90_us"],
                     "attention_avg_us": round(warm["decode_merge_avg_us"], 3),
                     "frac": round(r["launch_bytes"] / warm["decode_avg_us"] / 1e3
                                   / HBM_PEAK_GBS, 4)},
            "stream_read_ceiling_gbs": round(ceiling, 1),
            "frac_of_stream_ceiling": round(achieved / ceiling, 4),
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(line))
    bench.pool.close()


if __name__ == "__main__":
    main()
