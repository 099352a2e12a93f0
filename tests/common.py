"""Shared test helpers: build the oracle-side state of a generated workload."""
from __future__ import annotations

import math

import numpy as np

import oracle
from oracle.allocator_model import BlockPoolModel
from workloads import Generated


def softmax_scale(D: int) -> float:
    return float(np.float32(1.0 / math.sqrt(D)))


def table_width(gen: Generated) -> int:
    return max(1, -(-int(gen.lengths.max()) // gen.wl.p))


def oracle_state(gen: Generated, width: int | None = None, fill: int = 0):
    """Allocate the workload with the Python allocator model, write every
    stored token through the oracle's reshape_and_cache and return
    (desc, pools, block_tables, ctx_lens, model)."""
    wl = gen.wl
    model = BlockPoolModel(gen.num_blocks, wl.p, gen.free_order)
    model.run_ops(gen.ops)
    W = width or table_width(gen)
    bt, cl = model.block_tables(list(range(wl.B)), W)
    seq, pos, rows = gen.token_positions()
    slots = np.array([model.tables[s][t // wl.p] * wl.p + t % wl.p for s, t in zip(seq, pos)],
                     dtype=np.int64)
    d = oracle.desc(wl.kv_dtype, gen.in_dtype, wl.Hkv, wl.D, wl.p, gen.num_blocks)
    pools = oracle.pool_arrays(wl.kv_dtype, gen.num_blocks, wl.Hkv, wl.p, wl.D, fill=fill)
    oracle.reshape_and_cache(d, gen.k_bits[rows], gen.v_bits[rows], slots, pools)
    return d, pools, bt, cl, model


def dequant_rows(gen: Generated, which: str, b: int, h: int) -> np.ndarray:
    """Exact values of the cached K or V of sequence b, KV head h, computed
    from the raw inputs with the oracle's codec functions (fp64 [n, D])."""
    bits = (gen.k_bits if which == "k" else gen.v_bits)[gen.rows(b), h]
    x = oracle.decode16(bits, gen.in_dtype)
    kv = gen.wl.kv_dtype
    if kv in ("f16", "bf16"):
        return x
    if kv == "fp8_e4m3":
        codes, scales = oracle.fp8_quantize_rows(x.astype(np.float32))
        return oracle.fp8_dequant(codes, scales).astype(np.float64)
    codes, s, z = oracle.int4_quantize_rows(x.astype(np.float32))
    return oracle.int4_dequant(codes, s, z).astype(np.float64)
