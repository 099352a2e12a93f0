"""Oracle-side state of a generated workload (test infrastructure only):
the allocator model builds the block tables, and every stored token is
written to host pools by the oracle's reshape_and_cache."""
from __future__ import annotations

import numpy as np

import oracle
from oracle.allocator_model import BlockPoolModel


def table_width(gen) -> int:
    return max(1, -(-int(gen.lengths.max()) // gen.wl.p))


def oracle_state(gen, width: int | None = None, fill: int = 0):
    """Returns (desc, pools, block_tables, ctx_lens, model)."""
    wl = gen.wl
    model = BlockPoolModel(gen.num_blocks, wl.p, gen.free_order)
    model.run_ops(gen.ops)
    W = width or table_width(gen)
    bt, cl = model.block_tables(list(range(wl.B)), W)
    seq, pos, rows = gen.token_positions()
    tabs = model.tables
    p = wl.p
    slots = np.fromiter((tabs[s][t // p] * p + t % p for s, t in zip(seq.tolist(), pos.tolist())),
                        dtype=np.int64, count=len(seq))
    d = oracle.desc(wl.kv_dtype, gen.in_dtype, wl.Hkv, wl.D, wl.p, gen.num_blocks)
    pools = oracle.pool_arrays(wl.kv_dtype, gen.num_blocks, wl.Hkv, wl.p, wl.D, fill=fill)
    oracle.reshape_and_cache(d, gen.k_bits[rows], gen.v_bits[rows], slots, pools)
    return d, pools, bt, cl, model
