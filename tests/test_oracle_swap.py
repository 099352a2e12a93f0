"""Pins of swapping in the oracle's allocator model and of its block move.

"Reducing LLM Inference Latency: KV Cache Quantization and PagedAttention in
vLLM" (section "Prefill Swapping and GPU Thrashing") moves KV pages to host
memory when the pool is exhausted.  Whatever the policy, the result is
fixed: a sequence swapped out and back in must read back exactly its own
K/V, although its device blocks were reused and overwritten meanwhile, and
no block another sequence still reads may leave the device.  The replay
below checks that token by token through the oracle's reshape_and_cache,
block move and gather, with the allocator's invariants after every step.
"""
import numpy as np
import pytest

import oracle
from oracle import brute
from oracle.allocator_model import (AllocatorError, BlockPoolModel, CopiesPending, OutOfBlocks,
                                    Swapped)
from common import softmax_scale
from test_oracle_cow import _bits16, _exact_rows, check_invariants


def check_swap_invariants(m: BlockPoolModel):
    check_invariants(m) if not m.on_host else None
    host_used = [b for s, f in m.on_host.items() for b, x in zip(m.tables[s], f) if x]
    assert len(set(host_used)) == len(host_used)
    assert not set(host_used) & set(m.host_free)
    assert len(host_used) + len(m.host_free) == m.num_host_blocks
    counts = np.zeros(m.num_blocks, np.int64)
    for s, t in m.tables.items():
        f = m.on_host.get(s, [False] * len(t))
        for b, x in zip(t, f):
            if not x:
                counts[b] += 1
    assert list(counts) == m.ref


def test_swap_example():
    m = BlockPoolModel(6, 4)
    m.set_host_blocks(4)
    m.allocate(0, 10)                      # blocks 0, 1, 2
    m.fork(0, 1, 4)                        # block 0 shared
    m.append(1, 1)                         # 1 takes block 3
    assert m.swap_out(0) == [(1, 0), (2, 1)]   # block 0 is shared: it stays
    assert m.tables[0] == [0, 0, 1] and m.on_host[0] == [False, True, True]
    assert list(m.free) == [4, 5, 1, 2] and m.ref[0] == 2
    with pytest.raises(Swapped):
        m.append(0, 1)
    with pytest.raises(Swapped):
        m.block_tables([0], 3)
    m.allocate(2, 12)                      # reuses 4, 5, 1: the swapped data is overwritten
    assert m.tables[2] == [4, 5, 1] and list(m.free) == [2]
    with pytest.raises(OutOfBlocks):
        m.swap_in(0)                        # needs 2 device blocks
    assert m.on_host[0] == [False, True, True]
    m.free_seq(1)                          # block 0 keeps 0's reference; block 3 is freed
    assert m.ref[0] == 1 and list(m.free) == [2, 3]
    assert m.swap_in(0) == [(2, 0), (3, 1)]
    assert m.tables[0] == [0, 2, 3] and list(m.host_free) == [2, 3, 0, 1]
    assert m.swap_stats() == (0, 4, 0)
    check_swap_invariants(m)


def test_swap_in_takes_blocks_in_table_order():
    m = BlockPoolModel(5, 4)
    m.set_host_blocks(3)
    m.allocate(0, 8)                       # blocks 0, 1
    assert m.swap_out(0) == [(0, 0), (1, 1)]
    m.allocate(1, 4)                       # block 2
    assert m.swap_in(0) == [(3, 0), (4, 1)]
    assert m.tables[0] == [3, 4] and list(m.host_free) == [2, 0, 1]
    with pytest.raises(AllocatorError):
        m.swap_in(0)                        # not swapped out
    check_swap_invariants(m)


def test_swap_all_or_nothing():
    m = BlockPoolModel(4, 4)
    m.set_host_blocks(1)
    m.allocate(0, 8)
    before = (list(m.free), list(m.ref), {k: list(v) for k, v in m.tables.items()})
    with pytest.raises(OutOfBlocks):
        m.swap_out(0)                       # needs 2 host blocks
    assert (list(m.free), list(m.ref), {k: list(v) for k, v in m.tables.items()}) == before
    m.set_host_blocks(2)
    m.swap_out(0)
    m.allocate(1, 16)                       # all 4 device blocks
    with pytest.raises(OutOfBlocks):
        m.swap_in(0)
    assert 0 in m.on_host
    check_swap_invariants(m)
    # refused while copy-on-write copies are pending
    m = BlockPoolModel(6, 4)
    m.set_host_blocks(4)
    m.allocate(0, 5)
    m.fork(0, 1, 5)
    m.append(1, 1)
    with pytest.raises(CopiesPending):
        m.swap_out(0)
    assert m.take_copies() == [(1, 2)]
    # block 0 is shared with sequence 1 and stays; block 1 is 0's alone after the copy
    assert m.swap_out(0) == [(1, 0)]
    assert m.tables[0] == [0, 0] and m.on_host[0] == [False, True]
    check_swap_invariants(m)



@pytest.mark.parametrize("kv", ["f16", "fp8_e4m3", "int4_asym_g32"])
def test_swapped_sequences_read_back_their_own_kv(orc, kv):
    dt = "f16" if kv == "f16" else "bf16"
    p = 4 if kv == "f16" else 16
    Hkv, D, Hq, nb = 2, 32, 4, 30
    rng = np.random.default_rng(23)
    m = BlockPoolModel(nb, p, rng.permutation(nb))
    m.set_host_blocks(24)
    d = oracle.desc(kv, dt, Hkv, D, p, nb)
    dev = oracle.pool_arrays(kv, nb, Hkv, p, D, fill=0x11)
    host = oracle.pool_arrays(kv, 24, Hkv, p, D, fill=0x22)
    hist, rows_k, rows_v, nxt = {}, [], [], 0
    swaps_in = 0

    def new_rows(k):
        ids = []
        for _ in range(k):
            x = rng.standard_normal((2, Hkv, D))
            rows_k.append(_bits16(x[0], dt))
            rows_v.append(_bits16(x[1], dt))
            ids.append(len(rows_k) - 1)
        return ids

    def write(slots, ids):
        if ids:
            oracle.reshape_and_cache(d, np.stack([rows_k[i] for i in ids]),
                                     np.stack([rows_v[i] for i in ids]),
                                     np.asarray(slots, np.int64), dev)

    for step in range(120):
        live = [s for s in hist if s not in m.on_host]
        out = [s for s in hist if s in m.on_host]
        op = int(rng.integers(0, 6))
        try:
            if op == 0:
                n = int(rng.integers(1, 3 * p))
                m.allocate(nxt, n)
                ids = new_rows(n)
                write([m.slot(nxt, t) for t in range(n)], ids)
                hist[nxt] = ids
                nxt += 1
            elif op == 1 and live:
                s = live[int(rng.integers(0, len(live)))]
                k = int(rng.integers(1, p))
                n0 = m.ntok[s]
                got = m.append(s, k)
                oracle.copy_blocks(dev, m.take_copies())
                ids = new_rows(k)
                write(got, ids)
                hist[s] = hist[s] + ids
                assert got == [m.slot(s, t) for t in range(n0, n0 + k)]
            elif op == 2 and live:
                s = live[int(rng.integers(0, len(live)))]
                pre = int(rng.integers(0, m.ntok[s] + 1))
                m.fork(s, nxt, pre)
                hist[nxt] = hist[s][:pre]
                nxt += 1
            elif op == 3 and live:
                s = live[int(rng.integers(0, len(live)))]
                oracle.swap_blocks(dev, host, m.swap_out(s), to_host=True)
            elif op == 4 and out:
                s = out[int(rng.integers(0, len(out)))]
                oracle.swap_blocks(dev, host, m.swap_in(s), to_host=False)
                swaps_in += 1
            elif op == 5 and len(hist) > 3:
                s = list(hist)[int(rng.integers(0, len(hist)))]
                m.free_seq(s)
                del hist[s]
        except OutOfBlocks:
            pass
        check_swap_invariants(m)
        for s in hist:
            if s in m.on_host:
                continue
            n = len(hist[s])
            for h in range(Hkv):
                K, V = oracle.gather(d, dev, np.asarray(m.tables[s], np.int32), n, h)
                if n == 0:
                    continue
                kx = np.stack([rows_k[i][h] for i in hist[s]])
                vx = np.stack([rows_v[i][h] for i in hist[s]])
                assert np.array_equal(K, _exact_rows(kx, dt, kv)), (step, s, h)
                assert np.array_equal(V, _exact_rows(vx, dt, kv)), (step, s, h)
    assert swaps_in >= 5, "the replay should swap sequences back in"
    for s in [s for s in hist if s in m.on_host]:
        try:
            oracle.swap_blocks(dev, host, m.swap_in(s), to_host=False)
        except OutOfBlocks:
            m.free_seq(s)
            del hist[s]
    assert hist
    seqs = sorted(hist)
    W = max(1, max(len(m.tables[s]) for s in seqs))
    bt, cl = m.block_tables(seqs, W)
    qb = _bits16(rng.standard_normal((len(seqs), Hq, D)), dt)
    sc = softmax_scale(D)
    o = oracle.paged_attention(d, qb, dev, bt, cl, sc)
    q = oracle.decode16(qb, dt)
    for i, s in enumerate(seqs):
        for h in range(Hq):
            if not hist[s]:
                continue
            K = _exact_rows(np.stack([rows_k[j][h // 2] for j in hist[s]]), dt, kv)
            V = _exact_rows(np.stack([rows_v[j][h // 2] for j in hist[s]]), dt, kv)
            assert np.allclose(o[i, h], brute.attention_row(q[i, h], K, V, sc), rtol=1e-12,
                               atol=1e-13)
