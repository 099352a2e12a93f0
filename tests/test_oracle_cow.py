"""Pins of copy-on-write in the oracle's allocator model and of the oracle's
block copy.

"KV Cache Compression & Paged Attention Deep Dive" names copy-on-write for
forked sequences and per-block reference counts (sections "PagedAttention:
Operating System-Inspired Memory Management" and "Implementation Details:
PagedAttention Kernel and Page Table") without spelling out the steps.
Whatever the steps, two facts fix the result: every sequence must read back
exactly the tokens of its own history (a paged cache equals a contiguous one,
"Reducing LLM Inference Latency...", section "PagedAttention: Solving VRAM
Fragmentation"), and no write may land in a block another table still
points at.  These tests replay random forks, appends and frees through the
model, the oracle's copy and its reshape_and_cache, and check both facts
token by token, plus the reference-count and free-list invariants and
attention against textbook softmax over each history.
"""
import numpy as np
import pytest

import oracle
from oracle import brute
from oracle.allocator_model import AllocatorError, BlockPoolModel, CopiesPending, OutOfBlocks
from common import softmax_scale


def _bits16(x, dt):
    return oracle.f16_encode(x) if dt == "f16" else oracle.bf16_encode(x)


def _exact_rows(bits, dt, kv):
    """The values the cache must hold for rows of 16-bit inputs [n, D]."""
    x = oracle.decode16(bits, dt)
    if kv in ("f16", "bf16"):
        return x
    if kv in ("fp8_e4m3", "fp8_e5m2"):
        c, s = oracle.fp8_quantize_rows(x.astype(np.float32), kv[4:])
        return oracle.fp8_dequant(c, s, kv[4:]).astype(np.float64)
    c, s, z = oracle.int4_quantize_rows(x.astype(np.float32))
    return oracle.int4_dequant(c, s, z).astype(np.float64)


def check_invariants(m: BlockPoolModel):
    counts = np.zeros(m.num_blocks, np.int64)
    for t in m.tables.values():
        for b in t:
            counts[b] += 1
    assert list(counts) == m.ref
    free = list(m.free) + list(m.lru)
    assert len(set(free)) == len(free)
    assert all(m.ref[b] == 0 for b in free)
    assert sum(1 for r in m.ref if r == 0) == len(free)
    assert all(b in m.entry for b in m.lru)
    assert all(m.cache[key] == b for b, (_, key) in m.entry.items())
    for s, t in m.tables.items():
        assert len(t) == -(-m.ntok[s] // m.p)
    srcs = [a for a, _ in m.copies]
    dsts = [b for _, b in m.copies]
    assert len(set(dsts)) == len(dsts)
    assert not set(srcs) & set(dsts)
    assert all(m.ref[b] == 1 for b in dsts)


class Replay:
    """Random fork / append / free traffic, applied to a model and to host
    pools through the oracle's copy and reshape_and_cache."""

    def __init__(self, kv, dt, seed, num_blocks=40, p=4, Hkv=2, D=32, Hq=4):
        self.rng = np.random.default_rng(seed)
        self.kv, self.dt, self.p, self.Hkv, self.D, self.Hq = kv, dt, p, Hkv, D, Hq
        order = self.rng.permutation(num_blocks)
        self.m = BlockPoolModel(num_blocks, p, order)
        self.d = oracle.desc(kv, dt, Hkv, D, p, num_blocks)
        self.pools = oracle.pool_arrays(kv, num_blocks, Hkv, p, D, fill=0xA5)
        self.hist = {}       # seq -> list of row ids
        self.k_rows = []     # row id -> [Hkv, D] bits
        self.v_rows = []
        self.copies_seen = 0
        self.next_seq = 0

    def _new_rows(self, k):
        ids = []
        for _ in range(k):
            x = self.rng.standard_normal((2, self.Hkv, self.D))
            self.k_rows.append(_bits16(x[0], self.dt))
            self.v_rows.append(_bits16(x[1], self.dt))
            ids.append(len(self.k_rows) - 1)
        return ids

    def _write(self, slots, ids):
        if not ids:
            return
        k = np.stack([self.k_rows[i] for i in ids])
        v = np.stack([self.v_rows[i] for i in ids])
        oracle.reshape_and_cache(self.d, k, v, np.asarray(slots, np.int64), self.pools)

    def step(self):
        m, rng = self.m, self.rng
        live = sorted(self.hist)
        # forks, frees and allocations first (no copies are pending here)
        for _ in range(int(rng.integers(0, 3))):
            op = int(rng.integers(0, 3))
            if op == 0 and live:
                src = live[int(rng.integers(0, len(live)))]
                pre = int(rng.integers(0, m.ntok[src] + 1))
                m.fork(src, self.next_seq, pre)
                self.hist[self.next_seq] = self.hist[src][:pre]
                self.next_seq += 1
            elif op == 1 and live and len(live) > 2:
                s = live[int(rng.integers(0, len(live)))]
                m.free_seq(s)
                del self.hist[s]
            elif op == 2:
                n = int(rng.integers(0, 3 * self.p))
                try:
                    m.allocate(self.next_seq, n)
                except OutOfBlocks:
                    continue
                ids = self._new_rows(n)
                self._write([m.slot(self.next_seq, t) for t in range(n)], ids)
                self.hist[self.next_seq] = ids
                self.next_seq += 1
            live = sorted(self.hist)
        # a batch of appends: copies are taken and run before the new tokens land
        slots, ids = [], []
        for s in live:
            if rng.random() < 0.3:
                continue
            k = int(rng.integers(1, 3))
            n0 = m.ntok[s]
            try:
                got = m.append(s, k)
            except OutOfBlocks:
                continue
            for t, sl in enumerate(got):
                blk = sl // self.p
                assert m.ref[blk] == 1, "a write would land in a shared block"
                assert sl == m.slot(s, n0 + t)
            new = self._new_rows(k)
            self.hist[s] = self.hist[s] + new
            slots += got
            ids += new
        check_invariants(m)
        if m.copies:
            with pytest.raises(CopiesPending):
                m.fork(live[0], 10**6, 0)
            with pytest.raises(CopiesPending):
                m.free_seq(live[0])
        pairs = m.take_copies()
        self.copies_seen += len(pairs)
        oracle.copy_blocks(self.pools, pairs)
        self._write(slots, ids)

    def check_contents(self):
        for s, ids in self.hist.items():
            n = len(ids)
            assert self.m.ntok[s] == n
            row = np.asarray(self.m.tables[s], np.int32)
            for h in range(self.Hkv):
                K, V = oracle.gather(self.d, self.pools, row, n, h)
                if n == 0:
                    continue
                kb = np.stack([self.k_rows[i][h] for i in ids])
                vb = np.stack([self.v_rows[i][h] for i in ids])
                assert np.array_equal(K, _exact_rows(kb, self.dt, self.kv)), (s, h)
                assert np.array_equal(V, _exact_rows(vb, self.dt, self.kv)), (s, h)

    def check_attention(self):
        seqs = sorted(self.hist)
        W = max(1, max(len(self.m.tables[s]) for s in seqs))
        bt, cl = self.m.block_tables(seqs, W)
        q_bits = _bits16(self.rng.standard_normal((len(seqs), self.Hq, self.D)) * 0.5, self.dt)
        sc = softmax_scale(self.D)
        out = oracle.paged_attention(self.d, q_bits, self.pools, bt, cl, sc)
        q = oracle.decode16(q_bits, self.dt)
        G = self.Hq // self.Hkv
        for i, s in enumerate(seqs):
            ids = self.hist[s]
            for h in range(self.Hq):
                if not ids:
                    assert np.all(out[i, h] == 0)
                    continue
                K = _exact_rows(np.stack([self.k_rows[j][h // G] for j in ids]), self.dt, self.kv)
                V = _exact_rows(np.stack([self.v_rows[j][h // G] for j in ids]), self.dt, self.kv)
                ref = brute.attention_row(q[i, h], K, V, sc)
                assert np.allclose(out[i, h], ref, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("kv", ["f16", "bf16", "fp8_e4m3", "int4_asym_g32", "fp8_e5m2"])
def test_forked_histories_read_back_exactly(orc, kv):
    dt = "f16" if kv == "f16" else "bf16"
    p = 4 if kv in ("f16", "bf16") else 16  # quantised layouts need p >= 16 in the oracle too
    r = Replay(kv, dt, seed=11, num_blocks=40 if p == 4 else 24, p=p)
    r.m.allocate(0, 6)
    ids = r._new_rows(6)
    r._write([r.m.slot(0, t) for t in range(6)], ids)
    r.hist[0] = ids
    r.next_seq = 1
    for _ in range(40):
        r.step()
    assert r.copies_seen > 5, "the replay should exercise copy-on-write"
    r.check_contents()
    r.check_attention()


def test_beam_fork_example():
    """Worked example: a 6-token sequence in blocks of 4 is forked twice at
    its full length (beam search), then every beam appends one token."""
    m = BlockPoolModel(8, 4, [5, 2, 7, 0, 1, 3, 4, 6])
    m.allocate(0, 6)                      # blocks 5, 2; block 2 holds tokens 4, 5
    m.fork(0, 1, 6)
    m.fork(0, 2, 6)
    assert m.ref[5] == 3 and m.ref[2] == 3
    assert m.append(0, 1) == [7 * 4 + 2]  # 0 writes into a copy of block 2 (block 7)
    assert m.append(1, 1) == [0 * 4 + 2]  # 1 copies too (block 0)
    assert m.append(2, 1) == [2 * 4 + 2]  # 2 is the last holder: writes in place
    assert m.take_copies() == [(2, 7), (2, 0)]
    assert m.tables == {0: [5, 7], 1: [5, 0], 2: [5, 2]}
    assert m.ref[5] == 3 and [m.ref[b] for b in (7, 0, 2)] == [1, 1, 1]
    # a fork at a block boundary shares only whole blocks: no copy later
    m.fork(2, 3, 4)
    assert m.tables[3] == [5]
    assert m.append(3, 1) == [1 * 4 + 0] and m.take_copies() == []
    # appending to a shared but full last block takes a fresh block, no copy
    m.fork(3, 4, 5)
    m.free_seq(3)
    assert m.append(4, 3) == [1 * 4 + 1, 1 * 4 + 2, 1 * 4 + 3]
    assert m.take_copies() == []
    check_invariants(m)


def test_copy_on_write_all_or_nothing():
    m = BlockPoolModel(3, 4)
    m.allocate(0, 6)                      # blocks 0, 1
    m.fork(0, 1, 6)
    before = (list(m.free), list(m.ref), {k: list(v) for k, v in m.tables.items()})
    with pytest.raises(OutOfBlocks):
        m.append(1, 3)                    # needs a copy and a new block; one is free
    assert (list(m.free), list(m.ref), {k: list(v) for k, v in m.tables.items()}) == before
    assert m.copies == []
    m.append(1, 2)                        # a copy only
    assert m.take_copies() == [(1, 2)]
    with pytest.raises(AllocatorError):
        m.fork(0, 2, 7)                   # past the source's end
