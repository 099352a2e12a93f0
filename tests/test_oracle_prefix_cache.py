"""Pins of the automatic prefix cache in the oracle's allocator model.

"KV Cache Optimization: 3x Faster LLM Inference on 24GB VRAM" (section
"Prefix Caching: The Hidden Multiplier") works an example: three RAG
requests with an 800-token common prefix and 20 tokens of their own need
860 tokens of cache instead of 2460, because requests 2 and 3 reuse the
first request's pages; pages are evicted in LRU order.  "KV Cache
Compression & Paged Attention Deep Dive" (section "Implementation Details:
PagedAttention Kernel and Page Table") looks a hashed prefix up before
allocating.  Beyond the worked example, what fixes the result is that a
reused block must hold exactly the K/V its new owner would have written:
K/V of a token depend on every token before it, so the tests give each
token K/V drawn from its whole prefix and check, through the oracle's
reshape_and_cache and gather, that every sequence reads back its own.
"""
import hashlib

import numpy as np
import pytest

import oracle
from oracle import brute
from oracle.allocator_model import BlockPoolModel, OutOfBlocks
from common import softmax_scale
from conftest import read_golden_kv
from test_oracle_cow import check_invariants


def test_rag_example_from_the_pages():
    g = read_golden_kv("allocator_examples.txt")
    p = int(g["prefix.block_size"])
    pre, uniq, reqs = (int(g["prefix.prefix_tokens"]), int(g["prefix.unique_tokens"]),
                       int(g["prefix.requests"]))
    m = BlockPoolModel(1000, p)
    prefix = list(range(1000, 1000 + pre))
    cached, used = [], []
    for r in range(reqs):
        toks = prefix + [5000 + 100 * r + i for i in range(uniq)]
        cached.append(m.allocate_cached(r, toks))
        used.append(m.stats()[1])
    assert cached == [0, pre, pre]                         # requests 2 and 3 reuse the prefix
    assert sum(pre + uniq - c for c in cached) == int(g["prefix.tokens_shared"])  # 860
    assert used[-1] == int(g["prefix.blocks_shared"])      # 56 blocks instead of 156
    check_invariants(m)
    # the first request's blocks after the prefix are its own; the prefix is shared
    t0, t1 = m.tables[0], m.tables[1]
    assert t0[: pre // p] == t1[: pre // p] and t0[pre // p] != t1[pre // p]
    assert m.cache_stats()[2:] == ((reqs - 1) * (pre // p), reqs * ((pre + uniq) // p))


def test_lru_eviction_example():
    """Pool of 7 blocks of 4 tokens.  A and B are cached prompts; after both
    are freed (B first), allocations use the free list first, then evict
    the least recently released cached block."""
    m = BlockPoolModel(7, 4)
    A = [1, 2, 3, 4, 5, 6, 7, 8]          # blocks 0, 1
    B = [9, 9, 9, 9]                      # block 2
    m.allocate_cached(0, A)
    m.allocate_cached(1, B)
    m.free_seq(1)                         # B released first
    m.free_seq(0)                         # then A's blocks (0, 1)
    assert list(m.free) == [3, 4, 5, 6] and list(m.lru) == [2, 0, 1]
    assert m.stats()[0] == 7
    m.allocate(2, 16)                     # the four free blocks
    assert m.tables[2] == [3, 4, 5, 6]
    m.allocate(3, 4)                      # evicts B's block (released first)
    assert m.tables[3] == [2]
    assert m._lookup(B) == [] and m._lookup(A) == [0, 1]
    m.free_seq(3)                         # no longer cached: back to the free list
    assert list(m.free) == [2] and list(m.lru) == [0, 1]
    # A is still cached: a prompt extending it reuses both blocks
    assert m.allocate_cached(4, A + [7]) == 8
    assert m.tables[4] == [0, 1, 2]
    check_invariants(m)


def test_same_block_tokens_after_different_prefixes_are_not_shared():
    m = BlockPoolModel(20, 4)
    x, y, z = [1, 1, 1, 1], [2, 2, 2, 2], [3, 3, 3, 3]
    assert m.allocate_cached(0, x + z) == 0
    assert m.allocate_cached(1, y + z) == 0              # z after y is another entry
    assert m.tables[0][1] != m.tables[1][1]
    assert m.allocate_cached(2, x + z + [4]) == 8
    assert m.allocate_cached(3, y + z) == 8
    assert m.tables[3] == m.tables[1]


def test_all_or_nothing():
    m = BlockPoolModel(4, 4)
    m.allocate_cached(0, list(range(8)))                # 2 blocks, both cached
    m.free_seq(0)                                       # both evictable
    m.allocate(1, 8)                                    # the 2 free blocks
    before = (list(m.free), list(m.lru), list(m.ref), dict(m.cache), m.cache_stats())
    with pytest.raises(OutOfBlocks):
        # reuses both cached blocks, then needs 1 more: none is left
        m.allocate_cached(2, list(range(8)) + [99])
    assert (list(m.free), list(m.lru), list(m.ref), dict(m.cache), m.cache_stats()) == before
    assert m.allocate_cached(2, list(range(8))) == 8     # fits: revives both
    check_invariants(m)


def _row(prefix, Hkv, D, dt):
    """K and V of the last token of `prefix`: a function of the whole prefix."""
    seed = int.from_bytes(hashlib.sha256(np.asarray(prefix, np.int64).tobytes()).digest()[:8],
                          "little")
    x = np.random.default_rng(seed).standard_normal((2, Hkv, D))
    enc = oracle.f16_encode if dt == "f16" else oracle.bf16_encode
    return enc(x[0]), enc(x[1])


@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3", "int4_asym_g32"])
def test_cached_prompts_read_back_their_own_kv(orc, kv):
    dt = "bf16"
    p, Hkv, D, Hq = 16, 2, 64, 4
    rng = np.random.default_rng(17)
    nb = 40
    m = BlockPoolModel(nb, p, rng.permutation(nb))
    d = oracle.desc(kv, dt, Hkv, D, p, nb)
    pools = oracle.pool_arrays(kv, nb, Hkv, p, D, fill=0x33)
    # prompts from a few shared stems, some stems equal in later blocks only
    stems = [list(rng.integers(0, 50, 48)) for _ in range(3)]
    stems.append(list(rng.integers(0, 50, 16)) + stems[0][16:48])
    live, hist, nxt, hits = [], {}, 0, 0
    for step in range(60):
        if live and (rng.random() < 0.4 or m.available() < 12):
            s = live.pop(int(rng.integers(0, len(live))))
            m.free_seq(s)
            del hist[s]
            continue
        stem = stems[int(rng.integers(0, len(stems)))]
        cut = int(rng.integers(1, len(stem) + 1))
        toks = stem[:cut] + list(rng.integers(50, 60, int(rng.integers(0, 20))))
        try:
            c = m.allocate_cached(nxt, toks)
        except OutOfBlocks:
            continue
        hits += c
        # only the tokens not found in the cache are computed and written
        rows = [_row(toks[:t + 1], Hkv, D, dt) for t in range(c, len(toks))]
        if rows:
            oracle.reshape_and_cache(d, np.stack([r[0] for r in rows]),
                                     np.stack([r[1] for r in rows]),
                                     np.array([m.slot(nxt, t) for t in range(c, len(toks))]),
                                     pools)
        live.append(nxt)
        hist[nxt] = toks
        nxt += 1
        check_invariants(m)
        for s in live:  # every live sequence reads back its own K/V
            n = len(hist[s])
            for h in range(Hkv):
                K, V = oracle.gather(d, pools, np.asarray(m.tables[s], np.int32), n, h)
                want = [_row(hist[s][:t + 1], Hkv, D, dt) for t in range(n)]
                kx = np.stack([w[0][h] for w in want])
                vx = np.stack([w[1][h] for w in want])
                from test_oracle_cow import _exact_rows
                assert np.array_equal(K, _exact_rows(kx, dt, kv)), (s, h)
                assert np.array_equal(V, _exact_rows(vx, dt, kv)), (s, h)
    assert hits >= 10 * p, "the replay should reuse cached blocks"
    assert m.cache_stats()[1] > 0 or len(m.lru) == 0
    # attention over the cached tables equals textbook softmax over each history
    seqs = sorted(hist)
    W = max(len(m.tables[s]) for s in seqs)
    bt, cl = m.block_tables(seqs, W)
    qb = oracle.bf16_encode(rng.standard_normal((len(seqs), Hq, D)))
    sc = softmax_scale(D)
    out = oracle.paged_attention(d, qb, pools, bt, cl, sc)
    q = oracle.decode16(qb, dt)
    from test_oracle_cow import _exact_rows
    for i, s in enumerate(seqs):
        want = [_row(hist[s][:t + 1], Hkv, D, dt) for t in range(len(hist[s]))]
        for h in range(Hq):
            K = _exact_rows(np.stack([w[0][h // 2] for w in want]), dt, kv)
            V = _exact_rows(np.stack([w[1][h // 2] for w in want]), dt, kv)
            assert np.allclose(out[i, h], brute.attention_row(q[i, h], K, V, sc), rtol=1e-12,
                               atol=1e-13)
