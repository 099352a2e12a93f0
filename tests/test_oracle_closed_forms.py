"""Pins of closed forms, the allocator model and the workload recipe.

Closed forms and worked examples come from the pages (tests/golden/*, each
line cited there).  The allocator model is pinned to the block-manager
emulation's worked example and to the prefix-sharing accounting.
"""
import numpy as np
import pytest

import oracle
from conftest import read_golden_kv, read_golden_rows
from oracle.allocator_model import AllocatorError, BlockPoolModel, OutOfBlocks
from workloads import WORKLOADS, generate


def test_kv_size_examples():
    for name, args, expected, unit, _src in read_golden_rows("kv_size_examples.txt"):
        L, H, D, S, B, P = args.split()
        val = oracle.kv_bytes(int(L), int(H), int(D), int(S), int(B), float(P))
        if unit == "GiB":
            assert f"{val / 2**30:.2f}" == expected, name
        else:
            assert val == int(expected), name


def test_paged_footprint_and_waste_bound():
    for args, expected, _src in read_golden_rows("paged_footprint.txt"):
        n, p = (int(x) for x in args.split())
        blocks = oracle.paged_blocks(n, p)
        assert blocks == int(expected)
        assert 0 <= blocks * p - n <= p - 1


def test_snippet3_worked_example():
    g = read_golden_kv("allocator_examples.txt")
    m = BlockPoolModel(int(g["snippet3.num_blocks"]), int(g["snippet3.block_size"]))
    m.allocate(int(g["snippet3.seq"]), int(g["snippet3.tokens"]))
    assert m.tables[42] == [int(x) for x in g["snippet3.table"].split()]
    assert m.physical_address(42, int(g["snippet3.lookup_token"])) == (
        int(g["snippet3.physical_block"]), int(g["snippet3.offset"]))
    m.free_seq(42)
    assert list(m.free)[-3:] == [0, 1, 2] and len(m.free) == 1024


def test_prefix_sharing_accounting():
    g = read_golden_kv("allocator_examples.txt")
    prefix, uniq, reqs = (int(g["prefix.prefix_tokens"]), int(g["prefix.unique_tokens"]),
                          int(g["prefix.requests"]))
    p = int(g["prefix.block_size"])
    tokens_shared = prefix + reqs * uniq
    tokens_unshared = reqs * (prefix + uniq)
    assert tokens_shared == int(g["prefix.tokens_shared"])
    assert tokens_unshared == int(g["prefix.tokens_unshared"])
    assert f"{tokens_unshared / tokens_shared:.2f}" == g["prefix.ratio"]
    m = BlockPoolModel(1000, p)
    m.allocate(0, prefix + uniq)
    for r in range(1, reqs):
        m.fork(0, r, prefix)
        m.append(r, uniq)
    assert m.stats()[1] == int(g["prefix.blocks_shared"])
    m2 = BlockPoolModel(1000, p)
    for r in range(reqs):
        m2.allocate(r, prefix + uniq)
    assert m2.stats()[1] == int(g["prefix.blocks_unshared"])
    # shared blocks are referenced by every request; free returns them only at the last
    shared = m.tables[0][: prefix // p]
    assert all(m.ref[b] == reqs for b in shared)
    for r in range(reqs):
        m.free_seq(r)
    assert m.stats() == (1000, 0, 0.0)


def test_append_allocates_only_on_block_boundary():
    m = BlockPoolModel(8, 4)
    m.allocate(1, 0)
    slots = []
    for t in range(9):
        slots += m.append(1, 1)
        assert len(m.tables[1]) == -(-(t + 1) // 4)
    assert slots == [b * 4 + o for b in (0, 1, 2) for o in range(4)][:9]


def test_all_or_nothing_errors():
    m = BlockPoolModel(4, 16, free_order=[3, 1, 2, 0])
    m.allocate(0, 33)  # 3 blocks
    before = (list(m.free), dict(m.tables), dict(m.ntok), list(m.ref))
    with pytest.raises(OutOfBlocks):
        m.allocate(1, 17)
    with pytest.raises(OutOfBlocks):
        m.append(0, 40)
    assert (list(m.free), dict(m.tables), dict(m.ntok), list(m.ref)) == before
    with pytest.raises(AllocatorError):
        m.allocate(0, 1)
    with pytest.raises(AllocatorError):
        m.fork(0, 5, 48)  # longer than the source
    with pytest.raises(AllocatorError):
        m.free_seq(9)
    assert m.tables[0] == [3, 1, 2]


@pytest.mark.parametrize("name,total,lo,hi,blocks,used", [
    ("c1", 436, 17, 255, 64, 29),
    ("c2", 154680, 654, 4071, 11639, 9699),
    ("c4", 583567, 132, 8138, 21466, 17888),
])
def test_workload_recipe_check_values(name, total, lo, hi, blocks, used):
    """The generators reproduce the recipe's published check values."""
    import math
    import numpy as np

    wl = WORKLOADS[name]
    rng = np.random.default_rng(wl.seed)
    from workloads import _draw_lengths

    n = _draw_lengths(wl, rng)
    if wl.shared_prefix:
        k, pre = wl.shared_prefix
        n[:k] = np.maximum(n[:k], pre + 1)
    assert (int(n.sum()), int(n.min()), int(n.max())) == (total, lo, hi)
    need = sum(-(-int(x) // wl.p) for x in n)
    if wl.shared_prefix:
        need -= (wl.shared_prefix[0] - 1) * wl.shared_prefix[1] // wl.p
    assert need == used
    nb = wl.pool_blocks or -(-6 * need // 5)
    assert nb == blocks


def test_workload_allocation_uses_all_blocks_once():
    gen = generate(WORKLOADS["c1"])
    m = BlockPoolModel(gen.num_blocks, gen.wl.p, gen.free_order)
    m.run_ops(gen.ops)
    used = [b for s in m.tables.values() for b in s]
    assert len(used) == len(set(used)) == 29
    assert m.stats()[0] + 29 == 64
