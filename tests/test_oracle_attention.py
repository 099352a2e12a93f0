"""Pins of the oracle's paged attention, split-K statistics and merge.

The pages print no attention output for any example, so the oracle is tied
to the textbook formula (softmax(q K^T / sqrt(d)) V, "KV Cache
Optimization: 3x Faster LLM Inference on 24GB VRAM", section "Why Standard
Approaches Fail") by brute force on tiny inputs, to contiguous attention on
the same data (the paged kernel must equal attention over a contiguous
cache: "Reducing LLM Inference Latency...", section "PagedAttention: Solving
VRAM Fragmentation"), to invariance under any physical block placement, and
to closed-form special cases.
"""
import numpy as np
import pytest

import oracle
from oracle import brute
from workloads import Workload, generate, scaled
from common import dequant_rows, oracle_state, softmax_scale


def _tiny(kv="f16", D=8, Hq=4, Hkv=2, p=4, lengths=(1, 3, 5, 8), seed=0, io=None):
    io = io or ("f16" if kv == "f16" else "bf16")
    return Workload("tiny", seed, len(lengths), Hq, Hkv, D, p, kv, io, ("fixed", tuple(lengths)))


def _q(gen):
    return oracle.decode16(gen.q_bits, gen.in_dtype)


@pytest.mark.parametrize("Hq,Hkv", [(4, 2), (4, 1), (3, 3), (8, 2)])
def test_brute_force_tiny(orc, Hq, Hkv):
    wl = _tiny(Hq=Hq, Hkv=Hkv, D=8, p=4, lengths=(1, 3, 5, 8, 2))
    gen = generate(wl)
    d, pools, bt, cl, _ = oracle_state(gen)
    sc = softmax_scale(8)
    out = orc.paged_attention(d, gen.q_bits, pools, bt, cl, sc)
    q = _q(gen)
    G = Hq // Hkv
    for b in range(wl.B):
        for h in range(Hq):
            K = oracle.decode16(gen.k_bits[gen.rows(b), h // G], gen.in_dtype)
            V = oracle.decode16(gen.v_bits[gen.rows(b), h // G], gen.in_dtype)
            ref = brute.attention_loops(q[b, h], K, V, sc)
            assert np.allclose(out[b, h], ref, rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("kv", ["f16", "bf16", "fp8_e4m3", "int4_asym_g32", "fp8_e5m2"])
def test_contiguous_equality(orc, kv):
    """Paged oracle == textbook attention over the gathered contiguous cache
    (dequantised independently from the raw inputs)."""
    wl = Workload("contig", 3, 5, 8, 2, 64, 16, kv, "f16" if kv == "f16" else "bf16",
                  ("fixed", (1, 16, 17, 100, 255)), outliers=(0.01, 20.0))
    gen = generate(wl)
    d, pools, bt, cl, _ = oracle_state(gen)
    sc = softmax_scale(64)
    out = orc.paged_attention(d, gen.q_bits, pools, bt, cl, sc)
    q = _q(gen)
    for b in range(wl.B):
        for h in range(wl.Hq):
            K = dequant_rows(gen, "k", b, h // wl.G)
            V = dequant_rows(gen, "v", b, h // wl.G)
            s = K @ q[b, h] * sc
            e = np.exp(s - s.max())
            ref = e @ V / e.sum()
            assert np.allclose(out[b, h], ref, rtol=1e-12, atol=1e-13)


def test_gather_layout_definition(orc):
    """A token written at a known slot lands where the documented layout
    puts it: K row [blk][h][off][:], V column [blk][h][:][off]."""
    rng = np.random.default_rng(4)
    H, D, p, NB = 2, 8, 4, 6
    d = orc.desc("bf16", "bf16", H, D, p, NB)
    pools = orc.pool_arrays("bf16", NB, H, p, D)
    k = rng.integers(0, 65535, (2, H, D), dtype=np.uint16) & 0x7F7F
    v = rng.integers(0, 65535, (2, H, D), dtype=np.uint16) & 0x7F7F
    orc.reshape_and_cache(d, k, v, np.array([4 * 3 + 1, -1]), pools)
    for h in range(H):
        assert np.array_equal(pools["k_pool"][3, h, 1, :], k[0, h])
        assert np.array_equal(pools["v_pool"][3, h, :, 1], v[0, h])
    written = np.zeros_like(pools["k_pool"], dtype=bool)
    written[3, :, 1, :] = True
    assert np.all(pools["k_pool"][~written] == 0)


def test_permutation_invariance_bitwise(orc):
    """Outputs depend only on logical positions: two different physical
    placements of the same data give identical bits."""
    base = scaled("c2", 3, ("fixed", (40, 77, 130)), label="perm")
    outs = []
    for seed_order in (0, 1):
        gen = generate(base)
        if seed_order:
            gen.free_order = np.random.default_rng(99).permutation(gen.num_blocks).astype(np.int32)
        d, pools, bt, cl, _ = oracle_state(gen)
        outs.append(orc.paged_attention(d, gen.q_bits, pools, bt, cl, softmax_scale(128)))
    assert np.array_equal(outs[0].view(np.uint64), outs[1].view(np.uint64))


def test_single_token_returns_v(orc):
    gen = generate(_tiny(kv="bf16", lengths=(1, 1, 1), D=16))
    d, pools, bt, cl, _ = oracle_state(gen)
    out = orc.paged_attention(d, gen.q_bits, pools, bt, cl, softmax_scale(16))
    for b in range(3):
        for h in range(4):
            v0 = oracle.decode16(gen.v_bits[gen.rows(b)[0], h // 2], "bf16")
            assert np.array_equal(out[b, h], v0)


def test_constant_v_and_zero_q(orc):
    wl = _tiny(kv="bf16", lengths=(7, 33, 64), D=16, p=16)
    gen = generate(wl)
    # constant V per KV head
    for h in range(wl.Hkv):
        gen.v_bits[:, h, :] = gen.v_bits[0, h, :]
    d, pools, bt, cl, _ = oracle_state(gen)
    out = orc.paged_attention(d, gen.q_bits, pools, bt, cl, softmax_scale(16))
    for b in range(wl.B):
        for h in range(wl.Hq):
            v = oracle.decode16(gen.v_bits[0, h // 2], "bf16")
            assert np.allclose(out[b, h], v, rtol=1e-14, atol=0)
    # Q = 0: uniform weights, output is the mean of V
    gen2 = generate(wl)
    gen2.q_bits[...] = 0
    d, pools, bt, cl, _ = oracle_state(gen2)
    out = orc.paged_attention(d, gen2.q_bits, pools, bt, cl, softmax_scale(16))
    for b in range(wl.B):
        for h in range(wl.Hq):
            V = oracle.decode16(gen2.v_bits[gen2.rows(b), h // 2], "bf16")
            assert np.allclose(out[b, h], V.mean(axis=0), rtol=1e-13, atol=1e-15)


def test_empty_sequence_gives_zero(orc):
    gen = generate(_tiny(kv="bf16", lengths=(0, 3), D=16))
    d, pools, bt, cl, _ = oracle_state(gen)
    out = orc.paged_attention(d, gen.q_bits, pools, bt, cl, softmax_scale(16))
    assert np.all(out[0] == 0.0)


@pytest.mark.parametrize("partition", [16, 32, 512])
def test_split_k_merge_equals_unsplit(orc, partition):
    wl = Workload("split", 7, 4, 8, 2, 64, 16, "bf16", "bf16", ("fixed", (15, 16, 300, 1000)))
    gen = generate(wl)
    d, pools, bt, cl, _ = oracle_state(gen)
    sc = softmax_scale(64)
    out, pm, pl, pa = orc.paged_attention(d, gen.q_bits, pools, bt, cl, sc, partition=partition)
    q = _q(gen)
    for b in range(wl.B):
        n = int(cl[b])
        npart = -(-n // partition)
        for h in range(wl.Hq):
            merged = orc.lse_merge(pm[b, h, :npart], pl[b, h, :npart], pa[b, h, :npart])
            assert np.allclose(merged, out[b, h], rtol=1e-12, atol=1e-14)
            # per-partition statistics against their definition, by brute force
            K = oracle.decode16(gen.k_bits[gen.rows(b), h // 4], "bf16")
            V = oracle.decode16(gen.v_bits[gen.rows(b), h // 4], "bf16")
            s = K @ q[b, h] * sc
            for k in range(npart):
                sl = s[k * partition:(k + 1) * partition]
                assert pm[b, h, k] == sl.max()
                e = np.exp(sl - sl.max())
                assert np.isclose(pl[b, h, k], e.sum(), rtol=1e-13)
                assert np.allclose(pa[b, h, k], e @ V[k * partition:(k + 1) * partition],
                                   rtol=1e-12, atol=1e-13)
        if npart == 1:
            # a partition covering the whole context is the identity
            assert np.allclose(pa[b, :, 0] / pl[b, :, 0, None], out[b], rtol=1e-13, atol=1e-15)


def test_invalid_tables_rejected(orc):
    gen = generate(_tiny(kv="bf16", lengths=(5, 3), D=16))
    d, pools, bt, cl, _ = oracle_state(gen)
    bad = bt.copy()
    bad[0, 0] = gen.num_blocks
    with pytest.raises(ValueError):
        orc.paged_attention(d, gen.q_bits, pools, bad, cl, 0.25)
    big = cl.copy()
    big[1] = bt.shape[1] * 4 + 1
    with pytest.raises(ValueError):
        orc.paged_attention(d, gen.q_bits, pools, bt, big, 0.25)
