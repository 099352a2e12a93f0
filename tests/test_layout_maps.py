"""The tests' map from the library's physical chunk layouts back to the
oracle's logical layout must itself be a bijection: every logical element
(or INT4 nibble) lands on a distinct physical one covering the whole chunk."""
import numpy as np
import pytest

import oracle
from gpu_common_maps import chunk_index_maps, logical_pools


@pytest.mark.parametrize("kv", ["f16", "bf16", "fp8_e4m3", "int4_asym_g32", "fp8_e5m2"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("p", [16, 32])
def test_chunk_maps_are_bijections(kv, D, p):
    mp = chunk_index_maps(kv, p, D)
    if kv == "int4_asym_g32":
        for key in ("k", "v"):                  # bit offsets of whole nibbles
            assert np.all(mp[key] % 4 == 0)
            assert np.array_equal(np.sort(mp[key].ravel() // 4), np.arange(p * D))
        assert np.array_equal(np.sort(mp["m"].ravel()), np.arange(p * D // 32))
    else:
        assert np.array_equal(np.sort(mp["k"].ravel()), np.arange(p * D))
        assert np.array_equal(np.sort(mp["v"].ravel()), np.arange(p * D))


@pytest.mark.parametrize("kv", ["f16", "bf16", "fp8_e4m3", "int4_asym_g32", "fp8_e5m2"])
@pytest.mark.parametrize("D,p", [(64, 32), (128, 16)])
def test_logical_pools_inverts_the_physical_layout(kv, D, p):
    """Scatter random logical pools into the physical layout with the maps,
    then map back: the oracle-shaped arrays come back unchanged."""
    rng = np.random.default_rng(5)
    nb, H = 3, 2
    ref = oracle.pool_arrays(kv, nb, H, p, D, fill=None)
    for a in ref.values():
        if a is not None:
            a.view(np.uint8)[...] = rng.integers(0, 256, a.nbytes, dtype=np.uint8).reshape(
                a.view(np.uint8).shape)
    mp = chunk_index_maps(kv, p, D)
    raw = {}
    if kv == "int4_asym_g32":
        kcodes = np.stack([ref["k_pool"] & 0xF, ref["k_pool"] >> 4], -1).reshape(nb, H, p, D)
        vcodes = np.stack([ref["v_pool"] & 0xF, ref["v_pool"] >> 4], -1).reshape(nb, H, D, p)
        for name, codes, bit in (("k_pool", kcodes, mp["k"]), ("v_pool", vcodes, mp["v"])):
            phys = np.zeros((nb, H, p * D // 2), np.uint8)
            for bb in range(nb):
                for h in range(H):
                    np.bitwise_or.at(phys[bb, h], (bit // 8).ravel(),
                                     (codes[bb, h] << (bit % 8)).astype(np.uint8).ravel())
            raw[name] = phys
        for name in ("k_meta", "v_meta"):
            words = ref[name].view(np.uint32).reshape(nb, H, p, D // 32)
            phys = np.zeros((nb, H, p * D // 32), np.uint32)
            phys[:, :, mp["m"]] = words
            raw[name] = phys
    else:
        dt = np.uint16 if kv in ("f16", "bf16") else np.uint8
        for name, key in (("k_pool", "k"), ("v_pool", "v")):
            phys = np.zeros((nb, H, p * D), dt)
            phys[:, :, mp[key]] = ref[name].reshape(nb, H, *mp[key].shape)
            raw[name] = phys
        raw["k_meta"], raw["v_meta"] = ref["k_meta"], ref["v_meta"]
    got = logical_pools(kv, p, D, nb, H, raw)
    for name in ("k_pool", "v_pool", "k_meta", "v_meta"):
        if ref[name] is None:
            assert got[name] is None
        else:
            assert np.array_equal(got[name].view(np.uint8), ref[name].view(np.uint8)), name
