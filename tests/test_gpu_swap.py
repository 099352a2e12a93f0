"""GPU parity of swapping: sequences swapped out to a pinned host pool
(pkv_seq_swap_out + pkv_swap_blocks) while their device blocks are reused
and overwritten, then swapped back in, against the same traffic through the
oracle's allocator model and block move.  Device pools and the host pool
bitwise, decode within the tolerance of the oracle.  A staging buffer of
three blocks makes every move run in several rounds.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - collected on CPU hosts too
    pytest.skip("no GPU", allow_module_level=True)

import oracle  # noqa: E402
import paged_kv_cache_250_amd as pkv  # noqa: E402
from oracle.allocator_model import BlockPoolModel, OutOfBlocks  # noqa: E402
from gpu_common import (TORCH_IO, check_f32, check_stored, logical_pools, note,  # noqa: E402
                        pool_shapes, softmax_scale)

KVS = ["f16", "bf16", "fp8_e4m3", "int4_asym_g32", "fp8_e5m2"]
NAMES = ("k_pool", "v_pool", "k_meta", "v_meta")


def _host_arrays(host, kv, nh, Hkv, p, D):
    """Split a host pool [nh][K | V | K meta | V meta] into the four arrays."""
    sizes = [x // nh for x in pool_shapes(kv, nh, Hkv, p, D)]
    raw = host.numpy().reshape(nh, sum(sizes))
    out, o = {}, 0
    for n, sz in zip(NAMES, sizes):
        out[n] = np.ascontiguousarray(raw[:, o:o + sz]).reshape(-1) if sz else None
        o += sz
    return logical_pools(kv, p, D, nh, Hkv, out)


@pytest.mark.parametrize("kv", KVS)
@pytest.mark.parametrize("p", [16, 32])
def test_swap_out_reuse_swap_in_decode(kv, p):
    note(f"swap kv={kv} p={p}")
    io = "f16" if kv == "f16" else "bf16"
    Hkv, Hq, D, nb, nh = 2, 8, 128, 48, 40
    rng = np.random.default_rng(90 + p + KVS.index(kv))
    order = rng.permutation(nb).astype(np.int32)
    lp, m = pkv.BlockPool(nb, p, order), BlockPoolModel(nb, p, order)
    lp.set_host_blocks(nh)
    m.set_host_blocks(nh)
    d = pkv.cache_desc(kv, io, Hkv, D, p, nb)
    d_orc = oracle.desc(kv, io, Hkv, D, p, nb)
    dev_o = oracle.pool_arrays(kv, nb, Hkv, p, D, fill=0x44)
    host_o = oracle.pool_arrays(kv, nh, Hkv, p, D, fill=0x55)
    dev = [torch.full((n,), 0x44, dtype=torch.uint8, device="cuda") if n else None
           for n in pool_shapes(kv, nb, Hkv, p, D)]
    bb = pkv.pkv_swap_block_bytes(d)
    assert bb == sum(pool_shapes(kv, 1, Hkv, p, D))
    host = torch.full((nh * bb,), 0x55, dtype=torch.uint8).pin_memory()
    staging = torch.empty(3 * bb, dtype=torch.uint8, device="cuda")
    enc = oracle.f16_encode if io == "f16" else oracle.bf16_encode
    td = lambda b: torch.from_numpy(b.view(np.int16)).cuda().view(TORCH_IO[io])  # noqa: E731

    def write(slots):
        if not slots:
            return
        x = rng.standard_normal((2, len(slots), Hkv, D))
        kb, vb = enc(x[0]), enc(x[1])
        sl = np.asarray(slots, np.int64)
        oracle.reshape_and_cache(d_orc, kb, vb, sl, dev_o)
        pkv.pkv_reshape_and_cache(d, td(kb), td(vb), torch.from_numpy(sl).cuda(), *dev)

    live, out, nxt, moved = [], [], 0, 0
    for step in range(80):
        op = int(rng.integers(0, 5))
        try:
            if op <= 1:
                n = int(rng.integers(1, 4 * p))
                m.allocate(nxt, n)
                lp.allocate(nxt, n)
                write([m.slot(nxt, t) for t in range(n)])
                live.append(nxt)
                nxt += 1
            elif op == 2 and live:
                s = live[int(rng.integers(0, len(live)))]
                want = m.swap_out(s)
                got = lp.swap_out(s)
                assert np.array_equal(got, np.array(want, np.int32).reshape(-1, 2))
                oracle.swap_blocks(dev_o, host_o, want, to_host=True)
                pkv.pkv_swap_blocks(d, got, True, *dev, host, nh, staging)
                live.remove(s)
                out.append(s)
                moved += len(want)
            elif op == 3 and out:
                s = out[int(rng.integers(0, len(out)))]
                want = m.swap_in(s)
                got = lp.swap_in(s)
                assert np.array_equal(got, np.array(want, np.int32).reshape(-1, 2))
                oracle.swap_blocks(dev_o, host_o, want, to_host=False)
                pkv.pkv_swap_blocks(d, got, False, *dev, host, nh, staging)
                out.remove(s)
                live.append(s)
                moved += len(want)
            elif op == 4 and len(live) + len(out) > 2:
                s = (live + out)[int(rng.integers(0, len(live) + len(out)))]
                m.free_seq(s)
                lp.free(s)
                (live if s in live else out).remove(s)
            if live:  # one decode step: every live sequence appends a token
                s = live[int(rng.integers(0, len(live)))]
                want = m.append(s, 1)
                assert list(lp.append(s, 1)) == want
                write(want)
        except OutOfBlocks:
            pass
        assert lp.swap_stats() == m.swap_stats()
    assert moved >= 20
    torch.cuda.synchronize()
    got = logical_pools(kv, p, D, nb, Hkv,
                        {n: (None if t is None else t.cpu().numpy()) for n, t in zip(NAMES, dev)})
    for n, a in dev_o.items():
        if a is not None:
            assert np.array_equal(got[n].view(np.uint8), a.view(np.uint8)), n
    goth = _host_arrays(host, kv, nh, Hkv, p, D)
    for n, a in host_o.items():
        if a is not None:
            assert np.array_equal(goth[n].view(np.uint8), a.view(np.uint8)), "host " + n
    seqs = sorted(live)
    W = max(len(m.tables[s]) for s in seqs)
    bt, cl = m.block_tables(seqs, W)
    qb = enc(rng.standard_normal((len(seqs), Hq, D)))
    sc = softmax_scale(D)
    ref = oracle.paged_attention(d_orc, qb, dev_o, bt, cl, sc)
    for o_io in (io, "f32"):
        q = td(qb)
        q = q.float().contiguous() if o_io == "f32" else q
        o = torch.empty((len(seqs), Hq, D), dtype=TORCH_IO[o_io], device="cuda")
        dd = pkv.cache_desc(kv, o_io, Hkv, D, p, nb)
        mx = int(cl.max())
        wsb = pkv.pkv_decode_workspace_bytes(dd, len(seqs), Hq, mx, 0)
        ws = torch.empty((wsb // 4 + 4,), dtype=torch.float32, device="cuda") if wsb else None
        args = pkv.decode_args(dd, o, q, *dev, torch.from_numpy(bt).cuda(),
                               torch.from_numpy(cl).cuda(), mx, sc, 0, ws)
        pkv.pkv_paged_decode(dd, args)
        torch.cuda.synchronize()
        (check_f32 if o_io == "f32" else check_stored)(o, ref, kv, *(() if o_io == "f32"
                                                                     else (o_io,)))
    lp.close()


def test_swap_blocks_rejects_bad_pairs():
    d = pkv.cache_desc("bf16", "bf16", 2, 128, 16, 8)
    dev = [torch.zeros(n, dtype=torch.uint8, device="cuda") if n else None
           for n in pool_shapes("bf16", 8, 2, 16, 128)]
    bb = pkv.pkv_swap_block_bytes(d)
    host = torch.zeros(4 * bb, dtype=torch.uint8).pin_memory()
    staging = torch.empty(bb, dtype=torch.uint8, device="cuda")
    for pairs in ([[8, 0]], [[0, 4]], [[-1, 0]], [[1, 0], [1, 2]], [[1, 0], [2, 0]]):
        with pytest.raises(pkv.PkvError) as e:
            pkv.pkv_swap_blocks(d, np.array(pairs, np.int32), True, *dev, host, 4, staging)
        assert e.value.name == "INVALID_ARG"
    with pytest.raises(pkv.PkvError):
        pkv.pkv_swap_blocks(d, np.array([[0, 0]], np.int32), True, *dev, host, 4, staging[:16])
