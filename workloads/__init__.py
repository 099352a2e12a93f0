"""Seeded synthetic workloads for paged decode attention.

This module is shared by the CPU oracle side and the HIP side of every test
and of the bench.  It only draws random numbers and lays them out: it holds
none of the method's arithmetic (no allocation, no quantisation, no
attention).  Allocation is described as a list of operations that each side
executes with its own allocator.

Recipe (numpy ``default_rng(seed)``, PCG64), calls in exactly this order:

1. context lengths (when the workload draws them);
2. ``permutation(num_blocks)`` -- the initial order of the free-block list;
3. ``Q = standard_normal((B, Hq, D), float32)``;
4. ``K``, then ``V = standard_normal((T, Hkv, D), float32)`` where ``T`` counts
   distinct logical tokens stored sequence-major, position-minor; sequences
   that share a prefix skip their prefix positions (those alias sequence 0);
5. outlier workloads only: ``random(K.shape) < frac`` then the same for V;
   the selected elements are multiplied by ``factor``.

Every value is then rounded to the workload's 16-bit input type with
round-to-nearest-even (torch's CPU casts).  Pool size is
``ceil(6 * need / 5)`` blocks where ``need`` counts shared blocks once.

The workload shapes follow the Llama-3 attention shapes named on the pages
(Reducing LLM Inference Latency..., "Understanding the Bottleneck": 8 KV
heads, head_dim 128; KV Cache Optimization..., "Why Standard Approaches
Fail": 64 query heads in 8 GQA groups for the 70B model).
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Tuple

import numpy as np

KV_DTYPES = ("f16", "bf16", "fp8_e4m3", "int4_asym_g32", "fp8_e5m2", "fp8_e4m3_block")
IO_DTYPES = ("f16", "bf16", "f32")


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    B: int
    Hq: int
    Hkv: int
    D: int
    p: int
    kv_dtype: str
    io_dtype: str
    # one of: ("fixed", [n0, n1, ...]), ("uniform", lo, hi), ("loguniform", lo, hi),
    # ("const", n)
    lengths: tuple
    shared_prefix: Optional[Tuple[int, int]] = None  # (num_sharing_sequences, prefix_tokens)
    outliers: Optional[Tuple[float, float]] = None  # (fraction, factor)
    partition: int = 0  # 0 = library's choice, -1 = single pass, >0 = tokens per partition
    pool_blocks: Optional[int] = None  # fixed pool size (else 1.2x need)
    description: str = ""

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads.  c1 is small enough for the oracle to finish in
# milliseconds; c2 is the Llama-3-8B-shaped headline batch.
WORKLOADS = {
    "c1": Workload(
        "c1", 1, 4, 8, 2, 64, 16, "f16", "f16", ("fixed", (17, 64, 100, 255)),
        pool_blocks=64, partition=-1,
        description="tiny paged decode: B=4, 8/2 heads, D=64, p=16, fp16 KV, 64-block pool"),
    "c2": Workload(
        "c2", 2, 64, 32, 8, 128, 16, "bf16", "bf16", ("uniform", 512, 4096),
        description="Llama-3-8B-shaped layer: B=64, 32/8 heads, D=128, p=16, bf16 KV, "
                    "n ~ U[512,4096]"),
    "c3": Workload(
        "c3", 2, 64, 32, 8, 128, 16, "fp8_e4m3", "bf16", ("uniform", 512, 4096),
        outliers=(0.01, 20.0),
        description="Llama-3-8B shape, FP8 E4M3 KV with one fp32 scale per (token, KV head), "
                    "1% outliers x20"),
    "c4": Workload(
        "c4", 4, 256, 64, 8, 128, 32, "bf16", "bf16", ("loguniform", 128, 8192),
        shared_prefix=(16, 1024),
        description="Llama-3-70B attention shape: B=256, 64/8 heads, D=128, p=32, bf16 KV, "
                    "n ~ logU[128,8192], 16 sequences share a 1024-token prefix"),
    "c5": Workload(
        "c5", 5, 8, 32, 8, 128, 16, "int4_asym_g32", "bf16", ("const", 32768),
        partition=512,
        description="long-context split-K: B=8, n=32768, 32/8 heads, D=128, p=16, INT4 "
                    "asymmetric g32 KV, 512-token partitions"),
}


def get(name: str) -> Workload:
    return WORKLOADS[name]


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


@dataclasses.dataclass
class Generated:
    wl: Workload
    lengths: np.ndarray  # int64 [B], context length including the new token
    num_blocks: int
    free_order: np.ndarray  # int32 [num_blocks]
    ops: List[tuple]  # allocation operations, executed in order
    q_bits: np.ndarray  # uint16 [B, Hq, D] (bit patterns of the 16-bit inputs)
    k_bits: np.ndarray  # uint16 [T, Hkv, D]
    v_bits: np.ndarray  # uint16 [T, Hkv, D]
    row_start: np.ndarray  # int64 [B]: first K/V row of each sequence's own positions
    own_from: np.ndarray  # int64 [B]: first position stored in the sequence's own rows

    @property
    def in_dtype(self) -> str:
        """16-bit type the K/V/Q inputs were rounded to."""
        return "f16" if self.wl.io_dtype == "f16" else "bf16"

    def rows(self, b: int) -> np.ndarray:
        """K/V row index of positions 0..n_b-1 of sequence b."""
        n = int(self.lengths[b])
        pos = np.arange(n, dtype=np.int64)
        r = self.row_start[b] + (pos - self.own_from[b])
        if self.own_from[b] > 0:
            shared = pos < self.own_from[b]
            r[shared] = self.row_start[0] + pos[shared]
        return r

    def token_positions(self) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
        """(seq, pos, row) for every distinct stored token, in row order."""
        seqs, poss, rows = [], [], []
        for b in range(self.wl.B):
            n = int(self.lengths[b])
            pos = np.arange(int(self.own_from[b]), n, dtype=np.int64)
            seqs.append(np.full(pos.shape, b, dtype=np.int64))
            poss.append(pos)
            rows.append(self.row_start[b] + pos - self.own_from[b])
        return np.concatenate(seqs), np.concatenate(poss), np.concatenate(rows)

    @property
    def T(self) -> int:
        return int(self.k_bits.shape[0])


def bits_to_f32(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float32 values of 16-bit bit patterns (a plain reinterpretation)."""
    if dtype == "bf16":
        return (bits.astype(np.uint32) << 16).view(np.float32)
    if dtype == "f16":
        return bits.view(np.float16).astype(np.float32)
    raise ValueError(dtype)


def _round_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype == "bf16":
        return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    if dtype == "f16":
        return t.to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    raise ValueError(dtype)


def _draw_lengths(wl: Workload, rng) -> np.ndarray:
    kind = wl.lengths[0]
    if kind == "fixed":
        n = np.array(wl.lengths[1], dtype=np.int64)
        assert n.shape == (wl.B,)
        return n
    if kind == "const":
        return np.full(wl.B, int(wl.lengths[1]), dtype=np.int64)
    if kind == "uniform":
        lo, hi = wl.lengths[1], wl.lengths[2]
        return rng.integers(lo, hi, size=wl.B, endpoint=True).astype(np.int64)
    if kind == "loguniform":
        lo, hi = wl.lengths[1], wl.lengths[2]
        n = np.floor(np.exp(rng.uniform(math.log(lo), math.log(hi), size=wl.B)))
        return np.clip(n.astype(np.int64), lo, hi)
    raise ValueError(kind)


@dataclasses.dataclass
class Plan:
    """The allocation side of a workload: lengths, pool size, free order and
    the operations that build the block tables."""
    lengths: np.ndarray
    num_blocks: int
    free_order: np.ndarray
    ops: List[tuple]
    own_from: np.ndarray


def plan(wl: Workload, rng=None) -> Plan:
    """Draw steps 1-2 of the recipe (lengths, free order)."""
    rng = np.random.default_rng(wl.seed) if rng is None else rng
    n = _draw_lengths(wl, rng)
    p = wl.p
    own_from = np.zeros(wl.B, dtype=np.int64)
    ops: List[tuple] = []
    if wl.shared_prefix is not None:
        k, prefix = wl.shared_prefix
        assert prefix % p == 0 and k <= wl.B
        n[:k] = np.maximum(n[:k], prefix + 1)
        own_from[1:k] = prefix
        need = sum(_ceil_div(int(x), p) for x in n) - (k - 1) * (prefix // p)
        ops.append(("allocate", 0, int(n[0])))
        for b in range(1, k):
            ops.append(("fork", 0, b, prefix))
            ops.append(("append", b, int(n[b]) - prefix))
        for b in range(k, wl.B):
            ops.append(("allocate", b, int(n[b])))
    else:
        need = sum(_ceil_div(int(x), p) for x in n)
        for b in range(wl.B):
            ops.append(("allocate", b, int(n[b])))
    num_blocks = wl.pool_blocks if wl.pool_blocks is not None else _ceil_div(6 * need, 5)
    assert num_blocks >= need
    free_order = rng.permutation(num_blocks).astype(np.int32)
    return Plan(n, num_blocks, free_order, ops, own_from)


def generate(wl: Workload) -> Generated:
    rng = np.random.default_rng(wl.seed)
    pl = plan(wl, rng)
    n, num_blocks, free_order, ops, own_from = (pl.lengths, pl.num_blocks, pl.free_order, pl.ops,
                                                pl.own_from)
    q = rng.standard_normal((wl.B, wl.Hq, wl.D), dtype=np.float32)
    own = (n - own_from).astype(np.int64)
    row_start = np.zeros(wl.B, dtype=np.int64)
    row_start[1:] = np.cumsum(own)[:-1]
    T = int(own.sum())
    k = rng.standard_normal((T, wl.Hkv, wl.D), dtype=np.float32)
    v = rng.standard_normal((T, wl.Hkv, wl.D), dtype=np.float32)
    if wl.outliers is not None:
        frac, factor = wl.outliers
        mk = rng.random(k.shape) < frac
        k[mk] *= np.float32(factor)
        del mk
        mv = rng.random(v.shape) < frac
        v[mv] *= np.float32(factor)
        del mv
    in_dtype = "f16" if wl.io_dtype == "f16" else "bf16"
    q_bits = _round_bits(q, in_dtype)
    del q
    k_bits = _round_bits(k, in_dtype)
    del k
    v_bits = _round_bits(v, in_dtype)
    del v
    return Generated(wl, n, num_blocks, free_order, ops, q_bits, k_bits, v_bits,
                     row_start, own_from)


def scaled(base_name: str, B: int, lengths: tuple, label: Optional[str] = None,
           **kw) -> Workload:
    """A smaller workload with the same recipe, heads, dtypes and block size."""
    base = WORKLOADS[base_name]
    shared = base.shared_prefix
    if shared is not None:
        shared = kw.pop("shared_prefix", (min(shared[0], B), shared[1]))
    return base.replace(name=label or base_name + "-small", B=B, lengths=lengths,
                        shared_prefix=shared, **kw)
