"""Shared test helpers: build the oracle-side state of a generated workload."""
from __future__ import annotations

import math

import numpy as np

import oracle
from oracle.state import oracle_state, table_width  # noqa: F401
from workloads import Generated


def softmax_scale(D: int) -> float:
    return float(np.float32(1.0 / math.sqrt(D)))


def dequant_rows(gen: Generated, which: str, b: int, h: int) -> np.ndarray:
    """Exact values of the cached K or V of sequence b, KV head h, computed
    from the raw inputs with the oracle's codec functions (fp64 [n, D])."""
    bits = (gen.k_bits if which == "k" else gen.v_bits)[gen.rows(b), h]
    x = oracle.decode16(bits, gen.in_dtype)
    kv = gen.wl.kv_dtype
    if kv in ("f16", "bf16"):
        return x
    if kv in ("fp8_e4m3", "fp8_e5m2"):
        fmt = kv[4:]
        codes, scales = oracle.fp8_quantize_rows(x.astype(np.float32), fmt)
        return oracle.fp8_dequant(codes, scales, fmt).astype(np.float64)
    codes, s, z = oracle.int4_quantize_rows(x.astype(np.float32))
    return oracle.int4_dequant(codes, s, z).astype(np.float64)
