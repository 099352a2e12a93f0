"""CPU oracle for paged decode attention -- test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its binding) never imports it and shares no code with it.

Contents:

* ``pkv_oracle.c`` -- plain C, fp64 scalar loops with OpenMP: number formats
  written from their definitions, the FP8/INT4 codecs, reshape_and_cache into
  host pools, paged attention with per-partition statistics, and the
  log-sum-exp merge.  Built with gcc by :func:`build`.
* :mod:`oracle.allocator_model` -- the block-pool allocator in plain Python,
  with copy-on-write of shared, partly filled blocks; :func:`copy_blocks`
  applies its copies to host pools.
* :mod:`oracle.brute` -- textbook softmax attention in NumPy for tiny inputs.

Parity pins (tests/test_oracle_*.py) tie every function here to the pages'
worked examples, closed forms, library routines or brute force.  Functions
with no such pin would say "parity unpinned"; every function exported here
has at least one pin.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Dict, Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pkv_oracle.c")
_LIBPATH = os.path.join(_HERE, "_build", "liboracle.so")

KV_CODES = {"f16": 0, "bf16": 1, "fp8_e4m3": 2, "int4_asym_g32": 3, "fp8_e5m2": 5,
            "fp8_e4m3_block": 6}
FP8_FORMATS = {"e4m3": 2, "e5m2": 5}
IN_CODES = {"f16": 0, "bf16": 1, "f32": 4}

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain C11, OpenMP, no FMA contraction)."""
    os.makedirs(os.path.dirname(_LIBPATH), exist_ok=True)
    if force or not os.path.exists(_LIBPATH) or os.path.getmtime(_LIBPATH) < os.path.getmtime(_SRC):
        tmp = _LIBPATH + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
             "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIBPATH)
    return _LIBPATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIBPATH) or os.path.getmtime(_LIBPATH) < os.path.getmtime(_SRC):
            build(force=True)
        L = ctypes.CDLL(_LIBPATH)
        vp, i64, i32, dbl, flt = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_double,
                                  ctypes.c_float)
        L.orc_f16_to_f64.restype = dbl
        L.orc_f16_to_f64.argtypes = [ctypes.c_uint16]
        L.orc_bf16_to_f64.restype = dbl
        L.orc_bf16_to_f64.argtypes = [ctypes.c_uint16]
        L.orc_e4m3_to_f64.restype = dbl
        L.orc_e4m3_to_f64.argtypes = [ctypes.c_uint8]
        L.orc_f64_to_e4m3.restype = ctypes.c_uint8
        L.orc_f64_to_e4m3.argtypes = [dbl]
        L.orc_f64_to_f16_bits.restype = ctypes.c_uint16
        L.orc_f64_to_f16_bits.argtypes = [dbl]
        L.orc_f64_to_bf16_bits.restype = ctypes.c_uint16
        L.orc_f64_to_bf16_bits.argtypes = [dbl]
        L.orc_e5m2_to_f64.restype = dbl
        L.orc_e5m2_to_f64.argtypes = [ctypes.c_uint8]
        L.orc_f64_to_e5m2.restype = ctypes.c_uint8
        L.orc_f64_to_e5m2.argtypes = [dbl]
        for name in ("orc_e4m3_encode_array", "orc_e4m3_decode_array", "orc_f16_encode_array",
                     "orc_bf16_encode_array", "orc_f16_decode_array", "orc_bf16_decode_array",
                     "orc_e5m2_encode_array", "orc_e5m2_decode_array"):
            getattr(L, name).restype = None
            getattr(L, name).argtypes = [vp, i64, vp]
        L.orc_fp8_quantize_rows.restype = None
        L.orc_fp8_quantize_rows.argtypes = [vp, i64, i32, vp, vp]
        L.orc_fp8_quantize_rows_fmt.restype = None
        L.orc_fp8_quantize_rows_fmt.argtypes = [vp, i64, i32, i32, vp, vp]
        L.orc_fp8_dequant_array_fmt.restype = None
        L.orc_fp8_dequant_array_fmt.argtypes = [vp, vp, i64, i32, i32, vp]
        L.orc_fp8_dequant_array.restype = None
        L.orc_fp8_dequant_array.argtypes = [vp, vp, i64, i32, vp]
        L.orc_int4_quantize_rows.restype = None
        L.orc_int4_quantize_rows.argtypes = [vp, i64, i32, vp, vp, vp]
        L.orc_int4_dequant_array.restype = None
        L.orc_int4_dequant_array.argtypes = [vp, vp, vp, i64, i32, vp]
        L.orc_reshape_and_cache.restype = i32
        L.orc_reshape_and_cache.argtypes = [vp, vp, vp, i32, vp, vp, vp, vp, vp]
        L.orc_gather.restype = i32
        L.orc_gather.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, vp, vp]
        L.orc_paged_attention.restype = i32
        L.orc_paged_attention.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, flt, vp,
                                          vp, i32, i32, vp, vp, vp]
        L.orc_lse_merge.restype = None
        L.orc_lse_merge.argtypes = [i32, vp, vp, vp, i32, vp]
        L.orc_num_threads.restype = i32
        L.orc_num_threads.argtypes = []
        _lib = L
    return _lib


def _p(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data


class Desc(ctypes.Structure):
    _fields_ = [("kv_dtype", ctypes.c_int), ("in_dtype", ctypes.c_int), ("Hkv", ctypes.c_int),
                ("D", ctypes.c_int), ("p", ctypes.c_int), ("num_blocks", ctypes.c_int64)]


def desc(kv_dtype: str, in_dtype: str, Hkv: int, D: int, p: int, num_blocks: int) -> Desc:
    return Desc(KV_CODES[kv_dtype], IN_CODES[in_dtype], Hkv, D, p, num_blocks)


# ------------------------------------------------------------------ formats

def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(c.shape, np.float64)
    lib().orc_e4m3_decode_array(_p(c), c.size, _p(out))
    return out


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(a.shape, np.uint8)
    lib().orc_e4m3_encode_array(_p(a), a.size, _p(out))
    return out


def e5m2_decode(codes: np.ndarray) -> np.ndarray:
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(c.shape, np.float64)
    lib().orc_e5m2_decode_array(_p(c), c.size, _p(out))
    return out


def e5m2_encode(x: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(a.shape, np.uint8)
    lib().orc_e5m2_encode_array(_p(a), a.size, _p(out))
    return out


def f16_encode(x: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(a.shape, np.uint16)
    lib().orc_f16_encode_array(_p(a), a.size, _p(out))
    return out


def bf16_encode(x: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(a.shape, np.uint16)
    lib().orc_bf16_encode_array(_p(a), a.size, _p(out))
    return out


def f16_decode(bits: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(b.shape, np.float64)
    lib().orc_f16_decode_array(_p(b), b.size, _p(out))
    return out


def bf16_decode(bits: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(b.shape, np.float64)
    lib().orc_bf16_decode_array(_p(b), b.size, _p(out))
    return out


def decode16(bits: np.ndarray, dtype: str) -> np.ndarray:
    return f16_decode(bits) if dtype == "f16" else bf16_decode(bits)


# ------------------------------------------------------------------- codecs

def fp8_quantize_rows(x: np.ndarray, fmt: str = "e4m3") -> Tuple[np.ndarray, np.ndarray]:
    """Rows of D fp32 values -> (codes [rows, D] u8, scale [rows] fp32);
    fmt "e4m3" or "e5m2"."""
    a = np.ascontiguousarray(x, dtype=np.float32)
    D = a.shape[-1]
    rows = a.size // D
    codes = np.empty(a.shape, np.uint8)
    scales = np.empty(a.shape[:-1], np.float32)
    lib().orc_fp8_quantize_rows_fmt(_p(a), rows, D, FP8_FORMATS[fmt], _p(codes), _p(scales))
    return codes, scales


def fp8_dequant(codes: np.ndarray, scales: np.ndarray, fmt: str = "e4m3") -> np.ndarray:
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    s = np.ascontiguousarray(scales, dtype=np.float32)
    D = c.shape[-1]
    if fmt == "e4m3":
        out = np.empty(c.shape, np.float32)
        lib().orc_fp8_dequant_array(_p(c), _p(s), c.size // D, D, _p(out))
        return out
    out = np.empty(c.shape, np.float32)
    lib().orc_fp8_dequant_array_fmt(_p(c), _p(s), c.size // D, D, FP8_FORMATS[fmt], _p(out))
    return out


def int4_quantize_rows(x: np.ndarray):
    """Rows of D fp32 values -> (codes [rows, D] u8 in 0..15, s, z [rows, D/32] fp16 bits)."""
    a = np.ascontiguousarray(x, dtype=np.float32)
    D = a.shape[-1]
    rows = a.size // D
    codes = np.empty(a.shape, np.uint8)
    s = np.empty(a.shape[:-1] + (D // 32,), np.uint16)
    z = np.empty(a.shape[:-1] + (D // 32,), np.uint16)
    lib().orc_int4_quantize_rows(_p(a), rows, D, _p(codes), _p(s), _p(z))
    return codes, s, z


def int4_dequant(codes: np.ndarray, s: np.ndarray, z: np.ndarray) -> np.ndarray:
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    sb = np.ascontiguousarray(s, dtype=np.uint16)
    zb = np.ascontiguousarray(z, dtype=np.uint16)
    D = c.shape[-1]
    out = np.empty(c.shape, np.float32)
    lib().orc_int4_dequant_array(_p(c), _p(sb), _p(zb), c.size // D, D, _p(out))
    return out


# -------------------------------------------------------------------- pools

def pool_arrays(kv_dtype: str, num_blocks: int, Hkv: int, p: int, D: int,
                fill: Optional[int] = 0) -> Dict[str, Optional[np.ndarray]]:
    """Host pools in the documented byte layout.  ``fill`` is a byte value
    (canary) written everywhere, or None for uninitialised memory."""
    def mk(shape, dt):
        a = np.empty(shape, dt)
        if fill is not None:
            a.view(np.uint8)[...] = fill
        return a
    if kv_dtype in ("f16", "bf16"):
        return {"k_pool": mk((num_blocks, Hkv, p, D), np.uint16),
                "v_pool": mk((num_blocks, Hkv, D, p), np.uint16),
                "k_meta": None, "v_meta": None}
    if kv_dtype in ("fp8_e4m3", "fp8_e5m2", "fp8_e4m3_block"):
        return {"k_pool": mk((num_blocks, Hkv, p, D), np.uint8),
                "v_pool": mk((num_blocks, Hkv, D, p), np.uint8),
                "k_meta": mk((num_blocks, Hkv, p), np.float32),
                "v_meta": mk((num_blocks, Hkv, p), np.float32)}
    if kv_dtype == "int4_asym_g32":
        return {"k_pool": mk((num_blocks, Hkv, p, D // 2), np.uint8),
                "v_pool": mk((num_blocks, Hkv, D, p // 2), np.uint8),
                "k_meta": mk((num_blocks, Hkv, p, D // 32, 2), np.uint16),
                "v_meta": mk((num_blocks, Hkv, p, D // 32, 2), np.uint16)}
    raise ValueError(kv_dtype)


def reshape_and_cache(d: Desc, k: np.ndarray, v: np.ndarray, slots: np.ndarray,
                      pools: Dict[str, Optional[np.ndarray]]) -> None:
    """Write new tokens' K/V ([N, Hkv, D], 16-bit bit patterns or fp32) to
    their slots in ``pools`` (host arrays, modified in place)."""
    k = np.ascontiguousarray(k)
    v = np.ascontiguousarray(v)
    s = np.ascontiguousarray(slots, dtype=np.int64)
    rc = lib().orc_reshape_and_cache(ctypes.byref(d), _p(k), _p(v), int(s.shape[0]), _p(s),
                                     _p(pools["k_pool"]), _p(pools["v_pool"]),
                                     _p(pools["k_meta"]), _p(pools["v_meta"]))
    if rc != 0:
        raise ValueError("slot outside the pool")


def copy_blocks(pools: Dict[str, Optional[np.ndarray]], pairs) -> None:
    """Copy-on-write copies: for each (source, destination) physical block,
    every KV head's K and V of the source block, with its scales or zero
    points, replaces the destination's ("KV Cache Compression & Paged
    Attention Deep Dive", copy-on-write of shared blocks).  The pairs of one
    call never overlap, so their order does not matter."""
    for src, dst in pairs:
        for a in pools.values():
            if a is not None:
                a[int(dst)] = a[int(src)]


def swap_blocks(device_pools: Dict[str, Optional[np.ndarray]],
                host_pools: Dict[str, Optional[np.ndarray]], pairs, to_host: bool) -> None:
    """Move whole blocks between the device pools and host pools of the same
    layout: for each (device block, host block) pair, every KV head's K and
    V with its scales or zero points ("Reducing LLM Inference Latency...",
    section "Prefill Swapping and GPU Thrashing": KV pages move between GPU
    and host memory)."""
    for b, h in pairs:
        for name, a in device_pools.items():
            if a is None:
                continue
            if to_host:
                host_pools[name][int(h)] = a[int(b)]
            else:
                a[int(b)] = host_pools[name][int(h)]


def gather(d: Desc, pools, table_row: np.ndarray, n: int, h: int) -> Tuple[np.ndarray, np.ndarray]:
    """Dequantised [n, D] K and V of one sequence and KV head (fp64)."""
    t = np.ascontiguousarray(table_row, dtype=np.int32)
    K = np.empty((max(n, 1), d.D), np.float64)
    V = np.empty((max(n, 1), d.D), np.float64)
    rc = lib().orc_gather(ctypes.byref(d), _p(pools["k_pool"]), _p(pools["v_pool"]),
                          _p(pools["k_meta"]), _p(pools["v_meta"]), _p(t), n, h, _p(K), _p(V))
    if rc != 0:
        raise ValueError("invalid block table entry")
    return K[:n], V[:n]


def paged_attention(d: Desc, q: np.ndarray, pools, block_tables: np.ndarray,
                    ctx_lens: np.ndarray, scale: float, seq_mask: Optional[np.ndarray] = None,
                    partition: int = 0):
    """fp64 paged decode attention.  Returns out [B, Hq, D] (and, when
    partition > 0, the per-partition (m, l, acc) arrays)."""
    q = np.ascontiguousarray(q)
    B, Hq, D = q.shape
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    cl = np.ascontiguousarray(ctx_lens, dtype=np.int32)
    W = bt.shape[1]
    out = np.zeros((B, Hq, D), np.float64)
    mask = None if seq_mask is None else np.ascontiguousarray(seq_mask, dtype=np.uint8)
    pm = pl = pa = None
    P_max = 0
    if partition > 0:
        P_max = max(1, -(-int(cl.max(initial=0)) // partition))
        pm = np.full((B, Hq, P_max), np.nan)
        pl = np.full((B, Hq, P_max), np.nan)
        pa = np.full((B, Hq, P_max, D), np.nan)
    rc = lib().orc_paged_attention(ctypes.byref(d), _p(q), _p(pools["k_pool"]),
                                   _p(pools["v_pool"]), _p(pools["k_meta"]), _p(pools["v_meta"]),
                                   _p(bt), _p(cl), B, Hq, W, float(np.float32(scale)), _p(mask),
                                   _p(out), int(partition), P_max, _p(pm), _p(pl), _p(pa))
    if rc != 0:
        raise ValueError("invalid context length or block table entry")
    if partition > 0:
        return out, pm, pl, pa
    return out


def lse_merge(m: np.ndarray, l: np.ndarray, acc: np.ndarray) -> np.ndarray:
    """Merge per-partition statistics of one (sequence, head): m, l [P], acc [P, D]."""
    m = np.ascontiguousarray(m, dtype=np.float64)
    l = np.ascontiguousarray(l, dtype=np.float64)
    acc = np.ascontiguousarray(acc, dtype=np.float64)
    out = np.empty(acc.shape[-1], np.float64)
    lib().orc_lse_merge(int(m.shape[0]), _p(m), _p(l), _p(acc), int(acc.shape[-1]), _p(out))
    return out


def num_threads() -> int:
    return int(lib().orc_num_threads())


# ------------------------------------------------------------ closed forms

def kv_bytes(layers: int, kv_heads: int, head_dim: int, seq_len: int, batch: int,
             bytes_per_elem: float) -> float:
    """KV-cache bytes: one K and one V element per (layer, KV head, channel,
    token, sequence) ("Reducing LLM Inference Latency...", section
    "Understanding the Bottleneck"; "Optimizing KV-Cache Memory Footprint...",
    section 2)."""
    return 2 * layers * kv_heads * head_dim * seq_len * batch * bytes_per_elem


def paged_blocks(n: int, p: int) -> int:
    """Blocks a sequence of n tokens occupies: ceil(n / p) ("KV Cache
    Optimization...", section "PagedAttention: The Real Solution")."""
    return -(-n // p)
