"""Host checks of the Python binding's argument validation (no GPU).

The binding checks shapes, dtypes and buffer sizes before any pointer
reaches the library: a tensor smaller than the descriptor says would
otherwise become an out-of-bounds device access.  The checks run before the
device-pointer conversion, so CPU tensors exercise them here: a bad argument
raises PkvError (INVALID_ARG); a good one gets as far as the pointer
conversion, which refuses a CPU tensor with ValueError."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pkv = pytest.importorskip("paged_kv_cache_250_amd")

B, HQ, HKV, D, P, NB = 3, 8, 2, 128, 16, 10


def _args(kv="bf16", io="bf16"):
    desc = pkv.cache_desc(kv, io, HKV, D, P, NB)
    pool_b, meta_b = pkv.pkv_cache_bytes(desc)
    tio = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[io]
    t = dict(
        out=torch.empty(B, HQ, D, dtype=tio), q=torch.empty(B, HQ, D, dtype=tio),
        k_pool=torch.empty(pool_b, dtype=torch.uint8), v_pool=torch.empty(pool_b, dtype=torch.uint8),
        k_meta=torch.empty(meta_b, dtype=torch.uint8) if meta_b else None,
        v_meta=torch.empty(meta_b, dtype=torch.uint8) if meta_b else None,
        block_tables=torch.zeros(B, 4, dtype=torch.int32), ctx_lens=torch.zeros(B, dtype=torch.int32))
    return desc, t


def _call(desc, t, **kw):
    return pkv.decode_args(desc, t["out"], t["q"], t["k_pool"], t["v_pool"], t["k_meta"],
                           t["v_meta"], t["block_tables"], t["ctx_lens"], 64, 0.1, **kw)


def test_good_arguments_reach_the_pointer_conversion():
    desc, t = _args()
    with pytest.raises(ValueError, match="GPU tensor"):
        _call(desc, t)


@pytest.mark.parametrize("field,bad", [
    ("q", torch.empty(B, HQ, D, dtype=torch.float16)),            # io is bf16
    ("q", torch.empty(B, HQ, 64, dtype=torch.bfloat16)),          # head_dim 128
    ("out", torch.empty(B, HQ, D, dtype=torch.float32)),          # without the fp32 flag
    ("out", torch.empty(B, HQ - 1, D, dtype=torch.bfloat16)),
    ("block_tables", torch.zeros(B, 4, dtype=torch.int64)),
    ("block_tables", torch.zeros(B + 1, 4, dtype=torch.int32)),
    ("ctx_lens", torch.zeros(B, dtype=torch.int64)),
    ("ctx_lens", torch.zeros(B - 1, dtype=torch.int32)),
    ("k_pool", torch.empty(100, dtype=torch.uint8)),
    ("v_pool", torch.empty(100, dtype=torch.uint8)),
])
def test_bad_decode_arguments_are_refused(field, bad):
    desc, t = _args()
    t[field] = bad
    with pytest.raises(pkv.PkvError) as e:
        _call(desc, t)
    assert e.value.name == "INVALID_ARG"


def test_fp32_output_flag_takes_an_fp32_out():
    desc, t = _args()
    t["out"] = torch.empty(B, HQ, D, dtype=torch.float32)
    with pytest.raises(ValueError, match="GPU tensor"):
        _call(desc, t, flags=pkv.PKV_DECODE_OUT_F32)
    t["out"] = torch.empty(B, HQ, D, dtype=torch.bfloat16)
    with pytest.raises(pkv.PkvError):
        _call(desc, t, flags=pkv.PKV_DECODE_OUT_F32)


@pytest.mark.parametrize("kv", ["fp8_e4m3", "int4_asym_g32"])
def test_quantised_caches_need_their_metadata(kv):
    desc, t = _args(kv)
    t["k_meta"] = None
    with pytest.raises(pkv.PkvError):
        _call(desc, t)
    desc, t = _args(kv)
    t["v_meta"] = t["v_meta"][:-4]
    with pytest.raises(pkv.PkvError):
        _call(desc, t)


def test_bad_blocks_counter_must_be_int32():
    desc, t = _args()
    with pytest.raises(pkv.PkvError):
        _call(desc, t, bad_blocks=torch.zeros(1, dtype=torch.int64))


def _rc(kv, k=None, v=None, slots=None, kp=None):
    desc = pkv.cache_desc(kv, "bf16", HKV, D, P, NB)
    pool_b, meta_b = pkv.pkv_cache_bytes(desc)
    N = 4
    k = torch.empty(N, HKV, D, dtype=torch.bfloat16) if k is None else k
    v = torch.empty(N, HKV, D, dtype=torch.bfloat16) if v is None else v
    slots = torch.tensor([0, 17, 40, 100], dtype=torch.int64) if slots is None else slots
    kp = torch.empty(pool_b, dtype=torch.uint8) if kp is None else kp
    vp = torch.empty(pool_b, dtype=torch.uint8)
    km = torch.empty(meta_b, dtype=torch.uint8) if meta_b else None
    vm = torch.empty(meta_b, dtype=torch.uint8) if meta_b else None
    pkv.pkv_reshape_and_cache(desc, k, v, slots, kp, vp, km, vm)


def test_reshape_and_cache_arguments():
    with pytest.raises(ValueError, match="GPU tensor"):
        _rc("bf16")
    for kw in (dict(k=torch.empty(4, HKV, D, dtype=torch.float16)),
               dict(v=torch.empty(4, HKV, 64, dtype=torch.bfloat16)),
               dict(k=torch.empty(5, HKV, D, dtype=torch.bfloat16)),
               dict(slots=torch.tensor([0, 1, 2, 3], dtype=torch.int32)),
               dict(kp=torch.empty(64, dtype=torch.uint8))):
        with pytest.raises(pkv.PkvError):
            _rc("bf16", **kw)


def test_block_scaled_fp8_refuses_two_tokens_of_one_block():
    """One call may write at most one token per block of a block-scaled FP8
    cache (the kernel requantises a block for its one new token): the
    binding checks the slots on the host before the call."""
    with pytest.raises(pkv.PkvError) as e:
        _rc("fp8_e4m3_block", slots=torch.tensor([0, 5, 40, 100], dtype=torch.int64))
    assert e.value.name == "INVALID_ARG"
    # one token per block passes the check (and stops at the CPU tensors)
    with pytest.raises(ValueError, match="GPU tensor"):
        _rc("fp8_e4m3_block", slots=torch.tensor([0, 17, 40, 100], dtype=torch.int64))
