"""Pins of the oracle's number formats and codecs.

The oracle writes fp16/bf16/e4m3 rounding from the format definitions; these
tests tie it to library routines (NumPy's fp16 casts, torch's bf16 and
float8_e4m3fn casts -- all round-to-nearest-even), to exhaustive tables and
to the values printed on "Reducing LLM Inference Latency: KV Cache
Quantization and PagedAttention in vLLM" (section "Block-Wise Scaling
Factors": E4M3 largest value 448, eps 1e-12).
"""
import numpy as np
import pytest
import torch

from conftest import read_golden_kv


def _f32_randoms(rng, n):
    """fp32 values spread over many binades, plus both signs."""
    mant = rng.uniform(1.0, 2.0, n)
    exp = rng.integers(-30, 20, n)
    sign = rng.choice([-1.0, 1.0], n)
    return (sign * np.ldexp(mant, exp)).astype(np.float32)


def test_f16_decode_exhaustive(orc):
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = orc.f16_decode(bits)
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(got[np.isinf(ref)], ref[np.isinf(ref)])


def test_bf16_decode_exhaustive(orc):
    bits = np.arange(65536, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy().astype(np.float64)
    got = orc.bf16_decode(bits)
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.isnan(got), np.isnan(ref))


def test_f16_encode_matches_numpy_rne(orc):
    rng = np.random.default_rng(11)
    x = _f32_randoms(rng, 200000)
    # halfway cases between adjacent fp16 values, subnormal range, overflow edge
    h = np.arange(0, 0x7C00, 7, dtype=np.uint16).view(np.float16).astype(np.float64)
    mids = ((h[:-1] + h[1:]) / 2).astype(np.float32)
    edges = np.array([0.0, -0.0, 65504.0, 65519.0, 65520.0, 70000.0, 2.0**-24, 2.0**-25,
                      3 * 2.0**-26, 2.0**-14, 5.96e-8, -65520.0], dtype=np.float32)
    for arr in (x, mids, edges):
        ref = arr.astype(np.float16).view(np.uint16)
        got = orc.f16_encode(arr.astype(np.float64))
        assert np.array_equal(got, ref)


def test_bf16_encode_matches_torch_rne(orc):
    rng = np.random.default_rng(12)
    x = _f32_randoms(rng, 200000)
    b = np.arange(0, 0x7F80, 5, dtype=np.uint16)
    vals = torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).double().numpy()
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    edges = np.array([0.0, -0.0, 1e-40, -3e-39, 3.3e38, 3.4e38, 1.0 + 2**-8, 1.0 + 3 * 2**-8],
                     dtype=np.float32)
    for arr in (x, mids, edges):
        ref = torch.from_numpy(arr).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        got = orc.bf16_encode(arr.astype(np.float64))
        assert np.array_equal(got, ref)


def test_e4m3_decode_exhaustive_matches_torch_and_page(orc):
    g = read_golden_kv("fp8_e4m3.txt")
    codes = np.arange(256, dtype=np.uint8)
    got = orc.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert int(np.isfinite(got).sum()) == int(g["finite_codes"])
    assert np.nanmax(got) == float(g["max_finite"]) == 448.0
    pos = got[np.isfinite(got) & (got > 0)]
    assert pos.min() == float(g["min_subnormal"])
    assert pos[pos >= float(g["min_normal"])].min() == float(g["min_normal"])
    assert int(g["exponent_bits"]) + int(g["mantissa_bits"]) + 1 == 8


def test_e4m3_encode_matches_torch_on_reachable_range(orc):
    """RNE with sign of zero kept; agrees with torch's cast for |x| <= 464."""
    rng = np.random.default_rng(13)
    x = rng.uniform(-464, 464, 100000).astype(np.float32)
    small = (rng.standard_normal(50000) * 0.01).astype(np.float32)  # subnormal region
    vals = np.sort(orc.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8)))
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)  # every tie in [0, 448]
    edges = np.array([0.0, -0.0, 448.0, 463.99, 464.0, -464.0, 2.0**-10, 3 * 2.0**-11],
                     dtype=np.float32)
    for arr in (x, small, mids, -mids, edges):
        ref = torch.from_numpy(arr).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        got = orc.e4m3_encode(arr.astype(np.float64))
        assert np.array_equal(got, ref), arr[got != ref][:5]


def test_e4m3_roundtrip_and_saturation(orc):
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    assert np.array_equal(orc.e4m3_encode(orc.e4m3_decode(codes)), codes)
    # reading: past the largest finite value the encoder saturates at +-448
    sat = orc.e4m3_encode(np.array([465.0, 1e6, -500.0]))
    assert list(sat) == [0x7E, 0x7E, 0xFE]


def test_fp8_row_quantizer(orc):
    """Absmax scale per row: scale = fp32(max|x| / 448), clamped at 1e-12;
    codes are the e4m3 rounding of fp32(x / scale)."""
    g = read_golden_kv("fp8_e4m3.txt")
    rng = np.random.default_rng(14)
    x = rng.standard_normal((500, 128)).astype(np.float32)
    x[::7] *= np.float32(20.0)
    x[3] = 0.0
    x[4] = np.float32(1e-14)
    codes, scales = orc.fp8_quantize_rows(x)
    a = np.abs(x).max(axis=1)
    ref_scale = np.maximum(a / np.float32(448.0), np.float32(g["eps"])).astype(np.float32)
    assert np.array_equal(scales.view(np.uint32), ref_scale.view(np.uint32))
    y = (x / ref_scale[:, None]).astype(np.float32)
    ref_codes = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, ref_codes)
    dec = orc.e4m3_decode(codes)
    big = a >= 448.0 * 1e-12
    assert np.all(np.abs(dec[big]).max(axis=1) == 448.0)
    assert np.all(codes[3] == 0) and scales[3] == np.float32(1e-12)
    # dequant: one fp32 product
    deq = orc.fp8_dequant(codes, scales)
    ref = (dec.astype(np.float32) * scales[:, None]).astype(np.float32)
    assert np.array_equal(deq, ref)
    # relative error of e4m3 with 3 mantissa bits: at most 2^-4 of |x| for normal codes
    err = np.abs(deq - x)
    assert np.all(err <= np.maximum(np.abs(x) * 2.0**-4, scales[:, None] * 2.0**-10) * 1.0001)


def test_int4_group_quantizer_invariants(orc):
    """Asymmetric min/max groups of 32: codes in 0..15, the group minimum maps
    to 0 and the maximum to 15, dequant error at most S/2 plus the fp16
    rounding of s and z, constant groups dequantise to z exactly."""
    rng = np.random.default_rng(15)
    x = rng.standard_normal((400, 128)).astype(np.float32)
    x[5, :32] = np.float32(0.75)  # constant group
    codes, s, z = orc.int4_quantize_rows(x)
    assert codes.max() <= 15
    S = s.view(np.float16).astype(np.float32)
    Z = z.view(np.float16).astype(np.float32)
    xg = x.reshape(400, 4, 32)
    cg = codes.reshape(400, 4, 32)
    mn, mx = xg.min(axis=2), xg.max(axis=2)
    # s and z: fp16 RNE of fp32 (max - min) / 15 and of min (NumPy casts)
    ref_s = ((mx - mn).astype(np.float32) / np.float32(15.0)).astype(np.float32).astype(np.float16)
    assert np.array_equal(s, ref_s.view(np.uint16))
    assert np.array_equal(z, mn.astype(np.float16).view(np.uint16))
    nz = S > 0
    idx_min = xg.argmin(axis=2)
    idx_max = xg.argmax(axis=2)
    r = np.arange(400)[:, None]
    gi = np.arange(4)[None, :]
    assert np.all(cg[r, gi, idx_min][nz] == 0)
    assert np.all(cg[r, gi, idx_max][nz] == 15)
    deq = orc.int4_dequant(codes, s, z).reshape(400, 4, 32)
    # fma(code, s, z) with one rounding: the fp64 sum is exact for these
    # operands (4-bit code times 11-bit s plus 11-bit z), then one fp32 rounding
    ref_deq = (cg.astype(np.float64) * S[..., None].astype(np.float64)
               + Z[..., None].astype(np.float64)).astype(np.float32)
    assert np.array_equal(deq.view(np.uint32), ref_deq.view(np.uint32))
    bound = S[..., None] / 2 + 2.0**-9 * np.maximum(np.abs(mn), np.abs(mx))[..., None]
    assert np.all(np.abs(deq - xg) <= bound + 1e-7)
    assert not nz[5, 0] and np.all(cg[5, 0] == 0) and np.all(deq[5, 0] == np.float32(0.75))


def test_int4_codes_are_nearest(orc):
    """Brute force over all 16 codes: the chosen code's dequantised value is
    the nearest one (up to fp32 rounding at ties)."""
    rng = np.random.default_rng(16)
    x = (rng.standard_normal((200, 64)) * rng.uniform(0.1, 10, (200, 1))).astype(np.float32)
    codes, s, z = orc.int4_quantize_rows(x)
    S = np.repeat(s.view(np.float16).astype(np.float64), 32, axis=1)
    Z = np.repeat(z.view(np.float16).astype(np.float64), 32, axis=1)
    cand = np.arange(16)[None, None, :] * S[..., None] + Z[..., None]
    dist = np.abs(cand - x[..., None].astype(np.float64))
    best = dist.min(axis=2)
    chosen = np.take_along_axis(dist, codes[..., None].astype(np.int64), axis=2)[..., 0]
    assert np.all(chosen <= best + 1e-6 * np.maximum(1.0, S))


def test_e5m2_decode_exhaustive_matches_torch_fp16_and_page(orc):
    """Every E5M2 code against torch's float8_e5m2, against the fp16 value
    whose top byte it is (same sign, exponent field and bias: the pages'
    "dynamic range identical to FP16"), and the pages' field widths."""
    g = read_golden_kv("fp8_e5m2.txt")
    codes = np.arange(256, dtype=np.uint8)
    got = orc.e5m2_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e5m2).float().numpy().astype(np.float64)
    as_f16 = orc.f16_decode(codes.astype(np.uint16) << 8)
    for r in (ref, as_f16):
        same = (got == r) | (np.isnan(got) & np.isnan(r))
        assert same.all()
    fin = np.isfinite(got)
    assert int(fin.sum()) == int(g["finite_codes"])
    assert got[fin].max() == float(g["max_finite"])
    pos = got[fin & (got > 0)]
    assert pos.min() == float(g["min_subnormal"])
    assert 1 + int(g["exponent_bits"]) + int(g["mantissa_bits"]) == 8
    # the smallest normal has exponent field 1 and fraction 0
    assert got[1 << int(g["mantissa_bits"])] == float(g["min_normal"])


def test_e5m2_encode_matches_torch_on_finite_range(orc):
    """Round-to-nearest-even into E5M2 against torch's cast, at every code,
    every midpoint between neighbours and random values in the finite range."""
    rng = np.random.default_rng(5)
    vals = np.sort(orc.e5m2_decode(np.arange(0, 0x7C, dtype=np.uint8)))
    mids = (vals[1:] + vals[:-1]) / 2
    rand = np.concatenate([rng.uniform(-57344, 57344, 20000),
                           rng.standard_normal(20000) * 1e-3, rng.standard_normal(20000)])
    for arr in (vals, -vals, mids, -mids, rand):
        arr = arr.astype(np.float32)
        ref = torch.from_numpy(arr).to(torch.float8_e5m2).view(torch.uint8).numpy()
        got = orc.e5m2_encode(arr.astype(np.float64))
        assert np.array_equal(got, ref)


def test_e5m2_roundtrip_and_saturation(orc):
    codes = np.array([c for c in range(256) if (c & 0x7C) != 0x7C], np.uint8)
    assert np.array_equal(orc.e5m2_encode(orc.e5m2_decode(codes)), codes)
    sat = orc.e5m2_encode(np.array([61440.0, 1e9, -70000.0]))
    assert list(sat) == [0x7B, 0x7B, 0xFB]


def test_fp8_e5m2_row_quantizer(orc):
    """scale = max(absmax / 57344, 1e-12) in fp32; the absmax element maps to
    +-57344; codes are the E5M2 rounding of fp32(x / scale)."""
    rng = np.random.default_rng(6)
    x = rng.standard_normal((64, 128)).astype(np.float32)
    x[3] = 0.0
    x[5, 7] = -900.0
    codes, scales = orc.fp8_quantize_rows(x, "e5m2")
    a = np.abs(x).max(axis=1)
    want = np.maximum((a / np.float32(57344.0)).astype(np.float32), np.float32(1e-12))
    assert np.array_equal(scales, want)
    y = (x / scales[:, None]).astype(np.float32)
    ref = torch.from_numpy(y).to(torch.float8_e5m2).view(torch.uint8).numpy()
    assert np.array_equal(codes, ref)
    dec = orc.e5m2_decode(codes)
    assert dec[5, 7] == -57344.0
    deq = orc.fp8_dequant(codes, scales, "e5m2")
    assert np.array_equal(deq, (dec.astype(np.float32) * scales[:, None]).astype(np.float32))
    # 2 mantissa bits: relative error at most 2^-3 for values in the normal range
    big = np.abs(y) >= 2.0 ** -14
    assert np.all(np.abs(deq[big] - x[big]) <= 2.0 ** -3 * np.abs(x[big]) * 1.0001)
