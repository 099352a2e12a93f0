"""Pins of the oracle's FP8 cache with one scale per (block, KV head).

"Reducing LLM Inference Latency: KV Cache Quantization and PagedAttention in
vLLM" (section "Block-Wise Scaling Factors") quantises a whole block with one
absmax scale: scale = max|block| / 448 (clamped by eps), codes =
float8_e4m3fn(block / scale).  Tokens of a decode reach a block one at a
time, so the oracle raises the block scale as they arrive and requantises the
block's earlier codes when it grows.  Whatever the arrival order, the final
scale is the page's formula over the whole block; when the largest token
arrives first nothing is requantised and the codes are exactly the page's
quantisation of the block (checked against torch's float8_e4m3fn cast); in
every order each value stays within two e4m3 roundings of its input.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402


def _append_all(kv_rows, order, p, D, H=1):
    """Write rows [p, H, D] (fp32-exact bf16 values) into one block of a
    pool, one token per call in `order` (offsets); returns pools."""
    d = oracle.desc("fp8_e4m3_block", "f32", H, D, p, 2)
    pools = oracle.pool_arrays("fp8_e4m3_block", 2, H, p, D, fill=0xA5)
    for off in order:
        k = np.ascontiguousarray(kv_rows[0][off:off + 1], np.float32)
        v = np.ascontiguousarray(kv_rows[1][off:off + 1], np.float32)
        oracle.reshape_and_cache(d, k, v, np.array([1 * p + off], np.int64), pools)
    return d, pools


def _rows(rng, p, D, H=1, outliers=False):
    x = rng.standard_normal((2, p, H, D)).astype(np.float32)
    if outliers:
        x[rng.random(x.shape) < 0.01] *= 20.0
    return x


@pytest.mark.parametrize("p", [16, 32])
def test_block_scale_is_the_page_formula_in_any_order(orc, p):
    rng = np.random.default_rng(p)
    D = 64
    for trial in range(6):
        x = _rows(rng, p, D, outliers=trial % 2 == 1)
        order = list(range(p))  # appends always fill offsets in order
        _, pools = _append_all(x, order, p, D)
        for which, name in ((0, "k_meta"), (1, "v_meta")):
            blk = torch.from_numpy(x[which][:, 0, :])
            want = (torch.max(torch.abs(blk)) / 448.0).clamp(min=1e-12).item()
            assert np.all(pools[name][1, 0] == np.float32(want))
            assert np.all(pools[name][0, 0].view(np.uint32) == 0xA5A5A5A5)  # other block


def test_largest_token_first_gives_the_page_quantisation(orc):
    rng = np.random.default_rng(3)
    p, D = 16, 64
    x = _rows(rng, p, D)
    x[:, 0, 0, 5] = 40.0  # token 0 holds the block's absmax: no requantisation later
    _, pools = _append_all(x, list(range(p)), p, D)
    for which, pool in ((0, "k_pool"), (1, "v_pool")):
        blk = torch.from_numpy(x[which][:, 0, :])
        scale = (torch.max(torch.abs(blk)) / 448.0).clamp(min=1e-12)
        want = (blk / scale).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        got = pools[pool][1, 0] if which == 0 else pools[pool][1, 0].T
        assert np.array_equal(got, want)


@pytest.mark.parametrize("outliers", [False, True])
def test_requantised_values_within_their_roundings(orc, outliers):
    """A token is rounded once when it is written and once more every time
    a later token raises the block scale; each rounding into e4m3 is within
    2^-4 of the value (3 fraction bits) or half the subnormal quantum."""
    rng = np.random.default_rng(11 + outliers)
    p, D = 16, 64
    raised = 0
    for trial in range(8):
        x = _rows(rng, p, D, outliers=outliers)
        x[:, -1] *= 8.0  # the last token raises the scale: everything is requantised
        d, pools = _append_all(x, list(range(p)), p, D)
        for which in (0, 1):
            K, V = oracle.gather(d, pools, np.array([1], np.int32), p, 0)
            got = (K, V)[which]
            ref = x[which][:, 0, :].astype(np.float64)
            tok = (torch.from_numpy(np.abs(x[which][:, 0, :])).max(dim=1).values / 448.0).clamp(
                min=1e-12).numpy()
            run = np.maximum.accumulate(tok)
            ups = np.concatenate([[0], (run[1:] > run[:-1]).astype(int)])
            r = ups[::-1].cumsum()[::-1] - ups  # raises after each token
            raised += int(r[0])
            s_fin = float(run[-1])
            k = (r + 1)[:, None].astype(np.float64)
            bound = ((1 + 2.0 ** -4) ** k - 1) * np.abs(ref) * 1.001 + k * 2.0 ** -10 * s_fin
            assert np.all(np.abs(got - ref) <= bound)
    assert raised >= 8


def test_per_block_error_exceeds_per_token_error_on_outlier_data(orc):
    """Quantisation error of the two FP8 scale granularities on data with 1%
    outliers at 20x (the FP8 workload's recipe): a block scale set by one
    outlier coarsens every other token of the block."""
    rng = np.random.default_rng(7)
    p, D, nblk = 16, 128, 64
    err_tok, err_blk, n = 0.0, 0.0, 0
    for b in range(nblk):
        x = _rows(rng, p, D, outliers=True)
        d, pools = _append_all(x, list(range(p)), p, D)
        K, _ = oracle.gather(d, pools, np.array([1], np.int32), p, 0)
        ref = x[0][:, 0, :].astype(np.float64)
        codes, scales = oracle.fp8_quantize_rows(x[0][:, 0, :])
        tok = oracle.fp8_dequant(codes, scales).astype(np.float64)
        err_blk += float(((K - ref) ** 2).sum())
        err_tok += float(((tok - ref) ** 2).sum())
        n += ref.size
    rms_tok, rms_blk = (err_tok / n) ** 0.5, (err_blk / n) ** 0.5
    print(f"\nFP8 E4M3 RMS error, 1% outliers x20: per token {rms_tok:.5f}, per block {rms_blk:.5f}")
    assert rms_blk > rms_tok
