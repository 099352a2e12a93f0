"""A host model of the balanced split's line (no GPU).

The unit-stream decode kernel cuts the (sequence, KV head) runs of 16-token
units into one share per wave.  On the cost line, `rc` positions stand
before every run (its per-piece work); wave w takes the units whose
positions fall in [w L / NW, (w + 1) L / NW), and the first unit at or past
a boundary position is found from the prefix of units per sequence.  This
model follows the kernel's formulas (sk_cost, sk_unit_at, SkLine in
pkv_decode.hip) and checks, over random batches with empty and short
sequences, what the kernel relies on:

- the shares tile the unit line in order;
- the owner of every unit is worker_of(its cost position);
- a run's part count is worker_of(last) - worker_of(first) + 1, its parts
  belong to consecutive workers, and each part index is in range;
- no run has more than nu_max / 8 + 2 parts (the workspace's slots).
"""
import numpy as np
import pytest

SK_MIN_UNITS = 8


def _check(lengths, Hkv, workers, rc):
    B = len(lengths)
    nu = (np.asarray(lengths) + 15) // 16
    PU = np.concatenate([[0], np.cumsum(nu)]).astype(np.int64)
    U = Hkv * int(PU[B])
    if U == 0:
        return
    L = Hkv * (int(PU[B]) + rc * B)
    cap = U // SK_MIN_UNITS
    nw = workers if workers < cap else (cap if cap > 0 else 1)

    def start(w):
        return w * L // nw

    def worker_of(x):
        return ((x + 1) * nw - 1) // L

    def cost(b, kvh, u):
        return Hkv * (int(PU[b]) + rc * b) + kvh * (int(nu[b]) + rc) + rc + u

    def unit_at(y):
        if y >= L:
            return U
        lo, hi = 0, B - 1
        while lo < hi:
            mid = (lo + hi + 1) >> 1
            if Hkv * (int(PU[mid]) + rc * mid) <= y:
                lo = mid
            else:
                hi = mid - 1
        n = int(nu[lo])
        r = y - Hkv * (int(PU[lo]) + rc * lo)
        kvh = r // (n + rc)
        assert kvh < Hkv
        off = r - kvh * (n + rc) - rc
        return Hkv * int(PU[lo]) + kvh * n + max(off, 0)

    xs = [unit_at(start(w)) for w in range(nw + 1)]
    assert xs[0] == 0 and xs[nw] == U
    assert all(xs[i] <= xs[i + 1] for i in range(nw))
    owner = np.empty(U, np.int64)
    for w in range(nw):
        owner[xs[w]:xs[w + 1]] = w
    pmax = int(nu.max()) // SK_MIN_UNITS + 2
    for b in range(B):
        if nu[b] == 0:
            continue
        for kvh in range(Hkv):
            seg = Hkv * int(PU[b]) + kvh * int(nu[b])
            for u in range(int(nu[b])):
                assert owner[seg + u] == worker_of(cost(b, kvh, u))
            ws = sorted(set(owner[seg:seg + nu[b]].tolist()))
            parts = worker_of(cost(b, kvh, nu[b] - 1)) - worker_of(cost(b, kvh, 0)) + 1
            assert parts == len(ws) and ws == list(range(ws[0], ws[0] + len(ws)))
            assert parts <= pmax
            for w in ws:
                part = 0 if seg >= xs[w] else w - worker_of(cost(b, kvh, 0))
                assert 0 <= part < parts


@pytest.mark.parametrize("rc", [0, 1, 2])
def test_split_line_invariants(rc):
    rng = np.random.default_rng(100 + rc)
    for _ in range(100):
        B = int(rng.integers(1, 60))
        lengths = rng.integers(0, 3000, B)
        lengths[rng.random(B) < 0.2] = 0
        lengths[rng.random(B) < 0.2] = rng.integers(1, 40)
        Hkv = int(rng.choice([1, 2, 8]))
        workers = int(rng.choice([4, 64, 1024, 2048]))
        _check(lengths, Hkv, workers, rc)
