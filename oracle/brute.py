"""Textbook attention in NumPy fp64 -- test infrastructure (oracle side).

softmax(q K^T * scale) V for one query row over contiguous K, V, written as
the formula reads ("KV Cache Optimization: 3x Faster LLM Inference on 24GB
VRAM", section "Why Standard Approaches Fail"): exponentials of the raw
scores, no max subtraction, so only small inputs are valid.  Used as an
independent pin of the C oracle on tiny cases.
"""
from __future__ import annotations

import numpy as np


def attention_row(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    s = (K.astype(np.float64) @ q.astype(np.float64)) * float(scale)
    e = np.exp(s)
    return (e[:, None] * V.astype(np.float64)).sum(axis=0) / e.sum()


def attention_loops(q, K, V, scale):
    """Same, with explicit Python loops (smallest cases only)."""
    n, D = K.shape
    e = []
    for t in range(n):
        acc = 0.0
        for d in range(D):
            acc += float(q[d]) * float(K[t, d])
        e.append(np.exp(acc * float(scale)))
    tot = sum(e)
    return np.array([sum(e[t] * float(V[t, d]) for t in range(n)) / tot for d in range(D)])
