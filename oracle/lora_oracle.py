"""CPU oracle for the LoRA-adapted QKV projection that produces q, k, v for the attention path.

TEST INFRASTRUCTURE ONLY.  Only the test suite and the benchmark's CPU-baseline leg may import
this module.  The HIP library never calls it, and it never calls the HIP library.

Source: "Introducing Unsloth：LLM 训练提速 30 倍" (dbyun.net/tutorial/10038), "手动 Autograd":
each of Q, K, V is the input times an adapted weight, Q = X W~_q = X (W_q + A_q B_q), and
likewise for K and V, with W the frozen weight and A B the low-rank adapter.  With
x [T, K] (tokens x hidden), W [K, N], A [K, r], B [r, N] and an adapter scale s (the usual
alpha / r; the page's form is s = 1):
    Y = x (W + s A B)                                        (the merged-weight definition)
N stacks the query, key and value projections, N = (hq + 2 hkv) d; columns [0, hq d) are q,
then k, then v, each row-major [T, heads, d].

Pins (tests/oracle_pins.py): a scalar triple loop on tiny shapes, the unmerged two-step form
x W + s (x A) B, the zero-scale case against a product computed by a different routine, and
the q/k/v split against hand-placed columns.
"""
from __future__ import annotations

import numpy as np


def lora_qkv(x, w, a, b, scale: float = 1.0) -> np.ndarray:
    """Y = x (W + s A B) in float64: the projection with the adapter merged into the weight."""
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    merged = w + float(scale) * (a @ b)
    return x @ merged


def split_qkv(y, hq: int, hkv: int, d: int):
    """The stacked projection's columns as q [T, hq, d], k [T, hkv, d], v [T, hkv, d]."""
    y = np.asarray(y)
    t = y.shape[0]
    q = y[:, :hq * d].reshape(t, hq, d)
    k = y[:, hq * d:(hq + hkv) * d].reshape(t, hkv, d)
    v = y[:, (hq + hkv) * d:].reshape(t, hkv, d)
    return q, k, v
