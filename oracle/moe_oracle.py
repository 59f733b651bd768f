"""CPU oracle for grouping MoE routing assignments by expert.

TEST INFRASTRUCTURE ONLY.  Only the test suite and the benchmark's CPU-baseline leg may import
this module.  The HIP library never calls it, and it never calls the HIP library.

Source: [UN-2026] "如何用 Unsloth 和 NVIDIA 让 LLM 训练更快" (Unsloth x NVIDIA,
dbyun.net/tutorial/10079), §3 "一个更小但实用的 MoE 优化".  The routing step asks, for every
expert, which (token, slot) assignments of the router's [n_tokens, top_k] index matrix chose it.
The page's starting point asks that once per expert with a data-dependent `where`; its fix groups
all assignments at once: flatten, stable sort by expert, count per expert, offsets from the
counts, split.  Both give the same grouping; this oracle is the per-expert definition.

Outputs, for M = n_tokens * top_k flattened assignments f = token * top_k + slot:
  counts[e]   number of assignments to expert e
  offsets[e]  start of expert e's group (offsets[0] = 0, offsets[E] = M)
  perm[i]     the flat assignment at grouped position i: groups in expert order, and inside a
              group ascending f (the row-major order `where` returns, i.e. a stable sort)
  inv[f]      grouped position of flat assignment f (perm[inv[f]] = f)
  status      bit 1 set when some index lies outside [0, E); the other outputs are then not
              defined.

Pins (tests/oracle_pins.py): a token-by-token brute force on tiny inputs, numpy's stable argsort
plus bincount (the page's one-shot recipe through library routines), and the invariants
(permutation, non-decreasing experts, ascending inside groups, inverse).
"""
from __future__ import annotations

from typing import Dict

import numpy as np

STATUS_BAD_EXPERT = 1   # some index outside [0, n_experts)


def group_by_expert(router_indices, n_experts: int) -> Dict:
    """Counts, offsets, grouped order and its inverse, one expert at a time (the definition)."""
    idx = np.asarray(router_indices, dtype=np.int64)
    if idx.ndim != 2:
        raise ValueError("router_indices must be [n_tokens, top_k]")
    n_tokens, top_k = idx.shape
    m = n_tokens * top_k
    out = {"status": 0, "n_experts": int(n_experts), "n_assign": m}
    if m and (idx.min() < 0 or idx.max() >= n_experts):
        out["status"] = STATUS_BAD_EXPERT
        return out
    counts = np.zeros(n_experts, dtype=np.int64)
    perm = []
    for e in range(n_experts):
        tok, slot = np.nonzero(idx == e)          # row-major: by token, then slot
        counts[e] = tok.shape[0]
        perm.extend((tok * top_k + slot).tolist())
    perm = np.asarray(perm, dtype=np.int64)
    offsets = np.zeros(n_experts + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    inv = np.empty(m, dtype=np.int64)
    inv[perm] = np.arange(m)
    out.update(counts=counts, offsets=offsets, perm=perm, inv=inv)
    return out


def tokens_of_expert(grouping: Dict, e: int, top_k: int) -> np.ndarray:
    """The token ids routed to expert e, as the split of the grouped list ([UN-2026] §3 step 5)."""
    a, b = int(grouping["offsets"][e]), int(grouping["offsets"][e + 1])
    return grouping["perm"][a:b] // top_k
