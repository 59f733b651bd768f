"""Seeded synthetic packs: the only module shared by the HIP path's callers and the oracle's tests.

It draws inputs and nothing else: sequence lengths for a pack, and N(0,1) tensors rounded to
bfloat16.  It holds none of the attention arithmetic (no prefix sums, no RoPE, no softmax), so
a mistake in the method cannot hide here and show up identically on both sides.

The five workloads are the packs the attention path is measured on.  Their shapes come from the
model shapes the Unsloth/NVIDIA post names ("如何用 Unsloth 和 NVIDIA 让 LLM 训练更快",
dbyun.net/tutorial/10079, §1 "快速合理性验证" for the 2048-token synthetic pack and the
Llama-3.2-1B / Qwen3-0.6B runs, §1 "基准测试" for Qwen3-14B QLoRA SFT).  The pages' datasets are
not available; these seeded packs stand in for them.

Length recipe (all with ``numpy.random.default_rng(seed)``; draw until the sum reaches T, then
trim the last sequence so the pack holds exactly T tokens):
  tiny        fixed lengths [37, 100, 5, 114]
  llama1b     integers in [64, 512]
  qwen06b     rint(lognormal(ln 300, 0.8)) clipped to [1, 4096]
  qwen14b     integers in [256, 4096]
  skewed      four sequences of 8192, then integers in [1, 16]
Tensor recipe: per (layer l, tensor index k in q=0, k=1, v=2, dout=3) draw
``default_rng([seed, l, k]).standard_normal(shape, float32)``, multiply by the workload's input
scale (0.5 for qwen14b, else 1), and round to bfloat16 (round to nearest, ties to even).  The
arrays are returned as float32 holding bf16-exact values, so ``torch.tensor(a).bfloat16()`` is
exact and the oracle sees the very numbers the GPU sees.
"""
from __future__ import annotations

import dataclasses
from typing import Callable, List, Optional, Tuple

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    total_tokens: int
    hq: int
    hkv: int
    head_dim: int
    layers: int
    input_scale: float
    rope_base: float
    description: str

    @property
    def group(self) -> int:
        return self.hq // self.hkv

    @property
    def softmax_scale(self) -> float:
        return float(1.0 / np.sqrt(self.head_dim))


WORKLOADS = {
    "tiny": Workload("tiny", 256, 2, 1, 64, 1, 1.0, 10000.0,
                     "4 sequences [37,100,5,114], 2 q heads / 1 KV head, d=64, 1 layer"),
    "llama1b": Workload("llama1b", 2048, 32, 8, 64, 16, 1.0, 10000.0,
                        "Llama-3.2-1B-shaped: 2048 tokens, lengths U[64,512], 32/8 heads, d=64, 16 layers"),
    "qwen06b": Workload("qwen06b", 8192, 16, 8, 128, 28, 1.0, 10000.0,
                        "Qwen3-0.6B-shaped: 8192 tokens, lognormal(ln300,0.8) lengths, 16/8 heads, d=128, 28 layers"),
    "qwen14b": Workload("qwen14b", 16384, 40, 8, 128, 40, 0.5, 10000.0,
                        "Qwen3-14B-shaped: 16384 tokens, lengths U[256,4096], 40/8 heads, d=128, 40 layers, inputs x0.5"),
    "skewed": Workload("skewed", 65536, 32, 8, 128, 1, 1.0, 10000.0,
                       "skewed stress: 65536 tokens, 4x8192 then U[1,16], 32/8 heads, d=128, 1 layer"),
}
WORKLOAD_ORDER = ["tiny", "llama1b", "qwen06b", "qwen14b", "skewed"]


def _draw_until(total: int, prefix: List[int], draw: Callable[[], int]) -> List[int]:
    lengths = list(prefix)
    acc = sum(lengths)
    while acc < total:
        x = int(draw())
        lengths.append(x)
        acc += x
    if acc > total:
        lengths[-1] -= acc - total
    return lengths


def pack_lengths(name: str, seed: int = 0) -> np.ndarray:
    """Sequence lengths (int32) of the named pack; they sum to the workload's token count."""
    w = WORKLOADS[name]
    rng = np.random.default_rng(seed)
    if name == "tiny":
        out = [37, 100, 5, 114]
    elif name == "llama1b":
        out = _draw_until(w.total_tokens, [], lambda: rng.integers(64, 512, endpoint=True))
    elif name == "qwen06b":
        def one():
            x = np.rint(rng.lognormal(np.log(300.0), 0.8))
            return min(max(x, 1.0), 4096.0)
        out = _draw_until(w.total_tokens, [], one)
    elif name == "qwen14b":
        out = _draw_until(w.total_tokens, [], lambda: rng.integers(256, 4096, endpoint=True))
    elif name == "skewed":
        out = _draw_until(w.total_tokens, [8192] * 4, lambda: rng.integers(1, 16, endpoint=True))
    else:
        raise KeyError(name)
    arr = np.asarray(out, dtype=np.int32)
    assert int(arr.sum()) == w.total_tokens
    return arr


def random_lengths(rng: np.random.Generator, n_seqs: int, lo: int, hi: int) -> np.ndarray:
    """Free-form lengths for small test packs: n_seqs integers in [lo, hi]."""
    return rng.integers(lo, hi, size=n_seqs, endpoint=True).astype(np.int32)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returned as float32."""
    a = np.ascontiguousarray(x, dtype=np.float32)
    bits = a.view(np.uint32).astype(np.uint64)
    lsb = (bits >> 16) & 1
    rounded = ((bits + 0x7FFF + lsb) >> 16) << 16
    nan = np.isnan(a)
    out = rounded.astype(np.uint32).view(np.float32).copy()
    out[nan] = np.float32(np.nan)
    return out


def normal_bf16(shape: Tuple[int, ...], seed_words, scale: float = 1.0) -> np.ndarray:
    rng = np.random.default_rng(seed_words)
    x = rng.standard_normal(shape, dtype=np.float32)
    if scale != 1.0:
        x = x * np.float32(scale)
    return bf16_round(x)


def layer_tensors(w: Workload, layer: int, seed: int = 0,
                  total_tokens: Optional[int] = None) -> Tuple[np.ndarray, ...]:
    """(q, k, v, dout) for one layer, float32 arrays of bf16-exact values.

    q, dout: [T, hq, d]; k, v: [T, hkv, d].
    """
    t = w.total_tokens if total_tokens is None else total_tokens
    shapes = [(t, w.hq, w.head_dim), (t, w.hkv, w.head_dim), (t, w.hkv, w.head_dim), (t, w.hq, w.head_dim)]
    return tuple(normal_bf16(s, [seed, layer, idx], w.input_scale) for idx, s in enumerate(shapes))


# Hidden size of each pack's model (the K of the projection that produces its q, k, v):
# Llama-3.2-1B 2048, Qwen3-0.6B 1024, Qwen3-14B 5120; the tiny and skewed packs are not tied to a
# model and use hq x d.
PROJ_HIDDEN = {"tiny": 128, "llama1b": 2048, "qwen06b": 1024, "qwen14b": 5120, "skewed": 4096}


# MoE routing workloads ([UN-2026] §3 names GPT-OSS's router): a 16384-token batch routed top-4
# among 32 experts (gpt-oss-20b-shaped) or 128 experts (gpt-oss-120b-shaped).
MOE_WORKLOADS = {
    "gptoss20b": (16384, 32, 4),
    "gptoss120b": (16384, 128, 4),
}


def router_indices(n_tokens: int, n_experts: int, top_k: int, seed: int = 0,
                   skew: float = 1.0) -> np.ndarray:
    """Synthetic router output int32 [n_tokens, top_k]: each token's top_k experts (distinct, by
    descending logit) for logits N(0,1) plus a per-expert offset N(0, skew^2) that makes some
    experts popular, as trained routers are.  A random draw only: no grouping arithmetic."""
    rng = np.random.default_rng([seed, 77])
    bias = rng.standard_normal(n_experts) * skew
    logits = rng.standard_normal((n_tokens, n_experts)) + bias[None, :]
    return np.argsort(-logits, axis=1, kind="stable")[:, :top_k].astype(np.int32)


def small_problem(seed: int, lengths, hq: int, hkv: int, d: int, scale: float = 1.0):
    """(lengths, q, k, v, dout) for an ad-hoc pack used by tests."""
    lengths = np.asarray(lengths, dtype=np.int32)
    t = int(lengths.sum())
    shapes = [(t, hq, d), (t, hkv, d), (t, hkv, d), (t, hq, d)]
    arrs = tuple(normal_bf16(s, [seed, 1000 + idx], scale) for idx, s in enumerate(shapes))
    return (lengths,) + arrs
