"""pk_attn_fwd_noalloc (the forward on the library's fixed per-device workspace) against
pk_attn_fwd and the float64 oracle, through the C ABI (needs an MI355X)."""
import math

import numpy as np
import pytest
import torch

import packed_sequence_causal_pk_amd as pk
from packed_sequence_causal_pk_amd import _lib
from oracle import pk_oracle as O
from packed_sequence_causal_pk_amd import synth
from tests.gpu_helpers import LSE_MAX_ABS, compare, dev, say, to_np

pytestmark = pytest.mark.gpu


def _run_both(name, seqs):
    """Forward of one layer of a seeded workload through pk_attn_fwd_noalloc and pk_attn_fwd:
    bitwise equal (same kernels, same inputs), and within the gate of the oracle on `seqs`."""
    w = synth.WORKLOADS[name]
    lengths = synth.pack_lengths(name)
    q, k, v, _ = synth.layer_tensors(w, 0)
    say("noalloc forward", name, "T", w.total_tokens, "hq/hkv/d", w.hq, w.hkv, w.head_dim)
    meta = pk.build_meta(torch.tensor(lengths, device="cuda"), w.total_tokens)
    tq, tk, tv = dev(q), dev(k), dev(v)
    out = torch.full_like(tq, float("nan"))
    lse = torch.full((w.hq, w.total_tokens), float("nan"), device="cuda")
    pk.attn_fwd_noalloc(meta, tq, tk, tv, out, lse, w.softmax_scale, w.rope_base)
    ref_out, ref_lse = pk.attn_fwd(meta, tq, tk, tv, w.softmax_scale, w.rope_base)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse)
    cu = np.concatenate([[0], np.cumsum(lengths)])
    idx = np.concatenate([np.arange(cu[s], cu[s + 1]) for s in seqs])
    sub = [int(lengths[s]) for s in seqs]
    heads = list(range(min(w.hq, 2 * w.group)))
    o_ref, l_ref = O.attn_fwd(q[idx], k[idx], v[idx], sub, w.softmax_scale, w.rope_base, heads=heads)
    compare("out", to_np(out)[idx][:, heads], o_ref[:, heads])
    compare("lse", to_np(lse)[heads][:, idx], l_ref[heads], max_abs=LSE_MAX_ABS)


def test_noalloc_forward_two_calls_second_smaller():
    """Two calls in a row on one device, the second on a smaller pack than the first (the
    array keeps the first call's contents; the second overwrites what it reads)."""
    _run_both("qwen14b", [7, 9])
    _run_both("llama1b", [0, 3, 9])


def test_noalloc_forward_rejects_workspace_beyond_the_array():
    """A pack whose forward workspace exceeds PK_NOALLOC_SCRATCH_BYTES is refused with
    PK_ERR_CAPACITY before anything is enqueued (out keeps its contents)."""
    t, hq, hkv, d = 32768, 16, 16, 128
    need = None
    meta = pk.build_meta(torch.tensor([t // 2, t // 2], dtype=torch.int32, device="cuda"), t)
    need = pk.lib().pk_attn_fwd_workspace_bytes(meta.handle, hq, hkv, d)
    say("workspace", need, "bytes vs array", _lib.PK_NOALLOC_SCRATCH_BYTES)
    assert need > _lib.PK_NOALLOC_SCRATCH_BYTES
    q = torch.zeros(t, hq, d, dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros(t, hkv, d, dtype=torch.bfloat16, device="cuda")
    out = torch.full_like(q, 3.0)
    lse = torch.full((hq, t), 3.0, device="cuda")
    with pytest.raises(pk.PkError) as e:
        pk.attn_fwd_noalloc(meta, q, kv, kv, out, lse)
    assert e.value.status == _lib.PK_ERR_CAPACITY
    torch.cuda.synchronize()
    assert bool((out == 3.0).all().item()) and bool((lse == 3.0).all().item())
