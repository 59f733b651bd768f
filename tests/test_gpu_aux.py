"""The steps around the attention path against the oracle, through the C ABI (needs an MI355X):
the materialised T x T mask and the MoE grouping bit for bit, the standalone RoPE within the
bfloat16 rounding bound (and the parity gate)."""
import numpy as np
import pytest
import torch

import packed_sequence_causal_pk_amd as pk
from oracle import lora_oracle as LO
from oracle import moe_oracle as MO
from oracle import pk_oracle as O
from packed_sequence_causal_pk_amd import synth
from tests.gpu_helpers import compare, dev, say, to_np

pytestmark = pytest.mark.gpu


def _meta(lengths, t=None):
    lengths = np.asarray(lengths, np.int32)
    t = int(lengths.sum()) if t is None else t
    return pk.build_meta(torch.tensor(lengths, device="cuda"), t)


# ------------------------------------------------------------------------- materialised mask
@pytest.mark.parametrize("lengths", [[5, 1, 7], [1], [16], [3, 29], [37, 100, 5, 114],
                                     "llama1b", "random"])
def test_dense_mask_bit_exact(lengths):
    if lengths == "llama1b":
        lengths = synth.pack_lengths("llama1b")
    elif lengths == "random":
        lengths = synth.random_lengths(np.random.default_rng(5), 40, 1, 60)
    lengths = np.asarray(lengths, np.int32)
    t = int(lengths.sum())
    say("dense mask T", t, "N", len(lengths))
    meta = _meta(lengths)
    out = torch.ones((t, t), dtype=torch.bool, device="cuda")
    pk.dense_mask(meta, out=out)
    torch.cuda.synchronize()
    ref = O.dense_mask(lengths) == 0.0
    assert np.array_equal(out.cpu().numpy(), ref)


def test_dense_mask_sampled_rows_large():
    # 8192-token pack (a 64 MiB mask): rows checked against the oracle's metadata one by one
    name = "qwen06b"
    lengths = synth.pack_lengths(name)
    t = int(lengths.sum())
    say("dense mask sampled rows", name, "T", t)
    ref = O.build_meta(lengths, t)
    mask = pk.dense_mask(_meta(lengths))
    torch.cuda.synchronize()
    rng = np.random.default_rng(9)
    rows = np.unique(np.concatenate([rng.integers(0, t, 200), ref["cu_seqlens"][:-1],
                                     ref["cu_seqlens"][1:] - 1, [t - 1]]))
    got = mask[torch.tensor(rows, device="cuda")].cpu().numpy()
    for r, row in zip(rows, got):
        start = int(ref["cu_seqlens"][ref["seq_id"][r]])
        expect = np.zeros(t, bool)
        expect[start:r + 1] = True
        assert np.array_equal(row, expect), r
    assert int(mask.sum().item()) == O.unmasked_pairs(lengths)


def test_dense_mask_invalid_meta_and_empty():
    meta = _meta([3, 0, 5], 8)
    out = torch.ones((8, 8), dtype=torch.bool, device="cuda")
    pk.dense_mask(meta, out=out)
    torch.cuda.synchronize()
    assert not out.any().item()
    empty = pk.dense_mask(_meta([], 0))
    assert empty.shape == (0, 0)


# ------------------------------------------------------------------------------ RoPE alone
def _rope_bound(got, ref):
    """bfloat16 rounding (nearest even) of the float32 rotation: |error| <= 2^-8 |ref| + 1e-5."""
    err = np.abs(got - ref)
    bound = 2.0 ** -8 * np.abs(ref) + 1e-5
    bad = err > bound
    assert not bad.any(), "RoPE outside the bf16 rounding bound at %d entries (worst %.3e)" % (
        int(bad.sum()), float((err - bound).max()))


@pytest.mark.parametrize("case", [("tiny", 2, 64), ("llama1b", 32, 64), ("qwen06b", 16, 128),
                                  ("qwen14b", 8, 128), ("ragged", 3, 128)])
@pytest.mark.parametrize("inverse", [False, True])
def test_rope_apply_vs_oracle(case, inverse):
    name, h, d = case
    lengths = (synth.random_lengths(np.random.default_rng(3), 23, 1, 90) if name == "ragged"
               else synth.pack_lengths(name))
    t = int(lengths.sum())
    say("rope", name, "T", t, "h", h, "d", d, "inverse", inverse)
    x = synth.normal_bf16((t, h, d), [7, h, d])
    meta = _meta(lengths)
    got = to_np(pk.rope_apply(meta, dev(x), 10000.0, inverse=inverse))
    ref_meta = O.build_meta(lengths, t)
    ref = O.rope_apply(x, ref_meta["pos"], 10000.0, inverse=inverse)
    compare("rope", got, ref)
    _rope_bound(got, ref)


def test_rope_apply_in_place_roundtrip_and_bases():
    lengths = synth.pack_lengths("tiny")
    t = int(lengths.sum())
    meta = _meta(lengths)
    pos = O.build_meta(lengths, t)["pos"]
    x = synth.normal_bf16((t, 4, 128), [8, 1])
    for base in (10000.0, 500000.0, 1e6):
        say("rope in place, base", base)
        tx = dev(x)
        pk.rope_apply(meta, tx, base, out=tx)
        fwd = to_np(tx)
        _rope_bound(fwd, O.rope_apply(x, pos, base))
        pk.rope_apply(meta, tx, base, inverse=True, out=tx)
        back = to_np(tx)
        # the transpose undoes the rotation: two bf16 roundings away from the input
        compare("roundtrip", back, x.astype(np.float64))


def test_rope_apply_invalid_meta_writes_zeros():
    meta = _meta([4, -1, 5], 8)
    x = torch.randn(8, 2, 64, device="cuda").bfloat16()
    out = pk.rope_apply(meta, x)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0


# --------------------------------------------------------------------------- MoE grouping
def _moe_check(idx, n_experts, ws=None):
    got = pk.moe_group(torch.tensor(np.ascontiguousarray(idx, np.int32), device="cuda"), n_experts,
                       workspace=ws)
    torch.cuda.synchronize()
    ref = MO.group_by_expert(idx, n_experts)
    assert int(got["status"].item()) == ref["status"] == 0
    for key in ("counts", "offsets", "perm", "inv"):
        assert np.array_equal(got[key].cpu().numpy(), ref[key]), key
    return got


@pytest.mark.parametrize("name", sorted(synth.MOE_WORKLOADS))
def test_moe_group_workloads(name):
    n_tok, n_exp, top_k = synth.MOE_WORKLOADS[name]
    say("moe", name, n_tok, n_exp, top_k)
    _moe_check(synth.router_indices(n_tok, n_exp, top_k), n_exp)


@pytest.mark.parametrize("shape", [(0, 4, 8), (1, 1, 1), (5, 2, 1024), (3000, 1, 7),
                                   (50001, 2, 64), (4096, 1, 2), (2048, 2, 1000), (777, 8, 256)])
def test_moe_group_edges(shape):
    n_tok, top_k, n_exp = shape
    say("moe edge", shape)
    rng = np.random.default_rng(n_tok + 31 * top_k + n_exp)
    idx = rng.integers(0, n_exp, size=(n_tok, top_k))
    _moe_check(idx, n_exp)


def test_moe_group_all_to_one_expert_and_workspace_reuse():
    ws = pk.moe_workspace(40000 * 2, 16, "cuda")
    for n_tok, e in ((40000, 5), (1234, 15), (40000, 0)):
        say("moe single expert", n_tok, e)
        idx = np.full((n_tok, 2), e, np.int64)
        idx[::7, 1] = (e + 1) % 16
        _moe_check(idx, 16, ws)


def test_moe_group_bad_index_sets_status():
    idx = np.random.default_rng(4).integers(0, 8, size=(5000, 2))
    idx[17, 1] = 8
    idx[4000, 0] = -3
    got = pk.moe_group(torch.tensor(idx.astype(np.int32), device="cuda"), 8)
    torch.cuda.synchronize()
    assert MO.group_by_expert(idx, 8)["status"] == MO.STATUS_BAD_EXPERT
    assert int(got["status"].item()) == MO.STATUS_BAD_EXPERT
    inv = got["inv"].cpu().numpy()
    assert inv[17 * 2 + 1] == -1 and inv[4000 * 2] == -1
    assert int(got["counts"].sum().item()) == idx.size - 2


def test_moe_group_repeatable():
    idx = torch.tensor(synth.router_indices(16384, 128, 4, seed=1), device="cuda")
    a = pk.moe_group(idx, 128)
    b = pk.moe_group(idx, 128)
    torch.cuda.synchronize()
    for key in a:
        assert torch.equal(a[key], b[key]), key


# ------------------------------------------------------------------ double-buffered reload
@pytest.mark.parametrize("double", [False, True])
def test_reload_pipeline_matches_resident(double):
    """Backward of several layers whose q, k, v, out, lse come back from pinned host memory
    through the two-slot pipeline ([UN-2026] §2 "用双缓冲检查点重载隐藏延迟"):
      * when a slot is acquired, its bytes equal the pinned sources of its layer (checked by a
        bitwise comparison enqueued on the compute stream right after the acquire, so it sees
        exactly what the backward reads, with no host synchronisation in between);
      * every layer's gradients are bit-identical to the backward on resident tensors;
      * the first and the last reloaded layer match the float64 oracle at the parity gate."""
    w = synth.WORKLOADS["llama1b"]
    lengths = synth.pack_lengths("llama1b")
    t, n_layers = w.total_tokens, 6
    say("reload pipeline, double =", double)
    meta = _meta(lengths)
    acts, douts, ref, host = [], [], [], []
    for l in range(n_layers):
        q, k, v, do = (dev(a) for a in synth.layer_tensors(w, l))
        out, lse = pk.attn_fwd(meta, q, k, v)
        acts.append([x.cpu().pin_memory() for x in (q, k, v, out, lse)])
        douts.append(do)
        ref.append(pk.attn_bwd(meta, q, k, v, out, lse, do))
    torch.cuda.synchronize()
    # device copies of the pinned sources, for the acquire-time comparison (bit patterns)
    bits = lambda x: x.view(torch.int16) if x.element_size() == 2 else x.view(torch.int32)
    srcs = [[bits(a.to("cuda")) for a in layer] for layer in acts]
    torch.cuda.synchronize()
    slots = [[torch.empty_like(a, device="cuda") for a in acts[0]] for _ in range(2)]
    pipe = pk.ReloadPipeline()
    got = [None] * n_layers
    same = [None] * n_layers
    order = list(reversed(range(n_layers)))

    def fetch(slot, l):
        for dst, src in zip(slots[slot], acts[l]):
            pipe.fetch(slot, dst, src)

    if double:
        fetch(0, order[0])
    for i, l in enumerate(order):
        s = i % 2 if double else 0
        if not double:
            fetch(0, l)
        elif i + 1 < n_layers:
            fetch(1 - s, order[i + 1])
        pipe.acquire(s)
        same[l] = torch.stack([torch.eq(bits(x), y).all() for x, y in zip(slots[s], srcs[l])])
        q, k, v, out, lse = slots[s]
        got[l] = pk.attn_bwd(meta, q, k, v, out, lse, douts[l])
        pipe.release(s)
    torch.cuda.synchronize()
    pipe.close()
    for l in range(n_layers):
        assert bool(same[l].all().item()), "layer %d: slot bytes differ from the pinned sources %s" % (
            l, same[l].tolist())
        for a, b in zip(got[l], ref[l]):
            assert torch.equal(a, b), "layer %d" % l
    for l in (order[0], order[-1]):
        q, k, v, do = synth.layer_tensors(w, l)
        dq_ref, dk_ref, dv_ref = O.attn_bwd(q, k, v, do, lengths, w.softmax_scale, w.rope_base)
        say("  reloaded layer", l, "vs oracle")
        compare("dq", to_np(got[l][0]), dq_ref)
        compare("dk", to_np(got[l][1]), dk_ref)
        compare("dv", to_np(got[l][2]), dv_ref)


# ------------------------------------------------------------------- measured roofline aids
def test_peak_microbenchmarks_run_and_are_plausible():
    """The matrix-core and HBM microbenchmarks run and land in a plausible range for the part
    (their figures are reported, not asserted tightly)."""
    say("peak microbenchmarks")
    tf = pk.peak_mfma_tflops(iters=2000, reps=1)
    bw = pk.peak_hbm_gbps(nbytes=256 << 20, reps=1)
    say("  mfma %.1f TFLOP/s, hbm %s GB/s" % (tf, bw))
    assert 200.0 < tf < 3000.0
    assert all(500.0 < v < 10000.0 for v in bw.values())


# ------------------------------------------------------------------ LoRA-adapted QKV projection
def _lora_inputs(t, k, n, r, seed):
    """bf16-exact inputs: x ~ N(0,1), W, A ~ N(0, 1/K), B ~ N(0, 1/(16 r)): x W has unit spread
    and the adapter term s x A B a spread of s / 4 (an adapter is a small correction to the frozen
    weight), so the outputs stay in the range the absolute 2e-2 gate was set for (bf16 rounding
    of |y| >= 8 alone is 2^-5)."""
    x = synth.normal_bf16((t, k), [seed, 1])
    w = synth.normal_bf16((k, n), [seed, 2], 1.0 / np.sqrt(k))
    a = synth.normal_bf16((k, r), [seed, 3], 1.0 / np.sqrt(k))
    b = synth.normal_bf16((r, n), [seed, 4], 0.25 / np.sqrt(r))
    return x, w, a, b


def _lora_run(x, w, a, b, scale):
    tx = dev(x)
    twt, tat, tbt = dev(w.T.copy()), dev(a.T.copy()), dev(b.T.copy())
    y = pk.lora_qkv(tx, twt, tat, tbt, scale)
    torch.cuda.synchronize()
    return to_np(y)


def _lora_bound(got, ref, x, w, a, b, scale):
    """The error the kernel's roundings allow, element by element: the bf16 output (half an ulp,
    <= 2^-8 |y|), the bf16 rounding of scale * x A (each entry within 2^-8 of itself, so
    2^-8 (|scale x A| |B|)), and fp32 accumulation over K (2^-20 (|x| |W|), generous)."""
    x64, w64 = np.asarray(x, np.float64), np.asarray(w, np.float64)
    u = np.abs(float(scale) * (x64 @ np.asarray(a, np.float64)))
    bound = (2.0 ** -8 * np.abs(ref) + 2.0 ** -8 * (u @ np.abs(np.asarray(b, np.float64)))
             + 2.0 ** -20 * (np.abs(x64) @ np.abs(w64)) + 1e-6)
    err = np.abs(got - ref)
    bad = err > bound
    assert not bad.any(), "LoRA QKV outside the rounding bound at %d entries (worst excess %.3e)" % (
        int(bad.sum()), float((err - bound).max()))


@pytest.mark.parametrize("shape", [(300, 256, 384, 16, 0.5), (1, 64, 128, 1, 1.0),
                                   (129, 128, 256, 64, 2.0), (1000, 640, 640, 8, 0.25),
                                   (64, 1024, 128, 16, 0.0)])
def test_lora_qkv_vs_oracle(shape):
    t, k, n, r, scale = shape
    say("lora qkv T K N r s", shape)
    x, w, a, b = _lora_inputs(t, k, n, r, t + k + n + r)
    got = _lora_run(x, w, a, b, scale)
    ref = LO.lora_qkv(x, w, a, b, scale)
    compare("y", got, ref)
    _lora_bound(got, ref, x, w, a, b, scale)


@pytest.mark.parametrize("name", ["llama1b", "qwen06b", "qwen14b"])
def test_lora_qkv_model_shapes_sampled(name):
    """The projections that produce each pack's q, k, v (the model's hidden size K,
    N = (hq + 2 hkv) d, rank 16); rows sampled, each checked against the oracle on its own."""
    wl = synth.WORKLOADS[name]
    t, k, n, r = wl.total_tokens, synth.PROJ_HIDDEN[name], (wl.hq + 2 * wl.hkv) * wl.head_dim, 16
    say("lora qkv", name, "T K N r", t, k, n, r)
    x, w, a, b = _lora_inputs(t, k, n, r, 5)
    got = _lora_run(x, w, a, b, 2.0)
    rows = np.unique(np.concatenate([np.random.default_rng(6).integers(0, t, 48), [0, t - 1]]))
    ref = LO.lora_qkv(x[rows], w, a, b, 2.0)
    compare("y", got[rows], ref)
    _lora_bound(got[rows], ref, x[rows], w, a, b, 2.0)
    q, kk, v = LO.split_qkv(got, wl.hq, wl.hkv, wl.head_dim)
    assert q.shape == (t, wl.hq, wl.head_dim) and v.shape == (t, wl.hkv, wl.head_dim)


def test_lora_qkv_empty_and_repeatable():
    x, w, a, b = _lora_inputs(0, 64, 128, 4, 9)
    y = pk.lora_qkv(dev(x), dev(w.T.copy()), dev(a.T.copy()), dev(b.T.copy()))
    torch.cuda.synchronize()
    assert y.shape == (0, 128)
    x, w, a, b = _lora_inputs(500, 256, 256, 16, 10)
    args = (dev(x), dev(w.T.copy()), dev(a.T.copy()), dev(b.T.copy()), 1.5)
    y1, y2 = pk.lora_qkv(*args), pk.lora_qkv(*args)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


# ------------------------------------------------------------------------------ maximum sizes
def test_moe_group_max_size_properties():
    """PK_MOE_MAX_ASSIGN assignments (2^24 tokens x top-4) among PK_MOE_MAX_EXPERTS experts: too
    large for the per-expert oracle, so the properties that define the grouping are checked on the
    device: counts are the per-expert tallies, offsets their exclusive scan, perm a permutation
    whose experts never decrease and whose flat indices ascend inside each group, inv its inverse.
    A sampled block of tokens is also checked against the oracle on its own routing."""
    from packed_sequence_causal_pk_amd import _lib
    n_tok, top_k, n_exp = _lib.PK_MOE_MAX_ASSIGN // 4, 4, _lib.PK_MOE_MAX_EXPERTS
    say("moe max size", n_tok, top_k, n_exp)
    g = torch.Generator(device="cuda")
    g.manual_seed(77)
    idx = torch.randint(0, n_exp, (n_tok, top_k), generator=g, device="cuda", dtype=torch.int32)
    r = pk.moe_group(idx, n_exp)
    torch.cuda.synchronize()
    flat = idx.reshape(-1).long()
    m = flat.numel()
    assert int(r["status"].item()) == 0
    counts = torch.bincount(flat, minlength=n_exp)
    assert torch.equal(r["counts"].long(), counts)
    assert int(r["offsets"][0].item()) == 0 and int(r["offsets"][-1].item()) == m
    assert torch.equal(r["offsets"][1:].long(), torch.cumsum(counts, 0))
    perm = r["perm"].long()
    experts = flat[perm]
    assert bool((experts[1:] >= experts[:-1]).all().item())
    same = experts[1:] == experts[:-1]
    assert bool((perm[1:][same] > perm[:-1][same]).all().item())
    assert torch.equal(r["inv"].long()[perm], torch.arange(m, device="cuda"))
    del perm, experts, same, counts


def test_dense_mask_max_tokens_sampled():
    """The largest mask (PK_MASK_MAX_TOKENS = 65536 tokens, 4 GiB) of the skewed pack: sampled
    rows against the oracle's metadata, and the total of kept pairs in closed form."""
    name = "skewed"
    lengths = synth.pack_lengths(name)
    t = int(lengths.sum())
    say("dense mask max size T", t)
    ref = O.build_meta(lengths, t)
    mask = pk.dense_mask(_meta(lengths))
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.random.default_rng(12).integers(0, t, 64),
                                     ref["cu_seqlens"][:4], [8191, 8192, t - 1]]))
    got = mask[torch.tensor(rows, device="cuda")].cpu().numpy()
    for r, row in zip(rows, got):
        start = int(ref["cu_seqlens"][ref["seq_id"][r]])
        assert row[start:r + 1].all() and not row[:start].any() and not row[r + 1:].any(), r
    assert int(mask.sum(dtype=torch.int64).item()) == O.unmasked_pairs(lengths)


def test_rope_apply_max_tokens_sampled():
    """RoPE over the largest pack (2^20 tokens, positions up to 2047) and 8 heads: sampled tokens
    against the oracle, within the bf16 rounding bound."""
    t = 1 << 20
    rng = np.random.default_rng(13)
    lengths, acc = [], 0
    while acc < t:
        x = int(rng.integers(1, 2048, endpoint=True))
        lengths.append(x)
        acc += x
    lengths[-1] -= acc - t
    lengths = np.asarray(lengths, np.int32)
    say("rope max size T", t)
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    x = torch.randn(t, 8, 128, generator=g, device="cuda").bfloat16()
    y = pk.rope_apply(_meta(lengths), x)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([rng.integers(0, t, 256), [0, t - 1]]))
    tr = torch.tensor(rows, device="cuda")
    xs = x.index_select(0, tr).float().cpu().numpy()
    pos = O.build_meta(lengths, t)["pos"][rows]
    ref = O.rope_apply(xs, pos, 10000.0)
    got = y.index_select(0, tr).float().cpu().numpy().astype(np.float64)
    _rope_bound(got, ref)


def test_dense_mask_flat_path_near_max():
    """A pack whose token count is not a multiple of 16 (the flattened-byte form of the kernel,
    runs crossing rows) at 65519 tokens, the largest such size below the limit: sampled rows
    against the oracle's metadata and the kept-pair total."""
    lengths = np.concatenate([synth.pack_lengths("skewed")[:-1], [0]]).astype(np.int32)
    lengths = lengths[lengths > 0]
    lengths[-1] -= int(lengths.sum()) - 65519
    t = int(lengths.sum())
    assert t == 65519 and lengths.min() >= 1
    say("dense mask flat path T", t)
    ref = O.build_meta(lengths, t)
    mask = pk.dense_mask(_meta(lengths))
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.random.default_rng(14).integers(0, t, 64), [0, 1, t - 2, t - 1]]))
    got = mask[torch.tensor(rows, device="cuda")].cpu().numpy()
    for r, row in zip(rows, got):
        start = int(ref["cu_seqlens"][ref["seq_id"][r]])
        assert row[start:r + 1].all() and not row[:start].any() and not row[r + 1:].any(), r
    assert int(mask.sum(dtype=torch.int64).item()) == O.unmasked_pairs(lengths)


def test_kernel_timing_from_two_host_threads():
    """Launches recorded from two host threads at once (each on its own stream) are all counted,
    and the recorded times are positive."""
    import threading
    lengths = [37, 100, 5, 114]
    t = sum(lengths)
    meta = pk.build_meta(torch.tensor(lengths, dtype=torch.int32, device="cuda"), t)
    g = torch.Generator(device="cuda").manual_seed(0)
    q = torch.randn(t, 2, 64, device="cuda", generator=g).bfloat16()
    k = torch.randn(t, 1, 64, device="cuda", generator=g).bfloat16()
    v = torch.randn(t, 1, 64, device="cuda", generator=g).bfloat16()
    torch.cuda.synchronize()
    n_calls = 25
    errors = []

    def worker():
        try:
            s = torch.cuda.Stream()
            ws = pk.fwd_workspace(meta, 2, 1, 64)
            out = torch.empty_like(q)
            lse = torch.empty((2, t), dtype=torch.float32, device="cuda")
            for _ in range(n_calls):
                pk.attn_fwd(meta, q, k, v, out=out, lse=lse, workspace=ws, stream=s)
            s.synchronize()
        except Exception as e:  # reported below, in the test's own thread
            errors.append(e)

    pk.prof_enable(True, ["fwd"])
    pk.prof_reset()
    try:
        threads = [threading.Thread(target=worker) for _ in range(2)]
        for th in threads:
            th.start()
        for th in threads:
            th.join()
        ms, n = pk.prof_query("fwd")
    finally:
        pk.prof_enable(False)
        pk.prof_reset()
    say("timed fwd launches", n, "total ms", ms)
    assert not errors, errors
    assert n == 2 * n_calls and ms > 0.0
