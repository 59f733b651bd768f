"""HIP path vs the float64 oracle on the GPU, through the C ABI (needs an MI355X).

Metadata and work lists must match bit for bit; O, lse, dQ, dK, dV must match within the gate
(max-abs 2e-2 and relative L2 1e-2 per tensor; lse max-abs 1e-2).  Full-size workloads are
compared on whole sampled sequences and KV-head groups, which the oracle computes exactly
because packed sequences are independent (a property the oracle's own pins establish)."""
import math

import numpy as np
import pytest
import torch

import packed_sequence_causal_pk_amd as pk
from oracle import pk_oracle as O
from packed_sequence_causal_pk_amd import synth
from tests.gpu_helpers import LSE_MAX_ABS, MAX_ABS, compare, dev, meta_to_np, run_pk, say, to_np

pytestmark = pytest.mark.gpu


def _meta_matches_oracle(lengths, t):
    ref = O.build_meta(lengths, t)
    meta = pk.build_meta(torch.tensor(np.asarray(lengths, np.int32), device="cuda"), t)
    got = meta_to_np(meta)
    assert int(got["status"][0]) == ref["status"]
    assert np.array_equal(got["cu_seqlens"], ref["cu_seqlens"])
    assert int(got["max_seqlen"][0]) == ref["max_seqlen"]
    assert np.array_equal(got["seq_id"], ref["seq_id"])
    assert np.array_equal(got["pos"], ref["pos"])
    assert np.array_equal(got["fwd_items"], ref["fwd_items"])
    assert np.array_equal(got["bwd_items"], ref["bwd_items"])
    if ref["status"] == 0:
        assert np.array_equal(got["ds_off"], ref["ds_off"])
    return meta


@pytest.mark.parametrize("name", synth.WORKLOAD_ORDER)
def test_meta_bit_exact_workloads(name):
    say("meta", name)
    w = synth.WORKLOADS[name]
    _meta_matches_oracle(synth.pack_lengths(name), w.total_tokens)


def test_meta_bit_exact_fuzz():
    rng = np.random.default_rng(2024)
    for trial in range(24):
        hi = int(rng.choice([1, 2, 16, 200, 3000, 9000]))
        n = int(rng.integers(1, 5000 if hi <= 200 else 60))
        lengths = rng.integers(1, hi, size=n, endpoint=True).astype(np.int32)
        t = int(lengths.sum())
        say("meta fuzz", trial, "n", n, "T", t)
        _meta_matches_oracle(lengths, t)


def test_meta_invalid_lengths_flag_and_zero_outputs():
    for lengths, t in (([3, 0, 5], 8), ([4, -2, 6], 8), ([3, 3], 7), ([200, 100], 250)):
        say("invalid pack", lengths, t)
        ref = O.build_meta(lengths, t)
        lens_d = torch.tensor(lengths, dtype=torch.int32, device="cuda")
        meta = pk.build_meta(lens_d, t)
        status, _ = meta.check()
        assert status == ref["status"] and status != 0
        q = torch.randn(t, 2, 64, device="cuda").bfloat16()
        k = torch.randn(t, 1, 64, device="cuda").bfloat16()
        v = torch.randn(t, 1, 64, device="cuda").bfloat16()
        out = torch.full_like(q, 7.0)
        lse = torch.full((2, t), 7.0, device="cuda")
        pk.attn_fwd(meta, q, k, v, out=out, lse=lse)
        dq, dk, dv = pk.attn_bwd(meta, q, k, v, out, lse, q)
        torch.cuda.synchronize()
        for x in (out, lse, dq, dk, dv):
            assert torch.count_nonzero(x).item() == 0


def test_empty_pack():
    say("empty pack")
    meta = pk.build_meta(torch.zeros(0, dtype=torch.int32, device="cuda"), 0)
    status, mx = meta.check()
    assert status == 0 and mx == 0
    q = torch.zeros(0, 2, 64, device="cuda", dtype=torch.bfloat16)
    k = torch.zeros(0, 1, 64, device="cuda", dtype=torch.bfloat16)
    out, lse = pk.attn_fwd(meta, q, k, k)
    dq, dk, dv = pk.attn_bwd(meta, q, k, k, out, lse, q)
    torch.cuda.synchronize()
    assert out.shape == (0, 2, 64) and dq.shape == (0, 2, 64)


SMALL_CASES = [
    # (lengths, hq, hkv, d)
    ([37, 100, 5, 114], 2, 1, 64),          # the tiny workload's pack
    ([1], 2, 1, 64),                         # a single token
    ([1, 1, 1, 1, 1], 4, 2, 128),            # only length-1 sequences
    ([300], 2, 2, 128),                      # one sequence, ragged last tile
    ([700, 1, 29], 5, 1, 128),               # long sequence across tiles, GQA 5
    ([128, 128], 3, 3, 64),                  # tile-aligned boundaries, MHA
    ([64, 1, 63, 130, 2, 250], 8, 2, 64),    # boundaries inside tiles at many offsets
    ("short", 4, 1, 128),                    # many short sequences (1..16), skew-like
    ([2000, 47], 2, 1, 64),                  # long sequence, d = 64
    ([200, 56, 1], 16, 1, 64),               # 16 query heads on one KV head
    ([129, 127], 1, 1, 128),                 # a single head, boundaries one off the tile edge
]


@pytest.mark.parametrize("store", [True, False], ids=["ds_store", "recompute"])
@pytest.mark.parametrize("case", range(len(SMALL_CASES)))
def test_fwd_bwd_small(case, store):
    lengths, hq, hkv, d = SMALL_CASES[case]
    if lengths == "short":
        lengths = synth.random_lengths(np.random.default_rng(5), 120, 1, 16)
    say("small case", case, "T", int(np.sum(lengths)), "hq/hkv/d", hq, hkv, d, "dS store", store)
    lens, q, k, v, do = synth.small_problem(100 + case, lengths, hq, hkv, d)
    scale = 1.0 / math.sqrt(d)
    res = run_pk(lens, q, k, v, do, scale, store=store)
    o_ref, lse_ref = O.attn_fwd(q, k, v, lens, scale, 1e4)
    dq_ref, dk_ref, dv_ref = O.attn_bwd(q, k, v, do, lens, scale, 1e4)
    compare("out", to_np(res["out"]), o_ref)
    compare("lse", to_np(res["lse"]), lse_ref, max_abs=LSE_MAX_ABS)
    compare("dq", to_np(res["dq"]), dq_ref)
    compare("dk", to_np(res["dk"]), dk_ref)
    compare("dv", to_np(res["dv"]), dv_ref)


LAUNCH_SHAPE_CASES = [
    # (T, hq, hkv, d): packs on either side of the launch-shape choices.  128-token items x KV
    # heads <= 256 split each dK/dV item over two workgroups, and (from 64 up to twice the
    # device's compute units) run the dQ kernel on a side stream; items x query heads <= 2048 give
    # the forward 64-key tiles.
    (4096, 8, 8, 64),      # 32 items: split, side stream, 64-key forward tiles
    (4224, 16, 8, 64),     # 33 items: whole items, side stream, 64-key tiles
    (4224, 64, 8, 64),     # 2112 forward workgroups: 32-key tiles
    (8320, 8, 8, 128),     # 65 items x 8 = 520 > 512: one stream
]


@pytest.mark.parametrize("case", range(len(LAUNCH_SHAPE_CASES)))
def test_launch_shape_boundaries(case):
    t, hq, hkv, d = LAUNCH_SHAPE_CASES[case]
    rng = np.random.default_rng(700 + case)
    lengths = []
    while sum(lengths) < t:
        lengths.append(int(rng.integers(1, 600, endpoint=True)))
    lengths[-1] -= sum(lengths) - t
    lengths = [x for x in lengths if x > 0]
    say("launch shapes", case, "T", t, "hq/hkv/d", hq, hkv, d, "n", len(lengths))
    lens, q, k, v, do = synth.small_problem(700 + case, lengths, hq, hkv, d)
    scale = 1.0 / math.sqrt(d)
    res = run_pk(lens, q, k, v, do, scale)
    kv_heads = [0, hkv - 1]
    g = hq // hkv
    heads = [h for kvh in kv_heads for h in range(kvh * g, (kvh + 1) * g)]
    o_ref, lse_ref = O.attn_fwd(q, k, v, lens, scale, 1e4, heads=heads)
    dq_ref, dk_ref, dv_ref = O.attn_bwd(q, k, v, do, lens, scale, 1e4, kv_heads=kv_heads)
    compare("out", to_np(res["out"]), o_ref)
    compare("lse", to_np(res["lse"]), lse_ref, max_abs=LSE_MAX_ABS)
    compare("dq", to_np(res["dq"]), dq_ref)
    compare("dk", to_np(res["dk"]), dk_ref)
    compare("dv", to_np(res["dv"]), dv_ref)


SCALE_BASE_CASES = [
    # (softmax scale as a function of d, RoPE base, d, power-of-two factor on q and k)
    (lambda d: 1.0 / d, 1e4, 128, 4.0),
    (lambda d: 0.25, 5e5, 128, 0.5),
    (lambda d: 2.0 / math.sqrt(d), 1e6, 64, 0.5),
]


@pytest.mark.parametrize("case", range(len(SCALE_BASE_CASES)))
def test_softmax_scale_and_rope_base(case):
    """Softmax scales and RoPE bases other than the workloads' (the kernels fold the scale into
    their fp16 operands and exponents and read the table built for the base).  The max-abs gate
    is absolute and was set for scores of unit spread, so q and k are multiplied by a power of
    two (exact in bf16) that keeps scale * <q, k> near that spread."""
    scale_of, base, d, f = SCALE_BASE_CASES[case]
    scale = scale_of(d)
    say("scale %.6g base %g d %d qk factor %g" % (scale, base, d, f))
    lens, q, k, v, do = synth.small_problem(400 + case, [300, 1, 170, 45], 4, 2, d)
    q, k = (q * f).astype(np.float32), (k * f).astype(np.float32)
    res = run_pk(lens, q, k, v, do, scale, base)
    o_ref, lse_ref = O.attn_fwd(q, k, v, lens, scale, base)
    dq_ref, dk_ref, dv_ref = O.attn_bwd(q, k, v, do, lens, scale, base)
    compare("out", to_np(res["out"]), o_ref)
    compare("lse", to_np(res["lse"]), lse_ref, max_abs=LSE_MAX_ABS)
    compare("dq", to_np(res["dq"]), dq_ref)
    compare("dk", to_np(res["dk"]), dk_ref)
    compare("dv", to_np(res["dv"]), dv_ref)


@pytest.mark.parametrize("log2_scale", [-24, -12, 10])
def test_gradient_scale_invariance(log2_scale):
    """dout scaled by 2^e (exact in bf16) gives gradients scaled by 2^e: the backward's fp16
    operands follow the gradient's magnitude instead of under- or overflowing."""
    say("dout scaled by 2^%d" % log2_scale)
    lens, q, k, v, do = synth.small_problem(300, [90, 200, 3], 4, 2, 128)
    f = 2.0 ** log2_scale
    res = run_pk(lens, q, k, v, (do * f).astype(np.float32), 1.0 / math.sqrt(128))
    dq_ref, dk_ref, dv_ref = O.attn_bwd(q, k, v, do, lens, 1.0 / math.sqrt(128), 1e4)
    compare("dq", to_np(res["dq"]) / f, dq_ref)
    compare("dk", to_np(res["dk"]) / f, dk_ref)
    compare("dv", to_np(res["dv"]) / f, dv_ref)


@pytest.mark.parametrize("name", ["llama1b", "qwen06b"])
def test_ds_store_paths_agree(name):
    """The backward with a dS store, without one, and with one too small for the pack (the
    device then falls back to recomputing): dk and dv bitwise equal in all three (the store only
    adds writes), dq bitwise equal between the no-store and fall-back runs, and dq from the
    store within the gate of the oracle and of the recomputed dq."""
    w = synth.WORKLOADS[name]
    lengths = synth.pack_lengths(name)
    q, k, v, do = (dev(x) for x in synth.layer_tensors(w, 2))
    meta = pk.build_meta(torch.tensor(lengths, device="cuda"), w.total_tokens, max_seqlen=int(lengths.max()))
    out, lse = pk.attn_fwd(meta, q, k, v, w.softmax_scale)
    plain = pk.bwd_workspace(meta, w.hq, w.hkv, w.head_dim, store=False)
    full = pk.bwd_workspace(meta, w.hq, w.hkv, w.head_dim)
    small = torch.empty(plain.numel() + w.hq * 16384 * 4, dtype=torch.uint8, device="cuda")  # 4 blocks
    say("dS store paths", name, "workspace bytes", plain.numel(), full.numel(), small.numel())
    res = {}
    for key, ws in (("plain", plain), ("store", full), ("fallback", small)):
        res[key] = pk.attn_bwd(meta, q, k, v, out, lse, do, w.softmax_scale, workspace=ws)
    torch.cuda.synchronize()
    for key in ("store", "fallback"):
        assert torch.equal(res[key][1], res["plain"][1]) and torch.equal(res[key][2], res["plain"][2]), key
    assert torch.equal(res["fallback"][0], res["plain"][0])
    compare("dq~", to_np(res["store"][0]), to_np(res["plain"][0]))
    dq_ref, _, _ = O.attn_bwd(*synth.layer_tensors(w, 2), lengths, w.softmax_scale, w.rope_base)
    compare("dq", to_np(res["store"][0]), dq_ref)


def _bf16(x):
    """Round float32 values to bfloat16 (nearest even), kept as float32 (exact bf16 values)."""
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).bfloat16().float().numpy()


def _magnitude_gate(name, got, ref, max_abs=MAX_ABS):
    """The parity gate applied relative to the tensor's magnitude: the absolute max-abs bound
    was set for tensors of unit spread (scores and lse of order 1), so here it is scaled by
    max(1, max|ref| / 4); the relative-L2 bound is unchanged."""
    s = max(1.0, float(np.nanmax(np.abs(ref))) / 4.0)
    compare(name, np.asarray(got) / s, np.asarray(ref) / s, max_abs=max_abs)


def test_outlier_channels():
    """q and k with a few channels 4x larger and v with a few channels 512x larger (values to
    about 1600), the way trained projections concentrate magnitude in a few channels: results
    match the oracle (gate relative to each tensor's magnitude) and no range flag is raised.
    v's magnitude costs nothing (the backward scales v and dS by powers of two); the precision
    limit is the scores' magnitude, which fp16 operands resolve to about 2^-11 of their size
    (measured: q/k channels 8x larger put the backward at up to 7e-2 of this gate)."""
    lens, q, k, v, do = synth.small_problem(900, [300, 1, 170, 45, 512], 4, 2, 128)
    qk_ch, v_ch = [3, 64 + 3, 17, 100], [5, 70, 90, 127]
    q, k, v = q.copy(), k.copy(), v.copy()
    q[..., qk_ch] *= 4.0
    k[..., qk_ch] *= 4.0
    v[..., v_ch] *= 512.0
    say("outlier channels: max|q| %.1f max|k| %.1f max|v| %.1f" % (np.abs(q).max(), np.abs(k).max(), np.abs(v).max()))
    scale = 1.0 / math.sqrt(128)
    res = run_pk(lens, q, k, v, do, scale)
    status, _ = res["meta"].check()
    assert status == 0, status
    o_ref, lse_ref = O.attn_fwd(q, k, v, lens, scale, 1e4)
    # the backward forms D = rowsum(dout * out) from the bf16 out it is handed; on outlier
    # channels near 1600 that rounding alone (2^-9 relative) moves dq by up to 1.4e-2 of the
    # scaled gate, so the backward is compared with the oracle handed the same out
    dq_ref, dk_ref, dv_ref = O.attn_bwd(q, k, v, do, lens, scale, 1e4, out=to_np(res["out"]))
    _magnitude_gate("out", to_np(res["out"]), o_ref)
    _magnitude_gate("lse", to_np(res["lse"]), lse_ref, max_abs=LSE_MAX_ABS)
    _magnitude_gate("dq", to_np(res["dq"]), dq_ref)
    _magnitude_gate("dk", to_np(res["dk"]), dk_ref)
    _magnitude_gate("dv", to_np(res["dv"]), dv_ref)


@pytest.mark.parametrize("log2_v", [14, 40])
def test_backward_large_v(log2_v):
    """The backward with v multiplied by 2^e, past fp16's range (2^14 takes max|v| to about
    7e4, 2^40 to about 5e12): its fp16 copy of v and its dS are scaled by the power of two tau,
    so dQ and dK come out multiplied by 2^e and dV unchanged, with no range flag.  The forward
    outputs for the large v are formed exactly from a forward on the original v (O is linear in
    v and 2^e is exact in bf16; lse does not depend on v)."""
    lens, q, k, v, do = synth.small_problem(910, [400, 3, 250], 4, 2, 128)
    f = 2.0 ** log2_v
    scale = 1.0 / math.sqrt(128)
    meta = pk.build_meta(torch.tensor(lens, device="cuda"), int(lens.sum()))
    tq, tk, tv, tdo = dev(q), dev(k), dev(v), dev(do)
    out, lse = pk.attn_fwd(meta, tq, tk, tv, scale)
    big_v, big_out = tv * f, out * f
    say("v x 2^%d: max|v| %.3g" % (log2_v, float(big_v.float().abs().max())))
    dq, dk, dv = pk.attn_bwd(meta, tq, tk, big_v, big_out, lse, tdo, scale)
    torch.cuda.synchronize()
    status, _ = meta.check()
    assert status == 0, status
    dq_ref, dk_ref, dv_ref = O.attn_bwd(q, k, v, do, lens, scale, 1e4)
    compare("dq", to_np(dq) / f, dq_ref)
    compare("dk", to_np(dk) / f, dk_ref)
    compare("dv", to_np(dv), dv_ref)


def test_range_flag():
    """Inputs the fp16 operands cannot hold set PK_META_FP16_RANGE in the meta's range word,
    which pk_meta_check reports; the flag does not stop later calls, and a rebuild clears it."""
    lens, q, k, v, do = synth.small_problem(920, [100, 50], 2, 1, 64)
    lens_d = torch.tensor(lens, device="cuda")
    t = int(lens.sum())
    cases = []
    for what, idx, val in (("v", (10, 0, 5), 1.0e5), ("k", (0, 0, 3), 7.0e4), ("q", (100, 1, 7), 7.0e4)):
        qq, kk, vv = q.copy(), k.copy(), v.copy()
        {"q": qq, "k": kk, "v": vv}[what][idx] = val   # token 0 and 100 start sequences: position 0
        cases.append((what, qq, kk, vv))
    for what, qq, kk, vv in cases:
        meta = pk.build_meta(lens_d, t)
        assert meta.check()[0] == 0
        say("range flag from", what)
        pk.attn_fwd(meta, dev(qq), dev(kk), dev(vv))
        torch.cuda.synchronize()
        assert meta.check()[0] == 4, what   # PK_META_FP16_RANGE
        out, lse = pk.attn_fwd(meta, dev(q), dev(k), dev(v))   # still runs on a flagged meta
        torch.cuda.synchronize()
        assert torch.isfinite(out.float()).all().item()
        assert pk.build_meta(lens_d, t).check()[0] == 0
    # the backward flags a rotated q that exceeds the range once scaled: softmax scale 4 puts
    # |q| * scale * log2(e) past 65504 for |q| = 2e4 while the forward's unscaled copy holds it
    qq = q.copy()
    qq[0, 0, 2] = 2.0e4
    meta = pk.build_meta(lens_d, t)
    out, lse = pk.attn_fwd(meta, dev(qq), dev(k), dev(v), 4.0)
    torch.cuda.synchronize()
    assert meta.check()[0] == 0
    pk.attn_bwd(meta, dev(qq), dev(k), dev(v), out, lse, dev(do), 4.0)
    torch.cuda.synchronize()
    assert meta.check()[0] == 4


def _sub_pack(lengths, seqs):
    cu = np.concatenate([[0], np.cumsum(lengths)])
    idx = np.concatenate([np.arange(cu[s], cu[s + 1]) for s in seqs])
    return [int(lengths[s]) for s in seqs], idx


def _check_workload(name, layer, seqs=None, kv_heads=None, store=False):
    w = synth.WORKLOADS[name]
    lengths = synth.pack_lengths(name)
    q, k, v, do = synth.layer_tensors(w, layer)
    say("workload", name, "layer", layer, "seqs", "all" if seqs is None else len(seqs),
        "kv heads", "all" if kv_heads is None else list(kv_heads), "dS store", store)
    res = run_pk(lengths, q, k, v, do, w.softmax_scale, w.rope_base, store=store)
    if seqs is None:
        seqs = list(range(len(lengths)))
    sub_len, idx = _sub_pack(lengths, seqs)
    kvs = list(range(w.hkv)) if kv_heads is None else list(kv_heads)
    heads = [h for h in range(w.hq) if h // w.group in kvs]
    o_ref, lse_ref = O.attn_fwd(q[idx], k[idx], v[idx], sub_len, w.softmax_scale, w.rope_base, heads=heads)
    dq_ref, dk_ref, dv_ref = O.attn_bwd(q[idx], k[idx], v[idx], do[idx], sub_len, w.softmax_scale,
                                        w.rope_base, kv_heads=kvs)
    out = to_np(res["out"])[idx][:, heads]
    compare("out", out, o_ref[:, heads])
    compare("lse", to_np(res["lse"])[heads][:, idx], lse_ref[heads], max_abs=LSE_MAX_ABS)
    compare("dq", to_np(res["dq"])[idx][:, heads], dq_ref[:, heads])
    compare("dk", to_np(res["dk"])[idx][:, kvs], dk_ref[:, kvs])
    compare("dv", to_np(res["dv"])[idx][:, kvs], dv_ref[:, kvs])
    return res, lengths, (q, k, v, do)


def test_workload_tiny():
    _check_workload("tiny", 0)


@pytest.mark.parametrize("layer", [0, 15])
def test_workload_llama1b(layer):
    _check_workload("llama1b", layer)


@pytest.mark.parametrize("layer", [0, 27])
def test_workload_qwen06b(layer):
    _check_workload("qwen06b", layer)


@pytest.mark.parametrize("layer,store", [(0, False), (39, False), (0, True)])
def test_workload_qwen14b_sampled(layer, store):
    # the first and the last layer; the longest, the shortest and the last sequence plus one
    # from the middle of the pack; four of the eight KV-head groups (both ends and two inside);
    # layer 0 also through the dS store
    _check_workload("qwen14b", layer, seqs=[0, 4, 7, 9], kv_heads=[0, 3, 4, 7], store=store)


def test_workload_skewed_sampled():
    lengths = synth.pack_lengths("skewed")
    rng = np.random.default_rng(1)
    short = sorted(rng.choice(np.arange(4, len(lengths)), size=300, replace=False).tolist())
    # all four 8192-token sequences and 300 short ones, on the first and a middle KV-head group
    res, lengths, (q, k, v, do) = _check_workload("skewed", 0, seqs=[0, 1, 2, 3] + short, kv_heads=[0, 5])
    # closed forms on every length-1 sequence of the pack: O = V, lse = scale <q, k>,
    # dQ = dK = 0, dV = sum of the group's dout
    w = synth.WORKLOADS["skewed"]
    cu = np.concatenate([[0], np.cumsum(lengths)])
    ones = cu[:-1][lengths == 1]
    assert len(ones) == 249
    g = np.arange(w.hq) // w.group
    out, lse = to_np(res["out"])[ones], to_np(res["lse"])[:, ones]
    compare("out1", out, v[ones][:, g].astype(np.float64))
    lse_ref = w.softmax_scale * np.einsum("thd,thd->ht", q[ones].astype(np.float64), k[ones][:, g].astype(np.float64))
    compare("lse1", lse, lse_ref, max_abs=LSE_MAX_ABS)
    compare("dq1", to_np(res["dq"])[ones], np.zeros((len(ones), w.hq, w.head_dim)))
    compare("dk1", to_np(res["dk"])[ones], np.zeros((len(ones), w.hkv, w.head_dim)))
    dv_ref = do[ones].astype(np.float64).reshape(len(ones), w.hkv, w.group, w.head_dim).sum(axis=2)
    compare("dv1", to_np(res["dv"])[ones], dv_ref)


def test_meta_reuse_determinism_and_dk_invariant():
    """One meta reused by several layers gives the same results as a fresh meta per layer; fwd,
    dK and dV are bitwise repeatable; sum_j R(theta_j) dK_j = 0 per sequence and KV head."""
    w = synth.WORKLOADS["llama1b"]
    lengths = synth.pack_lengths("llama1b")
    say("meta reuse, llama1b")
    shared = pk.build_meta(torch.tensor(lengths, device="cuda"), w.total_tokens)
    for layer in (0, 1, 15):
        q, k, v, do = synth.layer_tensors(w, layer)
        a = run_pk(lengths, q, k, v, do, w.softmax_scale, meta=shared)
        b = run_pk(lengths, q, k, v, do, w.softmax_scale)
        c = run_pk(lengths, q, k, v, do, w.softmax_scale, meta=shared)
        for key in ("out", "lse", "dk", "dv"):
            assert torch.equal(a[key], b[key]) and torch.equal(a[key], c[key]), key
        assert torch.equal(a["dq"], b["dq"]) and torch.equal(a["dq"], c["dq"])
    pos = np.concatenate([np.arange(n) for n in lengths])
    dk = to_np(a["dk"])
    th = O.rope_angles(pos, w.head_dim, w.rope_base)
    c_, s_ = np.cos(th)[:, None, :], np.sin(th)[:, None, :]
    half = w.head_dim // 2
    dk_rot = np.concatenate([dk[..., :half] * c_ - dk[..., half:] * s_, dk[..., half:] * c_ + dk[..., :half] * s_], -1)
    cu = np.concatenate([[0], np.cumsum(lengths)])
    scale_ref = np.abs(dk).max()
    for s in range(len(lengths)):
        assert np.abs(dk_rot[cu[s]:cu[s + 1]].sum(axis=0)).max() < 2e-2 * max(1.0, scale_ref)


def test_autograd_function():
    say("autograd wrapper")
    lens, q, k, v, do = synth.small_problem(77, [50, 20, 1], 4, 2, 64)
    meta = pk.build_meta(torch.tensor(lens, device="cuda"), int(lens.sum()))
    tq, tk, tv = (dev(x).requires_grad_(True) for x in (q, k, v))
    out = pk.PackedCausalAttention.apply(tq, tk, tv, meta, 0.125, 1e4)
    out.backward(dev(do))
    dq_ref, dk_ref, dv_ref = O.attn_bwd(q, k, v, do, lens, 0.125, 1e4)
    compare("dq", to_np(tq.grad), dq_ref)
    compare("dk", to_np(tk.grad), dk_ref)
    compare("dv", to_np(tv.grad), dv_ref)


@pytest.mark.parametrize("d", [64, 128])
def test_max_tokens_sampled(d):
    """A pack of the largest supported size (PK_MAX_TOKENS tokens, lengths U[1, 2048] with every
    50th sequence of length 1): every
    64-bit offset and tile index is exercised.  Inputs are seeded N(0,1) tensors drawn on the
    device and rounded to bf16; a few whole sequences (the first, a long one, the last, and short
    ones) are copied back and checked against the oracle, and every length-1 sequence of the
    pack against the closed forms O = V, dQ = dK = 0."""
    t = 1 << 20   # PK_MAX_TOKENS
    rng = np.random.default_rng(11)
    lengths, acc = [], 0
    while acc < t:
        x = 1 if len(lengths) % 50 == 25 else int(rng.integers(1, 2048, endpoint=True))
        lengths.append(x)
        acc += x
    lengths[-1] -= acc - t
    lengths = np.asarray(lengths, np.int32)
    hq, hkv = 4, 1
    say("max-size pack: T", t, "sequences", len(lengths), "hq/hkv/d", hq, hkv, d)
    g = torch.Generator(device="cuda")
    g.manual_seed(1234 + d)
    mk = lambda *s: torch.randn(*s, generator=g, device="cuda").bfloat16()
    q, k, v, do = mk(t, hq, d), mk(t, hkv, d), mk(t, hkv, d), mk(t, hq, d)
    meta = pk.build_meta(torch.tensor(lengths, device="cuda"), t)
    scale = 1.0 / math.sqrt(d)
    out, lse = pk.attn_fwd(meta, q, k, v, scale)
    dq, dk, dv = pk.attn_bwd(meta, q, k, v, out, lse, do, scale)
    torch.cuda.synchronize()
    cu = np.concatenate([[0], np.cumsum(lengths)])
    longest = int(np.argmax(lengths))
    seqs = sorted({0, longest, len(lengths) - 1} | set(np.flatnonzero(lengths <= 8)[:20].tolist()))
    sub_len, idx = _sub_pack(lengths, seqs)
    tidx = torch.tensor(idx, device="cuda")
    host = lambda x: x.index_select(0, tidx).float().cpu().numpy().astype(np.float32)
    qs, ks, vs, dos = host(q), host(k), host(v), host(do)
    o_ref, lse_ref = O.attn_fwd(qs, ks, vs, sub_len, scale, 1e4)
    dq_ref, dk_ref, dv_ref = O.attn_bwd(qs, ks, vs, dos, sub_len, scale, 1e4)
    compare("out", host(out).astype(np.float64), o_ref)
    compare("lse", lse.index_select(1, tidx).cpu().numpy().astype(np.float64), lse_ref, max_abs=LSE_MAX_ABS)
    compare("dq", host(dq).astype(np.float64), dq_ref)
    compare("dk", host(dk).astype(np.float64), dk_ref)
    compare("dv", host(dv).astype(np.float64), dv_ref)
    ones = torch.tensor(cu[:-1][lengths == 1], device="cuda")
    say("length-1 sequences", len(ones))
    if len(ones):
        gmap = torch.arange(hq, device="cuda") // (hq // hkv)
        compare("out1", out.index_select(0, ones).float().cpu().numpy(),
                v.index_select(0, ones)[:, gmap].float().cpu().numpy())
        compare("dq1", dq.index_select(0, ones).cpu().numpy(), np.zeros((len(ones), hq, d)))
        compare("dk1", dk.index_select(0, ones).cpu().numpy(), np.zeros((len(ones), hkv, d)))


@pytest.mark.parametrize("name", ["tiny", "llama1b", "qwen06b"])
def test_split_backward_overlapped_matches_fused(name):
    """pk_attn_bwd_prep on a side stream and pk_attn_bwd_main on the current one, the prologue of
    each next layer overlapping the current layer's attention kernels through two workspaces (the
    benchmark's backward loop), give every layer the same dq, dk, dv as pk_attn_bwd."""
    w = synth.WORKLOADS[name]
    lengths = synth.pack_lengths(name)
    n_layers = 4
    say("split backward, overlapped", name, "layers", n_layers)
    meta = pk.build_meta(torch.tensor(lengths, device="cuda"), w.total_tokens)
    layers, ref = [], []
    for l in range(n_layers):
        q, k, v, do = (dev(x) for x in synth.layer_tensors(w, l))
        out, lse = pk.attn_fwd(meta, q, k, v, w.softmax_scale)
        layers.append((q, k, v, out, lse, do))
        ref.append(pk.attn_bwd(meta, q, k, v, out, lse, do, w.softmax_scale))
    torch.cuda.synchronize()
    cur, side = torch.cuda.current_stream(), torch.cuda.Stream()
    wss = [pk.bwd_workspace(meta, w.hq, w.hkv, w.head_dim) for _ in range(2)]
    ready, free, start = [torch.cuda.Event(), torch.cuda.Event()], [torch.cuda.Event(), torch.cuda.Event()], torch.cuda.Event()
    start.record(cur)
    side.wait_event(start)
    order = list(reversed(range(n_layers)))
    got = {}
    for i, l in enumerate(order):
        slot = i % 2
        if i == 0:
            q, k, v, out, lse, do = layers[l]
            pk.attn_bwd_prep(meta, q, k, v, out, lse, do, wss[0], w.softmax_scale, stream=side)
            ready[0].record(side)
        if i + 1 < n_layers:
            q, k, v, out, lse, do = layers[order[i + 1]]
            side.wait_event(free[1 - slot])
            pk.attn_bwd_prep(meta, q, k, v, out, lse, do, wss[1 - slot], w.softmax_scale, stream=side)
            ready[1 - slot].record(side)
        cur.wait_event(ready[slot])
        q = layers[l][0]
        dq = torch.empty(q.shape, dtype=torch.float32, device="cuda")
        dk = torch.empty((q.shape[0], w.hkv, w.head_dim), dtype=torch.float32, device="cuda")
        dv = torch.empty_like(dk)
        got[l] = pk.attn_bwd_main(meta, w.hq, w.hkv, w.head_dim, wss[slot], dq, dk, dv, w.softmax_scale)
        free[slot].record(cur)
    torch.cuda.synchronize()
    for l in range(n_layers):
        dq_a, dk_a, dv_a = got[l]
        dq_b, dk_b, dv_b = ref[l]
        assert torch.equal(dk_a, dk_b) and torch.equal(dv_a, dv_b), l
        assert torch.equal(dq_a, dq_b), l


def _fuzz_case(i):
    """Seeded random pack and head layout: 1..40 sequences mixing lengths 1..8 and 9..700, KV
    heads 1..8, query heads per KV head 1..6, d 64 or 128, the dS store on odd cases."""
    rng = np.random.default_rng(9000 + i)
    n = int(rng.integers(1, 41))
    short = rng.random(n) < 0.4
    lengths = np.where(short, rng.integers(1, 9, n), rng.integers(9, 701, n)).astype(np.int32)
    hkv = int(rng.integers(1, 9))
    group = int(rng.integers(1, 7))
    d = int(rng.choice([64, 128]))
    return lengths, hkv * group, hkv, d, bool(i % 2)


@pytest.mark.gpu
@pytest.mark.parametrize("case", range(16))
def test_random_packs_against_oracle(case):
    """Random packs and GQA layouts (including group sizes 3 and 5..6 and KV head counts that do
    not divide the 8 XCDs): every output against the oracle."""
    lengths, hq, hkv, d, store = _fuzz_case(case)
    say("fuzz case", case, "n_seqs", len(lengths), "T", int(lengths.sum()), "hq/hkv/d", hq, hkv, d,
        "dS store", store)
    lens, q, k, v, do = synth.small_problem(500 + case, lengths, hq, hkv, d)
    scale = 1.0 / math.sqrt(d)
    res = run_pk(lens, q, k, v, do, scale, store=store)
    o_ref, lse_ref = O.attn_fwd(q, k, v, lens, scale, 1e4)
    dq_ref, dk_ref, dv_ref = O.attn_bwd(q, k, v, do, lens, scale, 1e4)
    compare("out", to_np(res["out"]), o_ref)
    compare("lse", to_np(res["lse"]), lse_ref, max_abs=LSE_MAX_ABS)
    compare("dq", to_np(res["dq"]), dq_ref)
    compare("dk", to_np(res["dk"]), dk_ref)
    compare("dv", to_np(res["dv"]), dv_ref)


@pytest.mark.gpu
@pytest.mark.parametrize("d,store,hkv", [(64, False, 8), (128, False, 8), (128, True, 8), (64, False, 2)],
                         ids=["d64", "d128", "d128_ds_store", "d64_2kv"])
def test_persistent_dkdv_launch(d, store, hkv):
    """A pack whose (key tile, KV head) units outnumber the resident dK/dV workgroups (8506
    tokens in 28 sequences of 64..512: 67 tiles x 8 KV heads = 536 units; or, with 2 KV heads,
    40403 tokens in 140 sequences: 316 tiles x 2 = 632 units, so the XCD classes b mod 8 mix
    tiles and heads), so the dK/dV kernel runs as a persistent grid taking units from its work
    counters: every output against the oracle on the whole pack."""
    if hkv == 8:
        lengths = synth.random_lengths(np.random.default_rng(7), 28, 64, 512)
        hq = 16
    else:
        lengths = synth.random_lengths(np.random.default_rng(11), 140, 64, 512)
        hq = 4
    say("persistent dK/dV launch: T", int(np.sum(lengths)), "hq/hkv/d", hq, hkv, d, "dS store", store)
    lens, q, k, v, do = synth.small_problem(300 if hkv == 8 else 400, lengths, hq, hkv, d)
    assert -(-int(np.sum(lens)) // 128) * hkv > 256
    scale = 1.0 / math.sqrt(d)
    res = run_pk(lens, q, k, v, do, scale, store=store)
    o_ref, lse_ref = O.attn_fwd(q, k, v, lens, scale, 1e4)
    dq_ref, dk_ref, dv_ref = O.attn_bwd(q, k, v, do, lens, scale, 1e4)
    compare("out", to_np(res["out"]), o_ref)
    compare("lse", to_np(res["lse"]), lse_ref, max_abs=LSE_MAX_ABS)
    compare("dq", to_np(res["dq"]), dq_ref)
    compare("dk", to_np(res["dk"]), dk_ref)
    compare("dv", to_np(res["dv"]), dv_ref)


@pytest.mark.gpu
@pytest.mark.parametrize("store", [False, True], ids=["recompute", "ds_store"])
def test_bwd_main_repeats_on_one_prologue(store):
    """The dK/dV kernel's persistent launch (Qwen3-14B-shaped pack: 1024 key-tile x KV-head units,
    more than the resident workgroups) takes its units from work counters in the workspace.  The
    prologue clears them (here over a workspace filled with 0xff bytes first), and the launch sets
    them back to zero as it ends, so pk_attn_bwd_main run three times on one pk_attn_bwd_prep
    gives bitwise the gradients of the fused pk_attn_bwd every time."""
    name = "qwen14b"
    w = synth.WORKLOADS[name]
    lengths = synth.pack_lengths(name)
    say("backward main x3 on one prologue", name, "store", store)
    meta = pk.build_meta(torch.tensor(lengths, device="cuda"), w.total_tokens, max_seqlen=max(lengths))
    q, k, v, do = (dev(x) for x in synth.layer_tensors(w, 0))
    out, lse = pk.attn_fwd(meta, q, k, v, w.softmax_scale)
    ref = pk.attn_bwd(meta, q, k, v, out, lse, do, w.softmax_scale,
                      workspace=pk.bwd_workspace(meta, w.hq, w.hkv, w.head_dim, store=store))
    ws = pk.bwd_workspace(meta, w.hq, w.hkv, w.head_dim, store=store)
    ws.fill_(255)
    pk.attn_bwd_prep(meta, q, k, v, out, lse, do, ws, w.softmax_scale)
    for rep in range(3):
        dq = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
        dk = torch.full((q.shape[0], w.hkv, w.head_dim), float("nan"), dtype=torch.float32, device="cuda")
        dv = torch.full_like(dk, float("nan"))
        pk.attn_bwd_main(meta, w.hq, w.hkv, w.head_dim, ws, dq, dk, dv, w.softmax_scale)
        torch.cuda.synchronize()
        assert torch.equal(dk, ref[1]) and torch.equal(dv, ref[2]), rep
        assert torch.equal(dq, ref[0]), rep


def test_layer_loop_makes_no_host_sync():
    """Building B once and running several layers' forward and backward through the binding
    issues no synchronising torch operation (torch's sync debug mode turns one into an error);
    the library itself calls no HIP synchronisation on this path (see the HIP API trace)."""
    w = synth.WORKLOADS["llama1b"]
    lengths_d = torch.tensor(synth.pack_lengths("llama1b"), device="cuda")
    t = w.total_tokens
    mk = lambda *s: torch.randn(*s, device="cuda").bfloat16()
    layers = [(mk(t, w.hq, w.head_dim), mk(t, w.hkv, w.head_dim), mk(t, w.hkv, w.head_dim),
               mk(t, w.hq, w.head_dim)) for _ in range(3)]
    outs = [(torch.empty(t, w.hq, w.head_dim, dtype=torch.bfloat16, device="cuda"),
             torch.empty(w.hq, t, device="cuda")) for _ in range(3)]
    dq = torch.empty(t, w.hq, w.head_dim, device="cuda")
    dk = torch.empty(t, w.hkv, w.head_dim, device="cuda")
    dv = torch.empty_like(dk)
    torch.cuda.synchronize()
    say("layer loop under torch.cuda.set_sync_debug_mode('error')")
    torch.cuda.set_sync_debug_mode("error")
    try:
        meta = pk.build_meta(lengths_d, t)
        ws_f = pk.fwd_workspace(meta, w.hq, w.hkv, w.head_dim)
        ws_b = pk.bwd_workspace(meta, w.hq, w.hkv, w.head_dim)
        for (q, k, v, _), (out, lse) in zip(layers, outs):
            pk.attn_fwd(meta, q, k, v, out=out, lse=lse, workspace=ws_f)
        for (q, k, v, do), (out, lse) in reversed(list(zip(layers, outs))):
            pk.attn_bwd(meta, q, k, v, out, lse, do, dq=dq, dk=dk, dv=dv, workspace=ws_b)
    finally:
        torch.cuda.set_sync_debug_mode(0)
    torch.cuda.synchronize()
    assert torch.isfinite(dq).all().item() and torch.isfinite(dk).all().item()


@pytest.mark.parametrize("name", ["llama1b", "qwen06b"])
def test_work_list_order_does_not_change_results(name):
    """Items write disjoint outputs, so the longest-first order only schedules: with both work
    lists of B shuffled in place, out, lse, dq, dk, dv are bitwise the same (no kernel of the path
    uses atomics, so a race between items, or an item that depended on its neighbours, would show
    here)."""
    w = synth.WORKLOADS[name]
    lengths = synth.pack_lengths(name)
    q, k, v, do = (dev(x) for x in synth.layer_tensors(w, 1))
    meta = pk.build_meta(torch.tensor(lengths, device="cuda"), w.total_tokens)
    say("shuffled work lists", name)

    def run():
        out, lse = pk.attn_fwd(meta, q, k, v, w.softmax_scale)
        dq, dk, dv = pk.attn_bwd(meta, q, k, v, out, lse, do, w.softmax_scale)
        torch.cuda.synchronize()
        return out, lse, dq, dk, dv

    a = run()
    view = meta.view()
    g = torch.Generator(device="cpu")
    g.manual_seed(3)
    for key in ("fwd_items", "bwd_items"):
        items = view[key]
        perm = torch.randperm(items.shape[0], generator=g).to("cuda")
        items.copy_(items[perm].clone())
    torch.cuda.synchronize()
    b = run()
    for name_, x, y in zip(("out", "lse", "dq", "dk", "dv"), a, b):
        assert torch.equal(x, y), name_


@pytest.mark.parametrize("name", ["tiny", "llama1b"])
def test_layer_loop_in_a_hip_graph(name):
    """The whole step (B built once, then every layer's forward and backward, including the dQ
    kernel's side stream on small packs) captured into one HIP graph: every replay, with eager
    work and synchronisations between replays, gives the eager results."""
    w = synth.WORKLOADS[name]
    lengths_d = torch.tensor(synth.pack_lengths(name), device="cuda")
    t, n_layers = w.total_tokens, min(w.layers, 3)
    layers = []
    for l in range(n_layers):
        q, k, v, do = (dev(x) for x in synth.layer_tensors(w, l))
        layers.append({"q": q, "k": k, "v": v, "do": do,
                       "out": torch.empty_like(q), "lse": torch.empty(w.hq, t, device="cuda"),
                       "dq": torch.empty(q.shape, device="cuda"),
                       "dk": torch.empty(k.shape, device="cuda"), "dv": torch.empty(k.shape, device="cuda")})
    meta0 = pk.build_meta(lengths_d, t)
    ws_f = pk.fwd_workspace(meta0, w.hq, w.hkv, w.head_dim)
    ws_b = pk.bwd_workspace(meta0, w.hq, w.hkv, w.head_dim)

    def step():
        meta = pk.build_meta(lengths_d, t)
        for x in layers:
            pk.attn_fwd(meta, x["q"], x["k"], x["v"], w.softmax_scale, out=x["out"], lse=x["lse"], workspace=ws_f)
        for x in reversed(layers):
            pk.attn_bwd(meta, x["q"], x["k"], x["v"], x["out"], x["lse"], x["do"], w.softmax_scale,
                        dq=x["dq"], dk=x["dk"], dv=x["dv"], workspace=ws_b)
        return meta

    say("layer loop in a HIP graph", name, "layers", n_layers)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        keep = step()   # warm up on the capture stream's pool
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ref = [{k_: x[k_].clone() for k_ in ("out", "lse", "dq", "dk", "dv")} for x in layers]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        captured = step()
    for rep in range(3):
        for x in layers:   # eager work between replays: clobber every output
            for k_ in ("out", "lse", "dq", "dk", "dv"):
                x[k_].fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for x, r in zip(layers, ref):
            for k_ in ("out", "lse", "dq", "dk", "dv"):
                assert torch.equal(x[k_], r[k_]), (rep, k_)
    del keep, captured


def test_binding_rejects_mismatched_outputs_and_workspaces():
    """Caller-supplied outputs and workspaces are checked in the binding before any launch."""
    lengths = [37, 100, 5, 114]
    t = sum(lengths)
    meta = pk.build_meta(torch.tensor(lengths, dtype=torch.int32, device="cuda"), t)
    q = torch.randn(t, 2, 64, device="cuda").bfloat16()
    k = torch.randn(t, 1, 64, device="cuda").bfloat16()
    v = torch.randn(t, 1, 64, device="cuda").bfloat16()
    bad = [dict(out=torch.empty(t, 2, 32, device="cuda").bfloat16()),
           dict(out=torch.empty(t, 2, 64, device="cuda")),
           dict(lse=torch.empty(t, 2, device="cuda")),
           dict(lse=torch.empty(2, 2 * t, device="cuda")[:, ::2]),
           dict(workspace=torch.empty(1 << 20, dtype=torch.uint8, device="cuda")[::2])]
    for kw in bad:
        say("attn_fwd rejects", sorted(kw))
        with pytest.raises(ValueError):
            pk.attn_fwd(meta, q, k, v, **kw)
    out, lse = pk.attn_fwd(meta, q, k, v)
    for kw in [dict(dq=torch.empty(t, 2, 64, device="cuda").bfloat16()),
               dict(dk=torch.empty(t, 2, 64, device="cuda")),
               dict(dv=torch.empty(t, 1, 32, device="cuda"))]:
        say("attn_bwd rejects", sorted(kw))
        with pytest.raises(ValueError):
            pk.attn_bwd(meta, q, k, v, out, lse, out, **kw)
    with pytest.raises(ValueError):
        pk.attn_bwd(meta, q, k, v, out, lse, out.float())
    with pytest.raises(ValueError):
        pk.dense_mask(meta, out=torch.empty(t, t + 1, dtype=torch.bool, device="cuda"))
    torch.cuda.synchronize()
