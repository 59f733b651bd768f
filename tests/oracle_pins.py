"""Pins that tie the CPU oracle to facts fixed outside itself.

Each pin is a plain function that raises AssertionError on failure, so the mutation tests can run
the whole set against deliberately broken copies of the oracle.  No pin reuses the oracle code it
checks: RoPE is checked against complex multiplication, packed attention against a dense T x T
mask and against torch's own scaled_dot_product_attention + autograd in float64, gradients
against central finite differences, and the metadata and work lists against hand-derived
fixtures and brute-force enumeration.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

from oracle import lora_oracle as LO
from oracle import moe_oracle as MO
from oracle import pk_oracle as O
from packed_sequence_causal_pk_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _problem(seed, lengths, hq=2, hkv=1, d=16):
    return synth.small_problem(seed, lengths, hq, hkv, d)


# ----------------------------------------------------------------------------------- metadata
def pin_meta_golden():
    """Hand-derived metadata and work lists of two small packs."""
    for name in ("meta_tiny_pack.json", "meta_ragged_pack.json"):
        with open(os.path.join(GOLDEN, name)) as f:
            g = json.load(f)
        m = O.build_meta(g["lengths"], g["total_tokens"])
        assert m["status"] == 0
        assert m["cu_seqlens"].tolist() == g["cu_seqlens"], name
        assert m["max_seqlen"] == g["max_seqlen"], name
        for a, b, s in g["seq_id_runs"]:
            assert np.all(m["seq_id"][a:b] == s), name
            assert m["pos"][a:b].tolist() == list(range(b - a)), name
        assert m["fwd_items"].tolist() == g["fwd_items"], name
        assert m["bwd_items"].tolist() == g["bwd_items"], name


def pin_meta_bruteforce():
    """Token-by-token enumeration: walk the pack and count."""
    rng = np.random.default_rng(7)
    for trial in range(30):
        n = int(rng.integers(1, 12))
        lengths = rng.integers(1, 60, size=n)
        t = int(lengths.sum())
        m = O.build_meta(lengths, t)
        assert m["status"] == 0
        tok = 0
        for s, ln in enumerate(lengths):
            assert m["cu_seqlens"][s] == tok
            for p in range(int(ln)):
                assert m["seq_id"][tok] == s and m["pos"][tok] == p
                tok += 1
        assert m["cu_seqlens"][n] == t
        assert m["max_seqlen"] == max(int(x) for x in lengths)
    assert O.build_meta([3, 0, 2], 5)["status"] & O.META_BAD_LENGTH
    assert O.build_meta([3, 2], 6)["status"] & O.META_BAD_TOTAL


def pin_worklist_coverage():
    """Every kept (query, key) pair lies in exactly one forward item's rectangle and exactly one
    backward item's rectangle; the tile costs sum to the tile-pairs the rectangles span; the
    lists are in LPT order (cost descending, ties by tile index)."""
    rng = np.random.default_rng(11)
    for trial in range(12):
        n = int(rng.integers(1, 9))
        lengths = rng.integers(1, 90, size=n)
        t = int(lengths.sum())
        r = 16
        m = O.build_meta(lengths, t, tile_rows=r)
        seq = np.repeat(np.arange(n), lengths)
        keep = (seq[:, None] == seq[None, :]) & (np.arange(t)[None, :] <= np.arange(t)[:, None])
        for items, qcols, kcols in ((m["fwd_items"], (0, 1), (2, 3)), (m["bwd_items"], (2, 3), (0, 1))):
            hits = np.zeros((t, t), dtype=np.int64)
            idx = [int(x) for x in items[:, 7]]
            assert sorted(idx) == list(range(-(-t // r)))
            for it in items:
                qa, qb = int(it[qcols[0]]), int(it[qcols[1]])
                ka, kb = int(it[kcols[0]]), int(it[kcols[1]])
                hits[qa:qb, ka:kb] += 1
                own = (qa, qb) if items is m["fwd_items"] else (ka, kb)
                assert own[0] % r == 0 and own[1] - own[0] <= r
                other = (ka, kb) if items is m["fwd_items"] else (qa, qb)
                assert it[6] == -(-(other[1] - other[0]) // r)
                assert seq[own[0]] == it[4] and seq[own[1] - 1] == it[5]
            assert np.all(hits[keep] == 1)
            costs = [(-int(it[6]), int(it[7])) for it in items]
            assert costs == sorted(costs)


# ----------------------------------------------------------------------------------------- RoPE
def pin_ds_block_offsets():
    """The dS store's block offsets by walking the pack: key tile u's first block comes after
    every block of tiles before it, and tile u has one block per 64 query rows from its first
    token to the end of the last sequence it touches (found by stepping token by token)."""
    rng = np.random.default_rng(17)
    for trial in range(12):
        n = int(rng.integers(1, 9))
        lengths = rng.integers(1, 300, size=n)
        t = int(lengths.sum())
        m = O.build_meta(lengths, t)
        owner = np.repeat(np.arange(n), lengths)
        tiles = -(-t // 128)
        want = [0]
        for u in range(tiles):
            last = owner[min(128 * (u + 1), t) - 1]
            end = 128 * u
            while end < t and owner[end] <= last:
                end += 1
            rows = end - 128 * u
            want.append(want[-1] + (rows + 63) // 64)
        assert m["ds_off"].tolist() == want, (trial, lengths.tolist())
    # one sequence of 300 tokens: tiles of 300, 172 and 44 rows -> 5, 3 and 1 blocks
    assert O.build_meta([300], 300)["ds_off"].tolist() == [0, 5, 8, 9]


def _rope_complex(x, pos, base):
    """Rotate-half RoPE as complex multiplication: (x1 + i x2) * exp(i theta)."""
    d = x.shape[-1]
    half = d // 2
    freq = np.array([base ** (-(2.0 * i) / d) for i in range(half)])
    z = x[..., :half] + 1j * x[..., half:]
    rot = np.exp(1j * np.outer(pos, freq))[:, None, :]
    w = z * rot
    return np.concatenate([w.real, w.imag], axis=-1)


def pin_rope():
    rng = np.random.default_rng(3)
    for d in (2, 8, 64, 128):
        x = rng.standard_normal((40, 3, d))
        pos = rng.integers(0, 9000, size=40)
        y = O.rope_apply(x, pos, 10000.0)
        assert np.allclose(y, _rope_complex(x, pos, 10000.0), rtol=0, atol=1e-10)  # ulp of the angle at pos ~9000
        # position 0 is the identity, rotation keeps the norm
        assert np.allclose(O.rope_apply(x, np.zeros(40, int), 10000.0), x, atol=0)
        assert np.allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1))
        # inverse is the transpose: <R x, y> == <x, R^T y>
        z = rng.standard_normal(x.shape)
        lhs = np.sum(O.rope_apply(x, pos, 500.0) * z)
        rhs = np.sum(x * O.rope_apply(z, pos, 500.0, inverse=True))
        assert abs(lhs - rhs) < 1e-9 * max(1.0, abs(lhs))
        assert np.allclose(O.rope_apply(y, pos, 10000.0, inverse=True), x, atol=1e-12)
    # scores depend only on the position difference
    q = rng.standard_normal((1, 1, 64))
    k = rng.standard_normal((1, 1, 64))
    s0 = np.sum(O.rope_apply(q, np.array([17]), 1e4) * O.rope_apply(k, np.array([5]), 1e4))
    s1 = np.sum(O.rope_apply(q, np.array([117]), 1e4) * O.rope_apply(k, np.array([105]), 1e4))
    assert abs(s0 - s1) < 1e-9
    # for one pair (d = 2) the angle per position step is exactly one radian
    y = O.rope_apply(np.array([[[1.0, 0.0]]]), np.array([1]), 10000.0)
    assert np.allclose(y[0, 0], [math.cos(1.0), math.sin(1.0)], atol=1e-15)


# -------------------------------------------------------------------------------------- forward
def pin_fwd_dense_equals_per_sequence():
    for seed, lengths, hq, hkv in ((1, [5, 9, 1, 12], 4, 2), (2, [30], 2, 1), (3, [1, 1, 1], 3, 3)):
        lens, q, k, v, _ = _problem(seed, lengths, hq, hkv, 16)
        sc = 1.0 / 4.0
        o1, l1 = O.attn_fwd(q, k, v, lens, sc, 1e4)
        o2, l2 = O.attn_fwd_dense(q, k, v, lens, sc, 1e4)
        assert np.allclose(o1, o2, rtol=0, atol=1e-12) and np.allclose(l1, l2, rtol=0, atol=1e-12)
        # each sequence computed alone, as a pack of one
        cu = np.concatenate([[0], np.cumsum(lens)])
        for s in range(len(lens)):
            a, b = cu[s], cu[s + 1]
            o3, l3 = O.attn_fwd(q[a:b], k[a:b], v[a:b], [b - a], sc, 1e4)
            assert np.allclose(o1[a:b], o3, atol=1e-12) and np.allclose(l1[:, a:b], l3, atol=1e-12)


def pin_fwd_rows_and_closed_forms():
    lens, q, k, v, _ = _problem(5, [1, 7, 1, 20, 1], 4, 2, 32)
    sc = 1.0 / math.sqrt(32)
    o, lse = O.attn_fwd(q, k, v, lens, sc, 1e4)
    cu = np.concatenate([[0], np.cumsum(lens)])
    for s in range(len(lens)):
        for h in range(4):
            p = O.sequence_probs(q, k, lens, sc, 1e4, s, h)
            assert np.allclose(p.sum(axis=1), 1.0, atol=1e-12)
            assert np.all(p[np.triu_indices(p.shape[0], 1)] == 0.0)
        a = cu[s]
        g = np.arange(4) // 2
        # the first row of a sequence sees only itself: O = V, lse = scale * <q, k> (RoPE at 0 is 1)
        for h in range(4):
            assert np.allclose(o[a, h], v[a, g[h]], atol=1e-12)
            assert abs(lse[h, a] - sc * float(np.dot(q[a, h].astype(float), k[a, g[h]].astype(float)))) < 1e-12


def pin_fwd_lse_reconstruction():
    """O_i = sum_j exp(S_ij - lse_i) V_j over the kept keys."""
    lens, q, k, v, _ = _problem(9, [13, 6], 2, 1, 16)
    v = v.astype(np.float64)
    sc = 0.25
    o, lse = O.attn_fwd(q, k, v, lens, sc, 1e4)
    pos = np.concatenate([np.arange(n) for n in lens])
    qr, kr = _rope_complex(q.astype(float), pos, 1e4), _rope_complex(k.astype(float), pos, 1e4)
    cu = [0, 13, 19]
    for s in range(2):
        for i in range(cu[s], cu[s + 1]):
            for h in range(2):
                acc = np.zeros(16)
                for j in range(cu[s], i + 1):
                    acc += math.exp(sc * float(qr[i, h] @ kr[j, 0]) - lse[h, i]) * v[j, 0]
                assert np.allclose(acc, o[i, h], atol=1e-12)


def _torch_reference(q, k, v, dout, lengths, scale, base):
    """float64 torch: RoPE by complex multiplication, SDPA with a boolean block-diagonal causal
    mask, GQA by repeat_interleave, gradients by autograd."""
    lengths = [int(x) for x in lengths]
    t, hq, d = q.shape
    hkv = k.shape[1]
    pos = torch.cat([torch.arange(n, dtype=torch.float64) for n in lengths])
    freq = base ** (-(2.0 * torch.arange(d // 2, dtype=torch.float64)) / d)
    rot = torch.polar(torch.ones(t, d // 2, dtype=torch.float64), pos[:, None] * freq[None, :])[:, None, :]

    def rope(x):
        z = torch.complex(x[..., : d // 2], x[..., d // 2:]) * rot
        return torch.cat([z.real, z.imag], dim=-1)

    tq = torch.tensor(q, dtype=torch.float64, requires_grad=True)
    tk = torch.tensor(k, dtype=torch.float64, requires_grad=True)
    tv = torch.tensor(v, dtype=torch.float64, requires_grad=True)
    seq = torch.repeat_interleave(torch.arange(len(lengths)), torch.tensor(lengths))
    idx = torch.arange(t)
    mask = (seq[:, None] == seq[None, :]) & (idx[None, :] <= idx[:, None])
    qq = rope(tq).permute(1, 0, 2)[None]
    kk = rope(tk).permute(1, 0, 2).repeat_interleave(hq // hkv, dim=0)[None]
    vv = tv.permute(1, 0, 2).repeat_interleave(hq // hkv, dim=0)[None]
    out = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, attn_mask=mask, scale=scale)
    out = out[0].permute(1, 0, 2)
    (out * torch.tensor(dout, dtype=torch.float64)).sum().backward()
    return out.detach().numpy(), tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


def pin_torch_sdpa_and_autograd():
    for seed, lengths, hq, hkv, d in ((21, [7, 1, 16, 3], 4, 2, 16), (22, [40], 3, 1, 32), (23, [2, 9], 2, 2, 8)):
        lens, q, k, v, do = _problem(seed, lengths, hq, hkv, d)
        sc = 1.0 / math.sqrt(d)
        o_t, dq_t, dk_t, dv_t = _torch_reference(q, k, v, do, lens, sc, 1e4)
        o, _ = O.attn_fwd(q, k, v, lens, sc, 1e4)
        dq, dk, dv = O.attn_bwd(q, k, v, do, lens, sc, 1e4)
        for a, b in ((o, o_t), (dq, dq_t), (dk, dk_t), (dv, dv_t)):
            assert np.allclose(a, b, rtol=0, atol=1e-10), np.abs(a - b).max()


# ------------------------------------------------------------------------------------- backward
def pin_bwd_finite_differences():
    lens, q, k, v, do = _problem(31, [6, 11, 1], 4, 2, 8)
    q, k, v, do = (x.astype(np.float64) for x in (q, k, v, do))
    sc = 1.0 / math.sqrt(8)
    dq, dk, dv = O.attn_bwd(q, k, v, do, lens, sc, 1e4)

    def loss(qq, kk, vv):
        o, _ = O.attn_fwd(qq, kk, vv, lens, sc, 1e4)
        return float(np.sum(o * do))

    rng = np.random.default_rng(0)
    eps = 1e-6
    for which, grad in ((0, dq), (1, dk), (2, dv)):
        for _ in range(12):
            args = [q.copy(), k.copy(), v.copy()]
            idx = tuple(int(rng.integers(0, n)) for n in args[which].shape)
            args[which][idx] += eps
            lp = loss(*args)
            args[which][idx] -= 2 * eps
            lm = loss(*args)
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - grad[idx]) <= 1e-6 * max(1.0, abs(grad[idx])), (which, idx, fd, grad[idx])


def pin_bwd_invariants():
    """sum_j R(theta_j) dK_j = 0 per sequence and KV head (rows of dS sum to zero); length-1
    sequences get dQ = dK = 0 and dV = sum of the group's dout; first rows get dQ = 0."""
    lens, q, k, v, do = _problem(41, [1, 9, 1, 14, 2], 6, 2, 16)
    sc = 0.25
    dq, dk, dv = O.attn_bwd(q, k, v, do, lens, sc, 1e4)
    pos = np.concatenate([np.arange(n) for n in lens])
    dk_rot = _rope_complex(dk, pos, 1e4)
    cu = np.concatenate([[0], np.cumsum(lens)])
    for s in range(len(lens)):
        a, b = cu[s], cu[s + 1]
        assert np.allclose(dk_rot[a:b].sum(axis=0), 0.0, atol=1e-12)
        assert np.allclose(dq[a], 0.0, atol=1e-12)
        if b - a == 1:
            assert np.allclose(dk[a], 0.0, atol=1e-12)
            for g in range(2):
                assert np.allclose(dv[a, g], do[a, 3 * g:3 * g + 3].astype(float).sum(axis=0), atol=1e-12)


def pin_bwd_given_output():
    """D formed from a given forward output: handed the exact O it changes nothing; handed
    another tensor X, dV is unchanged and each query's dQ_rot moves by the closed form
    -scale * (dout_i . (X_i - O_i)) * sum_j P_ij k_rot_j, because D enters dS = P (dP - D) as
    a per-row shift (checked on a length-1 sequence, where P = 1 and dQ_rot = scale *
    dout . (v - X) k_rot, and on every row of a longer pack)."""
    lens, q, k, v, do = _problem(31, [5, 1, 9], hq=4, hkv=2, d=8)
    sc = 0.4
    o, _ = O.attn_fwd(q, k, v, lens, sc, 1e4)
    base = O.attn_bwd(q, k, v, do, lens, sc, 1e4)
    same = O.attn_bwd(q, k, v, do, lens, sc, 1e4, out=o)
    for a, b in zip(base, same):
        assert np.allclose(a, b, rtol=0, atol=1e-12)
    x = o + np.random.default_rng(5).standard_normal(o.shape) * 0.1
    dq2, dk2, dv2 = O.attn_bwd(q, k, v, do, lens, sc, 1e4, out=x)
    assert np.allclose(dv2, base[2], rtol=0, atol=1e-12)
    pos = np.concatenate([np.arange(n) for n in lens])
    th = O.rope_angles(pos, 8, 1e4)
    c_, s_ = np.cos(th), np.sin(th)
    kr = np.concatenate([k[..., :4] * c_[:, None] - k[..., 4:] * s_[:, None],
                         k[..., 4:] * c_[:, None] + k[..., :4] * s_[:, None]], -1)
    rot = lambda y: np.concatenate([y[..., :4] * c_[:, None] - y[..., 4:] * s_[:, None],
                                    y[..., 4:] * c_[:, None] + y[..., :4] * s_[:, None]], -1)
    dqr_base, dqr2 = rot(base[0]), rot(dq2)
    cu = [0, 5, 6, 15]
    for s_i in range(3):
        a, b = cu[s_i], cu[s_i + 1]
        for h in range(4):
            g = h // 2
            p = O.sequence_probs(q, k, lens, sc, 1e4, s_i, h)
            shift = -sc * np.sum(do[a:b, h] * (x[a:b, h] - o[a:b, h]), axis=1)[:, None] * (p @ kr[a:b, g])
            assert np.allclose(dqr2[a:b, h], dqr_base[a:b, h] + shift, rtol=0, atol=1e-10)
    # length-1 sequence (token 5): dQ_rot = scale * (dout . (v - X)) k_rot
    for h in range(4):
        g = h // 2
        want = sc * float(np.dot(do[5, h], v[5, g] - x[5, h])) * kr[5, g]
        assert np.allclose(dqr2[5, h], want, rtol=0, atol=1e-10)


def pin_permutation_invariance():
    """Reordering the sequences of a pack reorders the outputs and changes nothing else."""
    lens, q, k, v, do = _problem(51, [4, 10, 1, 7], 2, 1, 16)
    sc = 0.25
    o, lse = O.attn_fwd(q, k, v, lens, sc, 1e4)
    dq, dk, dv = O.attn_bwd(q, k, v, do, lens, sc, 1e4)
    cu = np.concatenate([[0], np.cumsum(lens)])
    order = [2, 0, 3, 1]
    idx = np.concatenate([np.arange(cu[s], cu[s + 1]) for s in order])
    lens2 = [lens[s] for s in order]
    o2, lse2 = O.attn_fwd(q[idx], k[idx], v[idx], lens2, sc, 1e4)
    dq2, dk2, dv2 = O.attn_bwd(q[idx], k[idx], v[idx], do[idx], lens2, sc, 1e4)
    for a, b in ((o[idx], o2), (lse[:, idx], lse2), (dq[idx], dq2), (dk[idx], dk2), (dv[idx], dv2)):
        assert np.allclose(a, b, atol=1e-12)


# ----------------------------------------------------------------------- materialised mask
def pin_dense_mask():
    """The T x T keep pattern: a hand-derived 6-token pack, and a walk over pairs of tokens of
    random packs (same sequence, key not after the query)."""
    with open(os.path.join(GOLDEN, "dense_mask_small.json")) as f:
        g = json.load(f)
    keep = O.dense_mask(g["lengths"]) == 0.0
    assert [np.nonzero(r)[0].tolist() for r in keep] == g["visible"]
    rng = np.random.default_rng(11)
    for _ in range(10):
        lens = rng.integers(1, 20, size=int(rng.integers(1, 8)))
        keep = O.dense_mask(lens) == 0.0
        owner = []
        for s, n in enumerate(lens):
            owner += [s] * int(n)
        for i in range(len(owner)):
            for j in range(len(owner)):
                assert keep[i, j] == (owner[i] == owner[j] and j <= i)


def pin_unmasked_pairs():
    """Kept-pair totals: a pair-by-pair count over random packs (same sequence, key not after the
    query); a token walk over the seeded packs (a token at position p keeps p + 1 keys); and the
    seed-0 totals of the five seeded packs as recorded when their generator was fixed."""
    rng = np.random.default_rng(13)
    for _ in range(25):
        lens = rng.integers(1, 25, size=int(rng.integers(1, 9)))
        owner = []
        for s, n in enumerate(lens):
            owner += [s] * int(n)
        count = 0
        for i in range(len(owner)):
            for j in range(len(owner)):
                count += int(owner[i] == owner[j] and j <= i)
        assert O.unmasked_pairs(lens) == count
    assert O.unmasked_pairs([]) == 0 and O.unmasked_pairs([1]) == 1 and O.unmasked_pairs([1] * 7) == 7
    recorded = {"tiny": 12323, "llama1b": 278607, "qwen06b": 1983322, "qwen14b": 19425559,
                "skewed": 134432516}
    for name, total in recorded.items():
        lens = synth.pack_lengths(name)
        walk = 0
        for n in lens:
            for p in range(int(n)):
                walk += p + 1
        assert walk == total, name
        assert O.unmasked_pairs(lens) == total, name


# --------------------------------------------------------------------------- MoE grouping
def pin_moe_golden():
    """A hand-derived grouping with an expert that receives nothing."""
    with open(os.path.join(GOLDEN, "moe_group_tiny.json")) as f:
        g = json.load(f)
    r = MO.group_by_expert(g["router_indices"], g["n_experts"])
    assert r["status"] == 0
    for key in ("counts", "offsets", "perm", "inv"):
        assert r[key].tolist() == g[key], key
    top_k = len(g["router_indices"][0])
    for e, toks in enumerate(g["tokens_per_expert"]):
        assert MO.tokens_of_expert(r, e, top_k).tolist() == toks


def pin_moe_bruteforce():
    """Walk the assignments token by token, slot by slot, appending each to its expert's list."""
    rng = np.random.default_rng(12)
    for _ in range(20):
        n_tok, top_k, n_exp = int(rng.integers(0, 40)), int(rng.integers(1, 5)), int(rng.integers(1, 9))
        idx = rng.integers(0, n_exp, size=(n_tok, top_k))
        r = MO.group_by_expert(idx, n_exp)
        lists = [[] for _ in range(n_exp)]
        for t in range(n_tok):
            for s in range(top_k):
                lists[idx[t, s]].append(t * top_k + s)
        assert r["counts"].tolist() == [len(x) for x in lists]
        assert r["perm"].tolist() == sum(lists, [])
        start = 0
        for e in range(n_exp):
            assert r["offsets"][e] == start
            start += len(lists[e])
        assert r["offsets"][n_exp] == n_tok * top_k


def pin_moe_sort_and_bincount():
    """The one-shot recipe through numpy's own routines: a stable argsort of the flattened
    indices and a bincount give the same grouping; perm and inv are inverse permutations."""
    for n_exp in (1, 32, 128):
        idx = synth.router_indices(500, n_exp, min(4, n_exp), seed=3)
        r = MO.group_by_expert(idx, n_exp)
        flat = idx.reshape(-1)
        assert r["perm"].tolist() == np.argsort(flat, kind="stable").tolist()
        assert r["counts"].tolist() == np.bincount(flat, minlength=n_exp).tolist()
        assert np.all(r["inv"][r["perm"]] == np.arange(flat.shape[0]))
        assert np.all(np.diff(flat[r["perm"]]) >= 0)
    bad = MO.group_by_expert([[0, 5]], 5)
    assert bad["status"] == MO.STATUS_BAD_EXPERT
    assert MO.group_by_expert([[-1, 0]], 5)["status"] == MO.STATUS_BAD_EXPERT


# ------------------------------------------------------------------- LoRA QKV projection
def pin_lora_scalar_loops():
    """Y[t, n] = sum_k x[t, k] (W[k, n] + s sum_j A[k, j] B[j, n]), summed element by element."""
    rng = np.random.default_rng(21)
    t, k, n, r, s = 3, 5, 4, 2, 0.75
    x, w = rng.standard_normal((t, k)), rng.standard_normal((k, n))
    a, b = rng.standard_normal((k, r)), rng.standard_normal((r, n))
    y = LO.lora_qkv(x, w, a, b, s)
    for i in range(t):
        for c in range(n):
            acc = 0.0
            for kk in range(k):
                adapted = w[kk, c]
                for j in range(r):
                    adapted += s * a[kk, j] * b[j, c]
                acc += x[i, kk] * adapted
            assert abs(y[i, c] - acc) <= 1e-12 * max(1.0, abs(acc))


def pin_lora_unmerged_and_zero_scale():
    """The merged weight equals the two-step adapter path x W + s (x A) B (what a LoRA layer
    computes without merging); with s = 0 the projection is torch's own float64 matmul of x and W;
    the q/k/v split takes columns in q, k, v order."""
    rng = np.random.default_rng(22)
    x, w = rng.standard_normal((17, 48)), rng.standard_normal((48, 40))
    a, b = rng.standard_normal((48, 8)), rng.standard_normal((8, 40))
    y = LO.lora_qkv(x, w, a, b, 0.5)
    two_step = x @ w + 0.5 * ((x @ a) @ b)
    assert np.allclose(y, two_step, rtol=1e-12, atol=1e-10)
    plain = torch.matmul(torch.from_numpy(x), torch.from_numpy(w)).numpy()
    assert np.allclose(LO.lora_qkv(x, w, a, b, 0.0), plain, rtol=1e-12, atol=1e-10)
    q, k, v = LO.split_qkv(np.arange(2 * 40).reshape(2, 40), 3, 1, 8)   # (3 + 2) heads x 8 = 40
    assert q.shape == (2, 3, 8) and k.shape == (2, 1, 8) and v.shape == (2, 1, 8)
    assert q[1, 2, 7] == 40 + 23 and k[0, 0, 0] == 24 and v[1, 0, 3] == 40 + 35


ALL_PINS = [
    pin_meta_golden, pin_meta_bruteforce, pin_worklist_coverage, pin_ds_block_offsets, pin_rope,
    pin_fwd_dense_equals_per_sequence, pin_fwd_rows_and_closed_forms, pin_fwd_lse_reconstruction,
    pin_torch_sdpa_and_autograd, pin_bwd_finite_differences, pin_bwd_invariants,
    pin_bwd_given_output, pin_permutation_invariance, pin_dense_mask, pin_unmasked_pairs, pin_moe_golden, pin_moe_bruteforce,
    pin_moe_sort_and_bincount, pin_lora_scalar_loops, pin_lora_unmerged_and_zero_scale,
]
