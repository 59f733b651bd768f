"""CPU oracle for packed-sequence causal attention with GQA and rotate-half RoPE.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and the benchmark's
CPU-baseline leg may import this module.  The HIP library never calls it, and it never calls
the HIP library: the two share no code.

Everything is plain numpy in float64.  Each function is the plain definition of what the fast
path computes, written for a reader to check by eye against the pages:

  [UN-2026] "如何用 Unsloth 和 NVIDIA 让 LLM 训练更快" (Unsloth x NVIDIA, dbyun.net/tutorial/10079)
            §1 "缓存 Packed-Sequence 元数据": the packed batch and its metadata
            B = {lengths, cu_seqlens, max_seqlen, mask structure}, built once, used by every layer.
  [UN-2023] "Introducing Unsloth：LLM 训练提速 30 倍" (dbyun.net/tutorial/10038)
            "手动 Autograd": A(X) = softmax(Q K^T / sqrt(d) + M) V  (the printed scale is garbled;
            this oracle reads it as 1/sqrt(d)), and "OpenAI Triton kernels": rotate-half RoPE,
            out1 = x1 cos - x2 sin, out2 = x2 cos + x1 sin over the two halves of the head dim.

Readings where the pages are silent (each one is listed with its reason in the design notes):
  * M is 0 where key j lies in the same packed sequence as query i and j <= i, else -inf.
  * RoPE angle for pair i (0 <= i < d/2) at position p is p * base**(-2i/d); positions restart at
    0 in every packed sequence; K is rotated like Q, V is not.
  * GQA: q head h reads KV head h // (Hq/Hkv).
  * lse is the natural-log sum of exp over the scaled, masked scores, laid out [Hq, T].
  * The backward is the softmax calculus of the formula above: D = rowsum(dO*O),
    dS = P*(dP - D), dQ_rot = scale*dS K_rot, dK_rot = scale*dS^T Q_rot, dV = P^T dO, then
    dQ = R(-theta) dQ_rot and dK = R(-theta) dK_rot (the transpose of the rotation).
  * Work lists (tile-to-sequence lists for the fast path) follow rule W below.

Pins: every function here is checked by tests that do not reuse its code (complex-number RoPE,
dense masked attention, torch's own scaled_dot_product_attention and autograd in float64,
central finite differences, closed forms for length-1 sequences, brute-force coverage of the
work lists, a pair-by-pair count of the dense keep pattern for unmasked_pairs, printed kept-pair
totals of the seeded packs).  No function here is left "parity unpinned".
"""
from __future__ import annotations

from typing import Dict, Iterable, Optional, Sequence

import numpy as np

TILE_ROWS = 128          # work-list granularity, shared with the HIP library by specification
ITEM_FIELDS = 8          # int32 fields per work item

# status bits of the metadata build
META_BAD_LENGTH = 1      # some length < 1
META_BAD_TOTAL = 2       # lengths do not sum to the token count


# ----------------------------------------------------------------------------------------------
# Metadata B  ([UN-2026] §1)
# ----------------------------------------------------------------------------------------------
def build_meta(lengths: Sequence[int], total_tokens: int, tile_rows: int = TILE_ROWS) -> Dict:
    """B for one pack: cu_seqlens, max_seqlen, per-token seq_id/pos, both work lists, status.

    cu_seqlens[0] = 0, cu_seqlens[s+1] = cu_seqlens[s] + lengths[s]; max_seqlen = max(lengths);
    token t belongs to sequence s when cu_seqlens[s] <= t < cu_seqlens[s+1] and sits at position
    t - cu_seqlens[s] inside it.
    """
    lengths = np.asarray(lengths, dtype=np.int64)
    n = int(lengths.shape[0])
    status = 0
    if n and np.any(lengths < 1):
        status |= META_BAD_LENGTH
    cu = np.zeros(n + 1, dtype=np.int64)
    if n:
        cu[1:] = np.cumsum(lengths)
    if int(cu[-1]) != int(total_tokens):
        status |= META_BAD_TOTAL
    out = {"status": status, "n_seqs": n, "total_tokens": int(total_tokens),
           "cu_seqlens": cu, "max_seqlen": int(lengths.max()) if n else 0}
    if status:
        return out
    seq_id = np.empty(total_tokens, dtype=np.int64)
    pos = np.empty(total_tokens, dtype=np.int64)
    for s in range(n):
        a, b = int(cu[s]), int(cu[s + 1])
        seq_id[a:b] = s
        pos[a:b] = np.arange(b - a)
    out["seq_id"] = seq_id
    out["pos"] = pos
    fwd, bwd = work_lists(cu, seq_id, total_tokens, tile_rows)
    out["fwd_items"] = fwd
    out["bwd_items"] = bwd
    out["ds_off"] = ds_block_offsets(bwd, total_tokens, tile_rows)
    return out


DS_BLOCK_ROWS = 64       # query rows per block of the fast path's dS store


def ds_block_offsets(bwd_items: np.ndarray, total_tokens: int, tile_rows: int = TILE_ROWS,
                     block_rows: int = DS_BLOCK_ROWS) -> np.ndarray:
    """Where the fast path's backward keeps dS (an index layout of this build, not of the pages,
    like rule W): key tile u owns ceil((q_end - q_start) / block_rows) consecutive blocks, one per
    block of its backward item's query rows, in tile order; off[u] is the first, off[n] the
    total."""
    n_items = -(-total_tokens // tile_rows)
    blocks = np.zeros(n_items, dtype=np.int64)
    for item in bwd_items:
        blocks[int(item[7])] = -(-(int(item[3]) - int(item[2])) // block_rows)
    off = np.zeros(n_items + 1, dtype=np.int64)
    off[1:] = np.cumsum(blocks)
    return off


def work_lists(cu: np.ndarray, seq_id: np.ndarray, total_tokens: int, tile_rows: int = TILE_ROWS):
    """Rule W: one item per tile of `tile_rows` tokens, ordered longest-processing-time first.

    Forward item for query tile t (rows [q_start, q_end)): its keys run from the start of the
    first sequence the tile touches up to the tile's end,
        {q_start, q_end, kv_start = cu[seq_first], kv_end = q_end, seq_first, seq_last, cost, t}.
    Backward item for key tile u (rows [kv_start, kv_end)): its queries run from the tile's start
    to the end of the last sequence the tile touches,
        {kv_start, kv_end, q_start = kv_start, q_end = cu[seq_last + 1], seq_first, seq_last, cost, u}.
    cost = number of tiles the other range spans.  Each list is sorted by cost, largest first,
    ties by tile index, which is a total order.
    """
    r = tile_rows
    n_items = -(-total_tokens // r)
    fwd = np.zeros((n_items, ITEM_FIELDS), dtype=np.int64)
    bwd = np.zeros((n_items, ITEM_FIELDS), dtype=np.int64)
    for t in range(n_items):
        lo, hi = r * t, min(r * (t + 1), total_tokens)
        sf, sl = int(seq_id[lo]), int(seq_id[hi - 1])
        kv_start, kv_end = int(cu[sf]), hi
        fwd[t] = [lo, hi, kv_start, kv_end, sf, sl, -(-(kv_end - kv_start) // r), t]
        q_start, q_end = lo, int(cu[sl + 1])
        bwd[t] = [lo, hi, q_start, q_end, sf, sl, -(-(q_end - q_start) // r), t]
    fwd = fwd[sorted(range(n_items), key=lambda i: (-fwd[i, 6], i))]
    bwd = bwd[sorted(range(n_items), key=lambda i: (-bwd[i, 6], i))]
    return fwd, bwd


# ----------------------------------------------------------------------------------------------
# RoPE  ([UN-2023] "OpenAI Triton kernels")
# ----------------------------------------------------------------------------------------------
def rope_angles(pos: np.ndarray, head_dim: int, base: float) -> np.ndarray:
    """theta[t, i] = pos[t] * base**(-2i/head_dim) for i < head_dim/2."""
    half = head_dim // 2
    inv_freq = np.power(float(base), -2.0 * np.arange(half, dtype=np.float64) / head_dim)
    return np.asarray(pos, dtype=np.float64)[:, None] * inv_freq[None, :]


def rope_apply(x: np.ndarray, pos: np.ndarray, base: float, inverse: bool = False) -> np.ndarray:
    """Rotate-half RoPE on x [T, H, d]: with x1 = x[..., :d/2], x2 = x[..., d/2:],
    out = [x1 cos - x2 sin, x2 cos + x1 sin].  inverse=True applies the transpose (sin -> -sin),
    which is the rotation's backward."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    half = d // 2
    th = rope_angles(pos, d, base)
    c = np.cos(th)[:, None, :]
    s = np.sin(th)[:, None, :]
    if inverse:
        s = -s
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def kv_head_of(h: int, group: int) -> int:
    """GQA: query head h shares the KV head of its contiguous group."""
    return h // group


def causal_keep(n: int) -> np.ndarray:
    """Inside one packed sequence of length n: key j is visible to query i iff j <= i."""
    return np.tril(np.ones((n, n), dtype=bool))


# ----------------------------------------------------------------------------------------------
# Attention, one packed sequence and one query head at a time  ([UN-2023] "手动 Autograd")
# ----------------------------------------------------------------------------------------------
def _softmax_rows(s: np.ndarray):
    m = s.max(axis=1)
    e = np.exp(s - m[:, None])
    z = e.sum(axis=1)
    return e / z[:, None], m + np.log(z)


def _sequence_probs(qr: np.ndarray, kr: np.ndarray, scale: float):
    """P = softmax(scale * Qr Kr^T + M) and its lse for one sequence and head."""
    n = qr.shape[0]
    s = (qr @ kr.T) * scale
    s = np.where(causal_keep(n), s, -np.inf)
    return _softmax_rows(s)


def _prepare(q, k, lengths, base):
    lengths = np.asarray(lengths, dtype=np.int64)
    t = int(lengths.sum())
    meta = build_meta(lengths, t)
    if meta["status"]:
        raise ValueError("invalid pack: status %d" % meta["status"])
    qr = rope_apply(q, meta["pos"], base)
    kr = rope_apply(k, meta["pos"], base)
    return meta, qr, kr


def _seq_list(meta, seqs: Optional[Iterable[int]]):
    return range(meta["n_seqs"]) if seqs is None else list(seqs)


def attn_fwd(q, k, v, lengths, scale: float, base: float,
             seqs: Optional[Iterable[int]] = None, heads: Optional[Iterable[int]] = None):
    """O [T, Hq, d] and lse [Hq, T] in float64.  With `seqs`/`heads` only those sequences and
    query heads are computed; other entries stay NaN."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    t, hq, d = q.shape
    group = hq // k.shape[1]
    meta, qr, kr = _prepare(q, k, lengths, base)
    cu = meta["cu_seqlens"]
    out = np.full((t, hq, d), np.nan)
    lse = np.full((hq, t), np.nan)
    for s in _seq_list(meta, seqs):
        a, b = int(cu[s]), int(cu[s + 1])
        for h in (range(hq) if heads is None else heads):
            g = kv_head_of(h, group)
            p, l = _sequence_probs(qr[a:b, h], kr[a:b, g], scale)
            out[a:b, h] = p @ v[a:b, g]
            lse[h, a:b] = l
    return out, lse


def score_grad(p: np.ndarray, do: np.ndarray, v: np.ndarray, o: Optional[np.ndarray] = None) -> np.ndarray:
    """dS for one sequence and head: with O = P V and D_i = sum_d dO_i * O_i,
    dP = dO V^T and dS = P * (dP - D) (the softmax Jacobian applied to dP).  When `o` is given,
    D is formed from it instead of from P V: the backward receives the forward's output as an
    input and forms D from what it receives (the FlashAttention-2 form of the backward that
    "利用 Unsloth 和 NVIDIA 硬件加速 LLM 训练" §2 names), so a test can hand the oracle the same
    rounded output the fast path is given."""
    if o is None:
        o = p @ v
    dcap = np.sum(do * o, axis=1)
    dp = do @ v.T
    return p * (dp - dcap[:, None])


def query_grad(ds: np.ndarray, kr: np.ndarray, scale: float) -> np.ndarray:
    """dQ_rot = scale * dS K_rot."""
    return scale * (ds @ kr)


def key_grad(ds: np.ndarray, qr: np.ndarray, scale: float) -> np.ndarray:
    """dK_rot contribution of one query head = scale * dS^T Q_rot."""
    return scale * (ds.T @ qr)


def attn_bwd(q, k, v, dout, lengths, scale: float, base: float,
             seqs: Optional[Iterable[int]] = None, kv_heads: Optional[Iterable[int]] = None,
             out=None):
    """dQ [T, Hq, d], dK, dV [T, Hkv, d] in float64 for L = sum(O * dout).

    With `seqs`/`kv_heads`, only those sequences and KV heads (and the query heads of their
    groups) are computed; other entries stay NaN.  With `out` [T, Hq, d], D = rowsum(dout * out)
    is formed from that tensor (see score_grad); by default from the exact O."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    dout = np.asarray(dout, np.float64)
    t, hq, d = q.shape
    hkv = k.shape[1]
    group = hq // hkv
    meta, qr, kr = _prepare(q, k, lengths, base)
    cu = meta["cu_seqlens"]
    dqr = np.full((t, hq, d), np.nan)
    dkr = np.full((t, hkv, d), np.nan)
    dv = np.full((t, hkv, d), np.nan)
    kvs = range(hkv) if kv_heads is None else list(kv_heads)
    for s in _seq_list(meta, seqs):
        a, b = int(cu[s]), int(cu[s + 1])
        for g in kvs:
            dkr[a:b, g] = 0.0
            dv[a:b, g] = 0.0
        for h in range(hq):
            g = kv_head_of(h, group)
            if g not in kvs:
                continue
            p, _ = _sequence_probs(qr[a:b, h], kr[a:b, g], scale)
            do = dout[a:b, h]
            ds = score_grad(p, do, v[a:b, g], None if out is None else np.asarray(out, np.float64)[a:b, h])
            dv[a:b, g] += p.T @ do
            dqr[a:b, h] = query_grad(ds, kr[a:b, g], scale)
            dkr[a:b, g] += key_grad(ds, qr[a:b, h], scale)
    dq = rope_apply(dqr, meta["pos"], base, inverse=True)
    dk = rope_apply(dkr, meta["pos"], base, inverse=True)
    return dq, dk, dv


# ----------------------------------------------------------------------------------------------
# Dense form: one T x T block-diagonal causal mask over the whole pack.  Used only on tiny packs
# to check that attention over the pack equals attention over each sequence alone.
# ----------------------------------------------------------------------------------------------
def dense_mask(lengths) -> np.ndarray:
    """Additive M [T, T]: 0 where the key is in the query's sequence and not after it."""
    lengths = np.asarray(lengths, dtype=np.int64)
    seq = np.repeat(np.arange(lengths.shape[0]), lengths)
    t = seq.shape[0]
    idx = np.arange(t)
    keep = (seq[:, None] == seq[None, :]) & (idx[None, :] <= idx[:, None])
    return np.where(keep, 0.0, -np.inf)


def attn_fwd_dense(q, k, v, lengths, scale: float, base: float):
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    t, hq, d = q.shape
    group = hq // k.shape[1]
    lengths = np.asarray(lengths, dtype=np.int64)
    pos = np.concatenate([np.arange(n) for n in lengths]) if len(lengths) else np.zeros(0, np.int64)
    qr = rope_apply(q, pos, base)
    kr = rope_apply(k, pos, base)
    m = dense_mask(lengths)
    out = np.empty((t, hq, d))
    lse = np.empty((hq, t))
    for h in range(hq):
        g = kv_head_of(h, group)
        s = (qr[:, h] @ kr[:, g].T) * scale + m
        p, l = _softmax_rows(s)
        out[:, h] = p @ v[:, g]
        lse[h] = l
    return out, lse


def sequence_probs(q, k, lengths, scale: float, base: float, seq: int, h: int) -> np.ndarray:
    """P for one sequence and query head (exposed so tests can check its rows)."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    group = q.shape[1] // k.shape[1]
    meta, qr, kr = _prepare(q, k, lengths, base)
    a, b = int(meta["cu_seqlens"][seq]), int(meta["cu_seqlens"][seq + 1])
    p, _ = _sequence_probs(qr[a:b, h], kr[a:b, kv_head_of(h, group)], scale)
    return p


# ----------------------------------------------------------------------------------------------
# Kept pairs of the mask (the expected total of the materialised keep pattern)
# ----------------------------------------------------------------------------------------------
def unmasked_pairs(lengths) -> int:
    """Number of (query, key) pairs the mask keeps: a sequence of n tokens keeps, for its query at
    position p, the p + 1 keys at positions 0..p, so it contributes n(n+1)/2."""
    return int(sum(int(n) * (int(n) + 1) // 2 for n in lengths))
