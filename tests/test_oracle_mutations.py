"""Plant plausible mistakes in the oracle (on the CPU) and check that some pin catches each one.

A pin set that lets any of these through would not be strong enough to trust the oracle."""
import numpy as np
import pytest

from oracle import lora_oracle as LO
from oracle import moe_oracle as MO
from oracle import pk_oracle as O
from tests import oracle_pins as P


def _run_all_pins():
    failures = []
    for pin in P.ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except (AssertionError, ValueError, FloatingPointError, IndexError) as e:
            failures.append(pin.__name__)
    return failures


def _interleaved_rope(x, pos, base, inverse=False):
    x = np.asarray(x, np.float64)
    d = x.shape[-1]
    th = O.rope_angles(pos, d, base)
    c, s = np.cos(th)[:, None, :], np.sin(th)[:, None, :]
    if inverse:
        s = -s
    out = np.empty_like(x)
    out[..., 0::2] = x[..., 0::2] * c - x[..., 1::2] * s
    out[..., 1::2] = x[..., 1::2] * c + x[..., 0::2] * s
    return out


_orig_rope = O.rope_apply
_orig_build = O.build_meta
_orig_softmax = O._softmax_rows


def _global_positions(lengths, total_tokens, tile_rows=O.TILE_ROWS):
    m = _orig_build(lengths, total_tokens, tile_rows)
    if "pos" in m:
        m["pos"] = np.arange(total_tokens)
    return m


def _cost_off_by_one(cu, seq_id, t, r=O.TILE_ROWS):
    f, b = _orig_work_lists(cu, seq_id, t, r)
    f[:, 3] -= 1  # forward keys stop one short of the tile's end
    return f, b


_orig_work_lists = O.work_lists
_orig_group = MO.group_by_expert


def _group_slot_major(idx, n_experts):
    """Mistake: assignments enumerated slot-major (a transposed operand) inside each group."""
    idx = np.asarray(idx)
    r = _orig_group(idx, n_experts)
    if r["status"] or idx.size == 0:
        return r
    n_tok, top_k = idx.shape
    perm = []
    for e in range(n_experts):
        s, t = np.nonzero(idx.T == e)
        perm += (t * top_k + s).tolist()
    r["perm"] = np.asarray(perm)
    r["inv"][r["perm"]] = np.arange(len(perm))
    return r


def _group_inclusive_offsets(idx, n_experts):
    """Mistake: offsets[e] taken as the end of group e instead of its start."""
    r = _orig_group(idx, n_experts)
    if not r["status"]:
        r["offsets"] = np.concatenate([np.cumsum(r["counts"]), [r["n_assign"]]])
    return r


def _group_descending(idx, n_experts):
    """Mistake: an unstable (reversed) order inside each group."""
    r = _orig_group(idx, n_experts)
    if not r["status"]:
        o = r["offsets"]
        r["perm"] = np.concatenate([r["perm"][o[e]:o[e + 1]][::-1] for e in range(n_experts)] or [r["perm"]])
        r["inv"][r["perm"]] = np.arange(r["perm"].shape[0])
    return r


def _mask_strict(lengths):
    """Mistake: the mask drops the diagonal."""
    m = _orig_dense_mask(lengths)
    np.fill_diagonal(m, -np.inf)
    return m


_orig_dense_mask = O.dense_mask
_orig_lora = LO.lora_qkv


def _lora_adapter_omitted(x, w, a, b, scale=1.0):
    """Mistake: the frozen weight alone (the adapter never added)."""
    return np.asarray(x, np.float64) @ np.asarray(w, np.float64)


def _lora_scale_dropped(x, w, a, b, scale=1.0):
    """Mistake: the adapter scale ignored."""
    return _orig_lora(x, w, a, b, 1.0)

_orig_probs = O._sequence_probs


def _probs_unscaled(qr, kr, scale):
    """Mistake: the softmax scale never applied to the scores."""
    return _orig_probs(qr, kr, 1.0)


def _probs_scale_squared(qr, kr, scale):
    """Mistake: 1/d where 1/sqrt(d) is meant (the scale applied twice)."""
    return _orig_probs(qr, kr, scale * scale)


def _meta_cu_inclusive(lengths, total_tokens, tile_rows=O.TILE_ROWS):
    """Mistake: cu_seqlens as an inclusive scan (no leading zero, the total repeated)."""
    m = _orig_build(lengths, total_tokens, tile_rows)
    cu = m["cu_seqlens"]
    if cu.shape[0] > 1:
        m["cu_seqlens"] = np.concatenate([cu[1:], cu[-1:]])
    return m


def _meta_max_is_sum(lengths, total_tokens, tile_rows=O.TILE_ROWS):
    """Mistake: max_seqlen taken as the total token count."""
    m = _orig_build(lengths, total_tokens, tile_rows)
    m["max_seqlen"] = int(np.sum(np.asarray(lengths, np.int64)))
    return m


_orig_score_grad = O.score_grad


def _ds_floor(bwd, t, r, br):
    """Mistake: a tile's partial last query block not counted."""
    n = -(-t // r)
    blocks = np.zeros(n, dtype=np.int64)
    for item in bwd:
        blocks[int(item[7])] = (int(item[3]) - int(item[2])) // br
    return np.concatenate([[0], np.cumsum(blocks)])


def _work_lists_ties_reversed(cu, seq_id, t, r=O.TILE_ROWS):
    """Mistake: equal-cost items ordered by descending tile index (not a stable order)."""
    f, b = _orig_work_lists(cu, seq_id, t, r)
    def reorder(x):
        return x[sorted(range(x.shape[0]), key=lambda i: (-x[i, 6], -x[i, 7]))]
    return reorder(f), reorder(b)


MUTATIONS = {
    "softmax_scale_missing": ("_sequence_probs", _probs_unscaled),
    "softmax_scale_squared": ("_sequence_probs", _probs_scale_squared),
    "cu_seqlens_inclusive": ("build_meta", _meta_cu_inclusive),
    "max_seqlen_is_total": ("build_meta", _meta_max_is_sum),
    "worklist_ties_reversed": ("work_lists", _work_lists_ties_reversed),
    "gqa_interleaved_groups": ("kv_head_of", lambda h, g: h % g),
    "mask_excludes_diagonal": ("causal_keep", lambda n: np.tril(np.ones((n, n), bool), -1)),
    "mask_not_causal": ("causal_keep", lambda n: np.ones((n, n), bool)),
    "rope_reversed_angle": ("rope_angles", lambda pos, d, base: -(np.asarray(pos, float)[:, None]
                             * np.power(float(base), -2.0 * np.arange(d // 2) / d)[None, :])),
    "rope_wrong_frequency": ("rope_angles", lambda pos, d, base: np.asarray(pos, float)[:, None]
                             * np.power(float(base), -1.0 * np.arange(d // 2) / d)[None, :]),
    "rope_interleaved_pairs": ("rope_apply", _interleaved_rope),
    "rope_backward_not_transposed": ("rope_apply", lambda x, pos, base, inverse=False: _orig_rope(x, pos, base)),
    "positions_not_reset": ("build_meta", _global_positions),
    "lse_without_max": ("_softmax_rows", lambda s: (_orig_softmax(s)[0], np.log(np.exp(s - s.max(1)[:, None]).sum(1)))),
    "dS_dropped_D": ("score_grad", lambda p, do, v, o=None: p * (do @ v.T)),
    "dS_sign": ("score_grad", lambda p, do, v, o=None: p * (np.sum(do * (p @ v), 1)[:, None] - do @ v.T)),
    "dS_given_output_ignored": ("score_grad", lambda p, do, v, o=None: _orig_score_grad(p, do, v)),
    "dQ_missing_scale": ("query_grad", lambda ds, kr, scale: ds @ kr),
    "dK_transposed_operand": ("key_grad", lambda ds, qr, scale: scale * (ds @ qr)),
    "worklist_short_range": ("work_lists", _cost_off_by_one),
    "dense_mask_strict": ("dense_mask", _mask_strict),
    "ds_blocks_floor": ("ds_block_offsets", lambda b, t, r=O.TILE_ROWS, br=O.DS_BLOCK_ROWS: _ds_floor(b, t, r, br)),
    "kept_pairs_strict": ("unmasked_pairs", lambda lengths: int(sum(int(n) * (int(n) - 1) // 2 for n in lengths))),
    "moe_slot_major": (MO, "group_by_expert", _group_slot_major),
    "moe_inclusive_offsets": (MO, "group_by_expert", _group_inclusive_offsets),
    "moe_unstable_order": (MO, "group_by_expert", _group_descending),
    "lora_adapter_omitted": (LO, "lora_qkv", _lora_adapter_omitted),
    "lora_scale_dropped": (LO, "lora_qkv", _lora_scale_dropped),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    spec = MUTATIONS[name]
    mod, attr, fn = spec if len(spec) == 3 else (O,) + spec
    monkeypatch.setattr(mod, attr, fn)
    failures = _run_all_pins()
    assert failures, "mutation %s passed every pin" % name


def test_unmutated_oracle_passes_all_pins():
    assert _run_all_pins() == []
