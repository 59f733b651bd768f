"""Seeded pack generator (host logic, CPU only)."""
import numpy as np
import torch

from packed_sequence_causal_pk_amd import synth


def test_pack_lengths_seed0():
    assert synth.pack_lengths("tiny").tolist() == [37, 100, 5, 114]
    assert synth.pack_lengths("llama1b").tolist() == [445, 349, 293, 185, 202, 82, 97, 71, 142, 182]
    assert synth.pack_lengths("qwen14b").tolist() == [3523, 2702, 2219, 1292, 1438, 413, 544, 319, 929, 3005]
    q = synth.pack_lengths("qwen06b")
    assert len(q) == 25 and q.max() == 895 and q.min() == 47
    s = synth.pack_lengths("skewed")
    assert s[:4].tolist() == [8192] * 4 and len(s) == 3814 and int((s == 1).sum()) == 249
    for name in synth.WORKLOAD_ORDER:
        w = synth.WORKLOADS[name]
        lens = synth.pack_lengths(name)
        assert int(lens.sum()) == w.total_tokens and lens.min() >= 1


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(100000) * np.exp(rng.uniform(-20, 20, 100000))).astype(np.float32)
    x[:4] = [0.0, -0.0, np.inf, -np.inf]
    ours = synth.bf16_round(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    assert np.array_equal(ours.view(np.uint32), ref.view(np.uint32))
    assert np.array_equal(torch.from_numpy(ours).bfloat16().float().numpy(), ours)


def test_layer_tensors_shapes_and_seeding():
    w = synth.WORKLOADS["tiny"]
    q, k, v, do = synth.layer_tensors(w, 0)
    assert q.shape == (256, 2, 64) and k.shape == (256, 1, 64) and do.shape == q.shape
    q2 = synth.layer_tensors(w, 0)[0]
    assert np.array_equal(q, q2)
    assert not np.array_equal(q, synth.layer_tensors(w, 1)[0])
    assert abs(float(q.std()) - 1.0) < 0.05
    w14 = synth.WORKLOADS["qwen14b"]
    assert abs(float(synth.layer_tensors(w14, 0, total_tokens=512)[2].std()) - 0.5) < 0.03


def test_router_indices_shape_distinct_and_seeded():
    """The synthetic router gives each token top_k distinct experts in range, is reproducible for a
    seed, and spreads load unevenly (the per-expert offset) without leaving most experts idle."""
    for (n_tok, n_exp, top_k) in synth.MOE_WORKLOADS.values():
        idx = synth.router_indices(n_tok, n_exp, top_k)
        assert idx.shape == (n_tok, top_k) and idx.dtype == np.int32
        assert idx.min() >= 0 and idx.max() < n_exp
        assert all(len(set(row)) == top_k for row in idx[:2000].tolist())
        assert np.array_equal(idx, synth.router_indices(n_tok, n_exp, top_k))
        counts = np.bincount(idx.ravel(), minlength=n_exp)
        assert counts.max() > 2 * counts.mean() and (counts > 0).sum() > n_exp // 2
