"""Host logic of the benchmark (CPU only): its FLOP and byte counts against closed forms and the
seed-0 figures of the packs, the traffic-profile reader, the uncached cost-model summary and the
one-GPU guard."""
import os
import subprocess
import sys

import pytest

import bench
from packed_sequence_causal_pk_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_flop_counts_match_kept_pairs():
    # kept pairs of a pack of lengths n: sum n(n+1)/2; forward 4 hq d P, backward 10 hq d P
    f, b = bench.attn_flops([3, 1], 2, 8)
    assert (f, b) == (4 * 2 * 8 * 7, 10 * 2 * 8 * 7)
    # the Qwen3-14B-shaped pack: P = 19,425,559 (seed 0), 40 heads, d = 128
    f, b = bench.attn_flops(synth.pack_lengths("qwen14b"), 40, 128)
    assert f == 4 * 40 * 128 * 19425559 and b == 10 * 40 * 128 * 19425559


def test_compulsory_bytes_closed_form():
    w = synth.WORKLOADS["qwen14b"]
    t = w.total_tokens
    q = t * w.hq * w.head_dim
    kv = t * w.hkv * w.head_dim
    fwd = 2 * (q + 2 * kv) + 2 * q + 4 * t * w.hq                      # read q, k, v; write out, lse
    bwd = 2 * (q + 2 * kv) + 2 * 2 * q + 4 * t * w.hq + 4 * (q + 2 * kv)   # + out, dout, lse; fp32 grads
    assert bench.min_bytes(w, t) == fwd + bwd


def test_traffic_profile_digest_and_parse():
    value = bench.measured_traffic()
    text = open(bench.TRAFFIC_PROFILE).read()
    line = [l for l in text.splitlines() if l.startswith("machine:")][0]
    fields = dict(kv.split("=") for kv in line.split()[1:])
    if fields["source_digest"] == bench.kernel_source_digest():
        assert value == int(fields["fetch_bytes_per_launch"]) + int(fields["write_bytes_per_launch"])
    else:
        assert value is None


def test_uncached_summary_cost_model():
    m = {"L": 16, "step_ms": 2.0,
         "uncached_step_ms": {"meta": {"step_ms": 3.5, "rebuild_ms": 0.05},
                              "meta_mask_sync": {"step_ms": 5.0, "rebuild_ms": 0.1}}}
    s = bench.uncached_summary(m)
    assert s["rebuilds_per_uncached_step"] == 32
    assert s["meta"]["saved_ms_per_step"] == pytest.approx(1.5)
    assert s["meta"]["predicted_saved_ms"] == pytest.approx(31 * 0.05)
    assert s["meta_mask_sync"]["predicted_saved_ms"] == pytest.approx(3.1)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr
