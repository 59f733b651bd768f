#!/usr/bin/env python3
"""Packed causal attention fwd+bwd benchmark on one MI355X.

One step = one pass of the whole path over one synthetic pack: build the packed metadata once,
then the forward of every layer, then the backward of every layer (the layer loop of a training
step), all on one stream with no host synchronisation inside the step.  Default workload: the
Qwen3-14B-shaped pack (16384 tokens, 40/8 heads, d=128, 40 layers).

Prints ONE JSON line.  `value` is algorithmic fwd+bwd TFLOP/s over the timed steps
(4*hq*d*P + 10*hq*d*P per layer, P = kept query/key pairs), `roofline` reports the dominant
kernel (the backward) against the chip's dense 16-bit matrix peak, timed per launch with HIP
events recorded by the library on its stream, and `cpu_baseline` times the float64 CPU oracle on
a bounded sample of the same workload.  `other_workloads` adds short runs of the other seeded
packs with their arithmetic intensity and the fraction of the attainable roofline
min(peak, intensity x HBM bandwidth) they reach; on the 16- and 28-layer packs it also runs the
step uncached (B rebuilt for every layer call, alone and with the materialised mask and a
host-visible sync) against the cost model T_saved ~ (n - 1) s.  `steps_around` times the
materialised mask, the standalone RoPE and the MoE grouping kernels, and the backward layer
loop with activations reloaded from pinned host memory, single- and double-buffered.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload qwen14b] [--no-cpu-baseline]
                    [--no-sweep]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "packed causal attn fwd+bwd TFLOP/s + tokens/s per layer; % bf16 MFMA peak"
PEAK_TFLOPS = 2516.6   # MI355X dense bf16/fp16 matrix peak (256 CUs x 4096 flop/clk x 2.4 GHz)
# v_mfma_f32_32x32x16_f16 rate, measured by pk_peak_mfma at the start of each run (the value
# here is only a placeholder until then)
MEASURED_MFMA_TFLOPS = 2200.0
HBM_GBS = 8000.0


def parse():
    p = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="qwen14b")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--steps-around-only", action="store_true",
                   help="time only the mask, RoPE, MoE-grouping and reload steps; print their JSON")
    p.add_argument("--no-sweep", action="store_true",
                   help="skip the short runs of the other packs reported under other_workloads")
    p.add_argument("--cpu-target-s", type=float, default=15.0,
                   help="approximate CPU seconds for the oracle sample")
    p.add_argument("--calibrate-copy-mib", type=int, default=0,
                   help="run a plain device copy of this many MiB before warmup (HBM counter "
                        "calibration under rocprofv3 --pmc)")
    return p.parse_args()


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "k_attn_bwd_kv_qwen14b_hbm_traffic.md")
KERNEL_SOURCES = [os.path.join(ROOT, "packed_sequence_causal_pk_amd", "csrc", f)
                  for f in ("pk_bwd_kv.hip", "pk_bwd.h", "pk_device.h")]


def kernel_source_digest():
    """Digest of the dK/dV kernel's sources and of the compiler flags its object is built with."""
    import hashlib
    from packed_sequence_causal_pk_amd import build
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    flags = build.COMMON_FLAGS + build.SOURCE_FLAGS.get("pk_bwd_kv.hip", [])
    h.update(" ".join(flags).encode())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch of the dK/dV kernel from the committed rocprofv3 counter summary,
    or None when the summary is missing or was taken on different kernel source."""
    try:
        text = open(TRAFFIC_PROFILE).read()
    except OSError:
        return None
    fields = {}
    for line in text.splitlines():
        if line.startswith("machine:"):
            for kv in line.split()[1:]:
                k, _, v = kv.partition("=")
                fields[k] = v
    if fields.get("source_digest") != kernel_source_digest():
        return None
    try:
        return int(fields["fetch_bytes_per_launch"]) + int(fields["write_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(w, lengths, target_s):
    """Time the float64 oracle (as it is) on whole sequences of layer 0, one KV-head group at a
    time (KV head 0 first), adding sequences shortest first until about target_s seconds."""
    import numpy as np
    from oracle import pk_oracle as O
    from packed_sequence_causal_pk_amd import synth

    q, k, v, do = synth.layer_tensors(w, 0)
    cu = np.concatenate([[0], np.cumsum(lengths)])
    order = np.argsort(lengths, kind="stable")
    done_flops, done_s, chosen = 0, 0.0, []
    for kvh in range(w.hkv):
        heads = [kvh * w.group + x for x in range(w.group)]
        for s in order:
            idx = np.arange(cu[s], cu[s + 1])
            n = len(idx)
            t0 = time.perf_counter()
            O.attn_fwd(q[idx], k[idx], v[idx], [n], w.softmax_scale, w.rope_base, heads=heads)
            O.attn_bwd(q[idx], k[idx], v[idx], do[idx], [n], w.softmax_scale, w.rope_base,
                       kv_heads=[kvh])
            done_s += time.perf_counter() - t0
            f, b = attn_flops([n], w.group, w.head_dim)
            done_flops += f + b
            chosen.append((kvh, int(n)))
            if done_s >= target_s:
                break
        if done_s >= target_s:
            break
    cores = len(os.sched_getaffinity(0))
    groups = sorted(set(c[0] for c in chosen))
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    rate = done_flops / done_s
    fl, bl = attn_flops(lengths, w.hq, w.head_dim)
    return {
        "value": rate / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
        "sample": "layer 0, KV heads %s each with its %d query heads, %d (KV head, sequence) "
                  "pairs of the pack (whole sequences, shortest first), fwd+bwd float64 numpy, "
                  "%.1f s; TFLOP/s counts the same algorithmic FLOPs as the GPU value"
                  % (groups, w.group, len(chosen), done_s),
        "seconds": round(done_s, 2),
        "cpu_model": model,
        "extrapolated_s_per_layer": round((fl + bl) / rate, 3),
        "extrapolated_s_per_step": round((fl + bl) * w.layers / rate, 3),
        "extrapolation": "the sample's FLOP rate applied to a whole layer and to the %d-layer step"
                         % w.layers,
    }


def attn_flops(lengths, hq, d):
    """Algorithmic FLOPs of one layer over the kept (query, key) pairs P = sum n(n+1)/2:
    forward 2 products (4 hq d P), backward 5 products (10 hq d P, S recomputed once)."""
    pairs = sum(int(n) * (int(n) + 1) // 2 for n in lengths)
    return 4 * hq * d * pairs, 10 * hq * d * pairs


def min_bytes(w, T):
    """Compulsory HBM bytes of one layer: forward reads q, k, v and writes out, lse; backward reads
    q, k, v, out, dout, lse and writes fp32 dq, dk, dv."""
    qkv = 2 * T * w.head_dim * (w.hq + 2 * w.hkv)
    fwd = qkv + 2 * T * w.hq * w.head_dim + 4 * T * w.hq
    bwd = qkv + 4 * T * w.hq * w.head_dim + 4 * T * w.hq + 4 * T * w.head_dim * (w.hq + 2 * w.hkv)
    return fwd + bwd


KINDS = ("meta", "fwd_prep", "fwd", "bwd_prep", "bwd", "bwd_dq")


def measure(name, steps, warmup, calibrate_mib=0, timed_kinds=(), uncached=False, graph=False,
            ds_compare=False):
    """Time `steps` steps (after `warmup`) of one workload, timing the kernel kinds
    `timed_kinds` inside that region; a second, shorter pass times every kind for the
    per-kernel breakdown.  Returns the timings and shapes."""
    import torch

    import packed_sequence_causal_pk_amd as pk
    from packed_sequence_causal_pk_amd import synth

    w = synth.WORKLOADS[name]
    lengths = synth.pack_lengths(name)
    T, L = w.total_tokens, w.layers
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    # inputs: independent seeded N(0,1) tensors per layer, rounded to bf16, resident in HBM
    gen = torch.Generator(device=dev)
    layers = []
    for l in range(L):
        gen.manual_seed(1000 + l)
        mk = lambda *shape: (torch.randn(*shape, generator=gen, device=dev) * w.input_scale).bfloat16()
        layers.append({"q": mk(T, w.hq, w.head_dim), "k": mk(T, w.hkv, w.head_dim),
                       "v": mk(T, w.hkv, w.head_dim), "do": mk(T, w.hq, w.head_dim),
                       "out": torch.empty(T, w.hq, w.head_dim, dtype=torch.bfloat16, device=dev),
                       "lse": torch.empty(w.hq, T, dtype=torch.float32, device=dev)})
    dq = torch.empty(T, w.hq, w.head_dim, dtype=torch.float32, device=dev)
    dk = torch.empty(T, w.hkv, w.head_dim, dtype=torch.float32, device=dev)
    dv = torch.empty(T, w.hkv, w.head_dim, dtype=torch.float32, device=dev)
    lengths_d = torch.tensor(lengths, dtype=torch.int32, device=dev)
    meta0 = pk.build_meta(lengths_d, T)
    ws_f = pk.fwd_workspace(meta0, w.hq, w.hkv, w.head_dim)
    # the backward recomputes S and dP for dQ (measured faster than the dS store on this part;
    # the store, sized from the pack's longest sequence, is timed beside it when ds_compare)
    ws_b = pk.bwd_workspace(meta0, w.hq, w.hkv, w.head_dim, store=False)
    meta0.close()
    if calibrate_mib > 0:
        nbytes = calibrate_mib << 20
        src = torch.ones(nbytes, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        print("bench: calibration copy of %d bytes done twice" % nbytes, file=sys.stderr, flush=True)
        del src, dst
    torch.cuda.synchronize()
    print("bench: %s, T=%d, %d layers, hq/hkv/d=%d/%d/%d" % (name, T, L, w.hq, w.hkv, w.head_dim),
          file=sys.stderr, flush=True)

    def step():
        meta = pk.build_meta(lengths_d, T)  # once per pack; every layer reuses it
        for x in layers:
            pk.attn_fwd(meta, x["q"], x["k"], x["v"], w.softmax_scale, w.rope_base,
                        out=x["out"], lse=x["lse"], workspace=ws_f)
        for x in reversed(layers):
            pk.attn_bwd(meta, x["q"], x["k"], x["v"], x["out"], x["lse"], x["do"], w.softmax_scale,
                        w.rope_base, dq=dq, dk=dk, dv=dv, workspace=ws_b)
        return meta

    mask_buf = torch.empty((T, T), dtype=torch.bool, device=dev) if uncached else None

    def rebuild(full):
        """The per-layer-call work an uncached path repeats: B itself, and with `full` also the
        materialised T x T mask and a host-visible read of max_seqlen (a device-to-host sync),
        the two costs the pages name for their unpatched path."""
        meta = pk.build_meta(lengths_d, T)
        if full:
            pk.dense_mask(meta, out=mask_buf)
            meta.check()
        return meta

    def step_uncached(full=False):
        # the same step with the metadata rebuilt for every layer call (no reuse across layers)
        metas = []
        for x in layers:
            metas.append(rebuild(full))
            pk.attn_fwd(metas[-1], x["q"], x["k"], x["v"], w.softmax_scale, w.rope_base,
                        out=x["out"], lse=x["lse"], workspace=ws_f)
        for x in reversed(layers):
            metas.append(rebuild(full))
            pk.attn_bwd(metas[-1], x["q"], x["k"], x["v"], x["out"], x["lse"], x["do"],
                        w.softmax_scale, w.rope_base, dq=dq, dk=dk, dv=dv, workspace=ws_b)
        return metas

    def rebuild_cost(full, n=50):
        """Wall-clock cost s of one rebuild on its own, ms (mean of n, synchronised at the end)."""
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        metas = [rebuild(full) for _ in range(n)]
        torch.cuda.synchronize()
        del metas
        return (time.perf_counter() - t0) * 1e3 / n

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    print("bench: %s warmup done" % name, file=sys.stderr, flush=True)

    def timed(n, kinds, fn=step):
        """n steps bracketed by events on the stream; the library times the given kernel kinds
        with its own event pairs (each pair costs a few microseconds, so only what is needed)."""
        pk.prof_reset()
        pk.prof_enable(bool(kinds), kinds=kinds or None)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        metas = [fn() for _ in range(n)]
        ev1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        pk.prof_enable(False)
        del metas
        kern = {}
        for kn in kinds:
            ms, cnt = pk.prof_query(kn)
            kern[kn] = {"total_ms": ms, "launches": cnt, "avg_us": 1000.0 * ms / max(cnt, 1)}
        return ev0.elapsed_time(ev1) / n, wall, kern

    # the timed region: whole-step time, plus the dominant kernel's own launches
    step_ms, wall, main_kern = timed(steps, timed_kinds)
    print("bench: %s timed %d steps, %.2f ms/step (wall %.2f s)" % (name, steps, step_ms, wall),
          file=sys.stderr, flush=True)
    # a second pass times every kernel kind (for the per-kernel breakdown only)
    nb = max(2, steps // 2)
    bd_ms, _, kern = timed(nb, list(KINDS))
    graph_ms = None
    if graph:
        # the whole step captured once into a HIP graph and replayed (launch-bound small packs)
        cap = torch.cuda.Stream(device=dev)
        cap.wait_stream(stream)
        with torch.cuda.stream(cap):
            step()
        stream.wait_stream(cap)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        for _ in range(2):
            g.replay()
        graph_ms = timed(steps, (), fn=g.replay)[0]
        del g
    ds_store = None
    if ds_compare:
        # the backward layer loop with the dS store against the recomputing dQ, alternating,
        # same inputs and process: per-layer kernel times and wall time
        meta_c = pk.build_meta(lengths_d, T)
        ws_s = pk.bwd_workspace(meta_c, w.hq, w.hkv, w.head_dim, max_seqlen=int(max(lengths)))
        for x in layers:
            pk.attn_fwd(meta_c, x["q"], x["k"], x["v"], w.softmax_scale, w.rope_base,
                        out=x["out"], lse=x["lse"], workspace=ws_f)

        def bwd_loop(ws):
            def run():
                for x in reversed(layers):
                    pk.attn_bwd(meta_c, x["q"], x["k"], x["v"], x["out"], x["lse"], x["do"],
                                w.softmax_scale, w.rope_base, dq=dq, dk=dk, dv=dv, workspace=ws)
                return meta_c
            return run

        ds_store = {"store_bytes": int(ws_s.numel()), "plain_bytes": int(ws_b.numel())}
        res = {"recompute": [], "store": []}
        for rep in range(2):
            for key, ws in (("recompute", ws_b), ("store", ws_s)):
                ms, _, kk = timed(1, ["bwd", "bwd_dq"], fn=bwd_loop(ws))
                res[key].append((ms / L, kk["bwd"]["avg_us"], kk["bwd_dq"]["avg_us"]))
        for key, vals in res.items():
            ds_store[key] = {"bwd_loop_us_per_layer": round(1000.0 * min(v[0] for v in vals), 1),
                             "dkdv_us": round(min(v[1] for v in vals), 1),
                             "dq_us": round(min(v[2] for v in vals), 1)}
        del ws_s, meta_c
    uncached_ms = None
    if uncached:
        uncached_ms = {}
        for full in (False, True):
            fn = (lambda: step_uncached(True)) if full else step_uncached
            for _ in range(2):
                fn()
            key = "meta_mask_sync" if full else "meta"
            uncached_ms[key] = {"step_ms": timed(steps, (), fn=fn)[0],
                                "rebuild_ms": rebuild_cost(full)}
    del layers, dq, dk, dv, ws_f, ws_b, mask_buf
    torch.cuda.empty_cache()
    fwd_flops, bwd_flops = attn_flops(lengths, w.hq, w.head_dim)
    layer_ms = step_ms / L
    return {"w": w, "lengths": lengths, "T": T, "L": L, "steps": nb, "step_ms": step_ms,
            "ds_store": ds_store,
            "main_kern": main_kern, "uncached_step_ms": uncached_ms, "graph_step_ms": graph_ms,
            "layer_ms": layer_ms, "kern": kern, "fwd_flops": fwd_flops, "bwd_flops": bwd_flops,
            "tflops": (fwd_flops + bwd_flops) * L / (step_ms * 1e-3) / 1e12}


def summary(m):
    """Per-layer figures of one measured workload."""
    k, steps, L = m["kern"], m["steps"], m["L"]
    fwd_ms = (k["fwd_prep"]["total_ms"] + k["fwd"]["total_ms"]) / steps / L
    bwd_ms = (k["bwd_prep"]["total_ms"] + k["bwd"]["total_ms"] + k["bwd_dq"]["total_ms"]) / steps / L
    ai = (m["fwd_flops"] + m["bwd_flops"]) / min_bytes(m["w"], m["T"])
    attainable = min(PEAK_TFLOPS, ai * HBM_GBS / 1000.0)
    return {
        "tflops": round(m["tflops"], 2),
        "pct_bf16_peak": round(100.0 * m["tflops"] / PEAK_TFLOPS, 2),
        "pct_measured_mfma_peak": round(100.0 * m["tflops"] / MEASURED_MFMA_TFLOPS, 2),
        "tokens_per_s_per_layer": round(m["T"] / (m["layer_ms"] * 1e-3), 1),
        "ms_per_layer_fwd_bwd": round(m["layer_ms"], 4),
        "ms_per_layer_fwd": round(fwd_ms, 4),
        "fwd_tflops": round(m["fwd_flops"] / (fwd_ms * 1e-3) / 1e12, 2),
        "ms_per_layer_bwd": round(bwd_ms, 4),
        "bwd_tflops": round(m["bwd_flops"] / (bwd_ms * 1e-3) / 1e12, 2),
        "arithmetic_intensity_flop_per_byte": round(ai, 1),
        "attainable_tflops": round(attainable, 1),
        "frac_of_attainable": round(m["tflops"] / attainable, 4),
        **({} if m["uncached_step_ms"] is None else {"uncached": uncached_summary(m)}),
        **({} if m.get("graph_step_ms") is None else {
            "graph_ms_per_step": round(m["graph_step_ms"], 4),
            "graph_tflops": round((m["fwd_flops"] + m["bwd_flops"]) * m["L"] / (m["graph_step_ms"] * 1e-3) / 1e12, 2),
            "graph_note": "the same step captured once into a HIP graph and replayed"}),
    }


def uncached_summary(m):
    """Cached vs uncached steps against the pages' cost model T_saved ~ (n - 1) s, with n the
    rebuilds an uncached step makes (one per layer call: 2L here, forward and backward) and s
    the cost of one rebuild measured on its own."""
    n = 2 * m["L"]
    out = {"cached_ms_per_step": round(m["step_ms"], 4), "rebuilds_per_uncached_step": n}
    what = {"meta": "B rebuilt per layer call (this library's own build, no sync)",
            "meta_mask_sync": "B + materialised T x T mask + host-visible max_seqlen read per layer call"}
    for key, u in m["uncached_step_ms"].items():
        saved = u["step_ms"] - m["step_ms"]
        out[key] = {"what": what[key], "uncached_ms_per_step": round(u["step_ms"], 4),
                    "saved_ms_per_step": round(saved, 4), "rebuild_ms": round(u["rebuild_ms"], 4),
                    "predicted_saved_ms": round((n - 1) * u["rebuild_ms"], 4)}
    return out


def measure_reload(name="qwen06b", reps=3):
    """The backward layer loop with each layer's q, k, v, out and lse copied back from pinned host
    memory, single- and double-buffered through the library's reload pipeline, against the model
    T_single ~ L (c + g) and T_double ~ c + (L - 1) max(c, g) + g, with c the copy of one layer
    and g one layer's backward, each measured on its own."""
    import torch

    import packed_sequence_causal_pk_amd as pk
    from packed_sequence_causal_pk_amd import synth

    dev = torch.device("cuda:0")
    w = synth.WORKLOADS[name]
    lengths = synth.pack_lengths(name)
    T, L = w.total_tokens, w.layers
    meta = pk.build_meta(torch.tensor(lengths, dtype=torch.int32, device=dev), T)
    gen = torch.Generator(device=dev)
    acts, douts = [], []
    for l in range(L):
        gen.manual_seed(2000 + l)
        mk = lambda *shape: (torch.randn(*shape, generator=gen, device=dev) * w.input_scale).bfloat16()
        q, k, v = mk(T, w.hq, w.head_dim), mk(T, w.hkv, w.head_dim), mk(T, w.hkv, w.head_dim)
        out, lse = pk.attn_fwd(meta, q, k, v, w.softmax_scale, w.rope_base)
        host = []
        for x in (q, k, v, out, lse):
            h = torch.empty(x.shape, dtype=x.dtype, pin_memory=True)
            h.copy_(x)
            host.append(h)
        acts.append(host)
        douts.append(mk(T, w.hq, w.head_dim))
        del q, k, v, out, lse
    slots = [[torch.empty(a.shape, dtype=a.dtype, device=dev) for a in acts[0]] for _ in range(2)]
    dq = torch.empty(T, w.hq, w.head_dim, dtype=torch.float32, device=dev)
    dk = torch.empty(T, w.hkv, w.head_dim, dtype=torch.float32, device=dev)
    dv = torch.empty_like(dk)
    ws = pk.bwd_workspace(meta, w.hq, w.hkv, w.head_dim, store=False)
    pipe = pk.ReloadPipeline()
    layer_bytes = sum(a.numel() * a.element_size() for a in acts[0])

    def fetch(slot, l):
        for dst, src in zip(slots[slot], acts[l]):
            pipe.fetch(slot, dst, src)

    def bwd(slot, l):
        q, k, v, out, lse = slots[slot]
        pk.attn_bwd(meta, q, k, v, out, lse, douts[l], w.softmax_scale, w.rope_base,
                    dq=dq, dk=dk, dv=dv, workspace=ws)

    def loop(double):
        order = list(reversed(range(L)))
        if double:
            fetch(0, order[0])
        for i, l in enumerate(order):
            s = i % 2 if double else 0
            if not double:
                fetch(0, l)
            elif i + 1 < L:
                fetch(1 - s, order[i + 1])
            pipe.acquire(s)
            bwd(s, l)
            pipe.release(s)

    def wall_ms(fn, n):
        fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(n):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / n

    def copies_only():
        for l in range(L):
            fetch(l % 2, l)
            pipe.acquire(l % 2)
            pipe.release(l % 2)

    def compute_only():
        for l in range(L):
            bwd(0, l)

    def copies_beside_compute():
        # the L copies and the L backwards at once, with no ordering between them: how much
        # the copies slow down while the backward kernels run
        for l in range(L):
            fetch(l % 2, l)
        compute_only()

    c = wall_ms(copies_only, reps) / L
    g = wall_ms(compute_only, reps) / L
    single = wall_ms(lambda: loop(False), reps)
    double = wall_ms(lambda: loop(True), reps)
    beside = wall_ms(copies_beside_compute, reps)
    pipe.close()
    return {
        "workload": name, "layers": L, "reloaded_per_layer": "q, k, v, out (bf16), lse (fp32)",
        "bytes_per_layer": layer_bytes, "copy_ms_per_layer_c": round(c, 4),
        "h2d_GBps": round(layer_bytes / (c * 1e-3) / 1e9, 1), "bwd_ms_per_layer_g": round(g, 4),
        "single_ms": round(single, 3), "double_ms": round(double, 3),
        "model_single_ms": round(L * (c + g), 3),
        "model_double_ms": round(c + (L - 1) * max(c, g) + g, 3),
        "saved_ms": round(single - double, 3), "model_saved_ms": round((L - 1) * min(c, g), 3),
        "copies_beside_compute_ms": round(beside, 3),
        "copies_beside_compute_note": "all L copies and all L backwards issued at once with no "
                                      "ordering between them; against L c = %.3f ms alone" % (L * c),
        # the model again with the raw copy time (no per-layer event ordering): c_raw = that run / L
        "copy_ms_per_layer_raw": round(beside / L, 4),
        "model_single_raw_ms": round(L * (beside / L + g), 3),
        "model_double_raw_ms": round(beside / L + (L - 1) * max(beside / L, g) + g, 3),
    }


def measure_steps_around(pk_names=("llama1b", "qwen06b", "qwen14b")):
    """The steps around the attention path, each timed per launch with the library's HIP event
    pairs: the materialised mask and the standalone RoPE (HBM streams: GB/s against 8 TB/s), and
    the MoE grouping (a latency-bound pass), with the per-expert data-dependent query it replaces
    (one torch.where per expert, each sizing its output on the host) timed beside it."""
    import torch

    import packed_sequence_causal_pk_amd as pk
    from packed_sequence_causal_pk_amd import synth

    dev = torch.device("cuda:0")

    def kind_avg_us(kind, fn, n):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        pk.prof_reset()
        pk.prof_enable(True, kinds=[kind])
        for _ in range(n):
            fn()
        torch.cuda.synchronize()
        pk.prof_enable(False)
        ms, cnt = pk.prof_query(kind)
        return 1000.0 * ms / max(cnt, 1)

    res = {"dense_mask": {}, "rope_apply": {}, "moe_group": {}}
    for name in pk_names:
        w = synth.WORKLOADS[name]
        lengths = synth.pack_lengths(name)
        T = w.total_tokens
        meta = pk.build_meta(torch.tensor(lengths, dtype=torch.int32, device=dev), T)
        mask = torch.empty((T, T), dtype=torch.bool, device=dev)
        us = kind_avg_us("mask", lambda: pk.dense_mask(meta, out=mask), 20)
        nbytes = T * T
        res["dense_mask"][name] = {"T": T, "avg_us": round(us, 2), "bytes_written": nbytes,
                                   "GBps": round(nbytes / us / 1e3, 1),
                                   "frac_hbm": round(nbytes / us / 1e3 / HBM_GBS, 4)}
        del mask
        x = (torch.randn(T, w.hq, w.head_dim, device=dev) * w.input_scale).bfloat16()
        y = torch.empty_like(x)
        us = kind_avg_us("rope", lambda: pk.rope_apply(meta, x, w.rope_base, out=y), 20)
        nbytes = 2 * x.numel() * 2
        res["rope_apply"][name] = {"shape": [T, w.hq, w.head_dim], "avg_us": round(us, 2),
                                   "bytes": nbytes, "GBps": round(nbytes / us / 1e3, 1),
                                   "frac_hbm": round(nbytes / us / 1e3 / HBM_GBS, 4)}
        del x, y
    for name, (n_tok, n_exp, top_k) in sorted(synth.MOE_WORKLOADS.items()):
        idx = torch.tensor(synth.router_indices(n_tok, n_exp, top_k), device=dev)
        M = n_tok * top_k
        ws = pk.moe_workspace(M, n_exp, dev)
        us = kind_avg_us("moe", lambda: pk.moe_group(idx, n_exp, workspace=ws), 50)

        def per_expert_where():
            return [torch.where(idx == e)[0] for e in range(n_exp)]
        for _ in range(2):
            per_expert_where()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(5):
            per_expert_where()
        torch.cuda.synchronize()
        naive_us = (time.perf_counter() - t0) * 1e6 / 5
        res["moe_group"][name] = {
            "n_tokens": n_tok, "n_experts": n_exp, "top_k": top_k, "avg_us": round(us, 2),
            "assignments_per_s": round(M / (us * 1e-6), 1),
            "algorithmic_bytes": 12 * M + 8 * n_exp + 8, "bound": "latency (3 launches)",
            "per_expert_where_us": round(naive_us, 1),
            "speedup_vs_per_expert_where": round(naive_us / us, 1)}
    res["lora_qkv"] = {}
    for name in pk_names:
        w = synth.WORKLOADS[name]
        T, K, N, r = w.total_tokens, synth.PROJ_HIDDEN[name], (w.hq + 2 * w.hkv) * w.head_dim, 16
        x = torch.randn(T, K, device=dev).bfloat16()
        wt = (torch.randn(N, K, device=dev) / K ** 0.5).bfloat16()
        at = (torch.randn(r, K, device=dev) / K ** 0.5).bfloat16()
        bt = (torch.randn(N, r, device=dev) * (0.25 / r ** 0.5)).bfloat16()
        y = torch.empty(T, N, dtype=torch.bfloat16, device=dev)
        ws = pk.lora_workspace(T, K, N, r, dev)
        us = kind_avg_us("lora", lambda: pk.lora_qkv(x, wt, at, bt, 2.0, out=y, workspace=ws), 10)
        flops = 2 * T * K * N + 2 * T * K * r + 2 * T * r * N
        tf = flops / (us * 1e-6) / 1e12
        res["lora_qkv"][name] = {"T": T, "K": K, "N": N, "rank": r, "avg_us": round(us, 2),
                                 "tflops": round(tf, 1), "frac_bf16_peak": round(tf / PEAK_TFLOPS, 4)}
        del x, wt, at, bt, y, ws
    res["reload"] = measure_reload()
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: the path is a single-GPU kernel (see the design notes "
              "for how it would shard); --gpus %d is not supported" % args.gpus, file=sys.stderr)
        sys.exit(2)

    if args.steps_around_only:
        print(json.dumps({"steps_around": measure_steps_around()}), flush=True)
        return
    # the measured roofline of this device: matrix-core rate and HBM bandwidths
    import packed_sequence_causal_pk_amd as pk
    import torch
    torch.cuda.set_device(0)
    global MEASURED_MFMA_TFLOPS
    burst_mfma = pk.peak_mfma_tflops(iters=2000)   # about 0.3 ms per launch
    MEASURED_MFMA_TFLOPS = pk.peak_mfma_tflops()   # about 3 ms per launch: the sustained clock
    measured_hbm = pk.peak_hbm_gbps()
    print("bench: measured MFMA %.1f TFLOP/s, HBM %s GB/s" % (MEASURED_MFMA_TFLOPS, measured_hbm),
          file=sys.stderr, flush=True)
    # the dK/dV kernel dominates the step on every pack measured here: its launches are timed
    # inside the timed region for the roofline
    m = measure(args.workload, args.steps, args.warmup, args.calibrate_copy_mib, timed_kinds=("bwd",),
                ds_compare=not args.no_sweep)
    w, lengths, T, L, kern = m["w"], m["lengths"], m["T"], m["L"], m["kern"]
    s = summary(m)

    # algorithmic FLOPs of each attention kernel over the kept pairs P: the forward's 2 products;
    # the key-outer backward's S, dP, dV, dK (4 products); the query-outer backward's dQ product
    # (its recomputed S and dP are counted once already, in the key-outer kernel)
    unit = m["fwd_flops"] // 2
    algo = {"fwd": 2 * unit, "bwd": 4 * unit, "bwd_dq": unit}
    achieved = {k: algo[k] / (kern[k]["avg_us"] * 1e-6) / 1e12 for k in algo}
    dominant = "bwd"   # timed inside the timed region (m["main_kern"])
    dominant_tflops = algo[dominant] / (m["main_kern"][dominant]["avg_us"] * 1e-6) / 1e12
    kernel_names = {"fwd": "k_attn_fwd (forward)", "bwd": "k_attn_bwd_kv (backward dK, dV)",
                    "bwd_dq": "k_attn_bwd_q (backward dQ)"}
    result = {
        "metric": METRIC,
        "value": s["tflops"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(m["step_ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {
            "workload": args.workload, "description": w.description, "total_tokens": T,
            "n_seqs": int(len(lengths)), "hq": w.hq, "hkv": w.hkv, "head_dim": w.head_dim,
            "layers": L, "step": "build meta once + %d layer forwards + %d layer backwards" % (L, L),
            "io_dtypes": "q/k/v/out/dout bf16, lse/dq/dk/dv fp32",
        },
        "tokens_per_s_per_layer": s["tokens_per_s_per_layer"],
        "pct_bf16_peak": s["pct_bf16_peak"],
        "pct_measured_mfma_peak": s["pct_measured_mfma_peak"],
        "measured_roofline": {"mfma_fp16_tflops": round(MEASURED_MFMA_TFLOPS, 1),
                              "mfma_fp16_tflops_short_launch": round(burst_mfma, 1),
                              "hbm_gbps": measured_hbm,
                              "how": "pk_peak_mfma (8 workgroups of 4 waves per CU, 4 chains of "
                                     "v_mfma_f32_32x32x16_f16 per wave; 20000 iterations, 2000 for the "
                                     "short launch) and pk_peak_hbm (2 GiB read / write / copy), best of 3"},
        "ms_per_layer_fwd_bwd": s["ms_per_layer_fwd_bwd"],
        "ms_per_layer_fwd": s["ms_per_layer_fwd"],
        "fwd_tflops": s["fwd_tflops"],
        "ms_per_layer_bwd": s["ms_per_layer_bwd"],
        "bwd_tflops": s["bwd_tflops"],
        "build_meta_us": round(kern["meta"]["avg_us"], 2),
        "kernels_avg_us": {k: round(v["avg_us"], 2) for k, v in kern.items()},
        "kernels_avg_us_note": "from a second pass of %d steps that times every kernel kind" % m["steps"],
        "kernels_algorithmic_tflops": {k: round(v, 2) for k, v in achieved.items()},
        "roofline": {
            "kernel": kernel_names[dominant],
            "bound": "mfma", "achieved": round(dominant_tflops, 2), "peak": PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": round(dominant_tflops / PEAK_TFLOPS, 4),
            "avg_launch_us": round(m["main_kern"][dominant]["avg_us"], 2),
            "traffic": measured_traffic(),
        },
    }
    if m["ds_store"] is not None:
        result["bwd_ds_store_vs_recompute"] = dict(
            m["ds_store"], note="the backward layer loop of this workload with the dS store "
                                "(pk_attn_bwd_workspace_bytes_ds, sized from the longest sequence) "
                                "and with the recomputing dQ kernel (the step above), alternating in "
                                "one process; best of 2 passes each")
    if not args.no_sweep:
        # the other packs, a few steps each (their own figures; `value` is the workload above)
        other = {}
        for name in ("tiny", "llama1b", "qwen06b", "qwen14b", "skewed"):
            if name == args.workload:
                continue
            # 20 timed steps on the small packs, 5 on the large ones; the multi-layer small
            # packs also run with the metadata rebuilt per layer call (the uncached mode)
            small = name in ("tiny", "llama1b", "qwen06b")
            other[name] = summary(measure(name, 20 if small else 5, 3,
                                          uncached=name in ("llama1b", "qwen06b"), graph=small))
        result["other_workloads"] = other
        result["steps_around"] = measure_steps_around()
    if not args.no_cpu_baseline:
        print("bench: timing the CPU oracle sample", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(w, lengths, args.cpu_target_s)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
