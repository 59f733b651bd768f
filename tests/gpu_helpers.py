"""Shared pieces of the GPU tests: run the HIP path on numpy inputs, compare with the oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

import packed_sequence_causal_pk_amd as pk

# tolerance of the parity gate, per tensor against the float64 oracle
MAX_ABS = 2e-2
REL_L2 = 1e-2
LSE_MAX_ABS = 1e-2


def say(*args):
    print(*args, flush=True)
    sys.stdout.flush()


def dev(x, dtype=torch.bfloat16):
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda").to(dtype).contiguous()


def run_pk(lengths, q, k, v, dout, scale, base=10000.0, meta=None, bwd=True, store=False):
    """Build the meta (unless given) and run fwd (+ bwd) through libpk.  Without `store` the dQ
    kernel recomputes S and dP (the path the benchmark times); with it the backward's workspace
    includes the dS store, sized from the pack's longest sequence."""
    t = q.shape[0]
    if meta is None:
        lens = np.asarray(lengths, np.int32)
        meta = pk.build_meta(torch.tensor(lens, device="cuda"), t,
                             max_seqlen=int(lens.max()) if lens.size else 0)
    tq, tk, tv = dev(q), dev(k), dev(v)
    out, lse = pk.attn_fwd(meta, tq, tk, tv, scale, base)
    res = {"meta": meta, "out": out, "lse": lse}
    if bwd:
        tdo = dev(dout)
        hq, hkv, d = q.shape[1], k.shape[1], q.shape[2]
        ws = pk.bwd_workspace(meta, hq, hkv, d, store=store,
                              max_seqlen=None if meta.max_seqlen_bound is not None else t)
        dq, dk, dv = pk.attn_bwd(meta, tq, tk, tv, out, lse, tdo, scale, base, workspace=ws)
        res.update(dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return res


def to_np(x):
    return x.detach().float().cpu().numpy().astype(np.float64)


def compare(name, got, ref, max_abs=MAX_ABS, rel_l2=REL_L2, where=None):
    """Element-wise comparison on the entries the oracle computed (finite in `ref`)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    mask = np.isfinite(ref) if where is None else where
    assert mask.any(), name
    g, r = got[mask], ref[mask]
    assert np.all(np.isfinite(g)), "%s: non-finite values" % name
    diff = np.abs(g - r)
    ma = float(diff.max())
    rnorm = float(np.linalg.norm(r))
    # relative L2 is undefined against an all-zero reference (e.g. dQ of length-1 sequences);
    # there the max-abs gate alone applies
    rl = float(np.linalg.norm(diff) / rnorm) if rnorm > 0 else 0.0
    say("  %-6s max_abs %.3e  rel_l2 %s  (n=%d)" % (name, ma, "%.3e" % rl if rnorm > 0 else "n/a", g.size))
    assert ma <= max_abs, "%s max-abs %.4e > %.1e" % (name, ma, max_abs)
    assert rl <= rel_l2, "%s rel-L2 %.4e > %.1e" % (name, rl, rel_l2)
    return ma, rl


def meta_to_np(meta):
    v = meta.view()
    return {k: (x.cpu().numpy().astype(np.int64) if isinstance(x, torch.Tensor) else x) for k, x in v.items()}
