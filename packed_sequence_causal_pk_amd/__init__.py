"""Packed-sequence causal attention for MI355X: Python binding of libpk.so.

Argument marshalling only: every step of the attention path runs in the library's HIP kernels.
PyTorch supplies device memory and the current stream.

    meta = build_meta(lengths_int32_cuda, total_tokens)           # once per pack
    out, lse = attn_fwd(meta, q, k, v)                              # every layer
    dq, dk, dv = attn_bwd(meta, q, k, v, out, lse, dout)            # every layer
"""
from __future__ import annotations

import ctypes
import math
from typing import Optional, Tuple

from . import _lib
from ._lib import PkError, lib

__all__ = ["PackedMeta", "build_meta", "attn_fwd", "attn_bwd", "fwd_workspace", "bwd_workspace",
           "PackedCausalAttention", "PkError", "tile_rows", "prof_enable", "prof_reset",
           "prof_query", "dense_mask", "rope_apply", "moe_group", "moe_workspace",
           "ReloadPipeline", "peak_mfma_tflops", "peak_hbm_gbps", "lora_qkv", "lora_workspace",
           "attn_bwd_prep", "attn_bwd_main", "attn_fwd_noalloc"]


def _torch():
    import torch
    return torch


def _stream_ptr(stream) -> ctypes.c_void_p:
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t) -> ctypes.c_void_p:
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def tile_rows() -> int:
    return int(lib().pk_tile_rows())


class PackedMeta:
    """B for one pack: a libpk handle plus the device buffer it lives in (kept alive here)."""

    def __init__(self, handle: ctypes.c_void_p, buf, lengths, total_tokens: int, n_seqs: int,
                 max_seqlen: Optional[int] = None):
        self._handle = handle
        self.buf = buf
        self.lengths = lengths
        self.total_tokens = total_tokens
        self.n_seqs = n_seqs
        self.device = buf.device
        # host-side bound on the longest sequence (the caller's packer knows it), used to size
        # the backward's dS store; None: no store unless a bound is given to bwd_workspace
        self.max_seqlen_bound = max_seqlen

    @property
    def handle(self) -> ctypes.c_void_p:
        if self._handle is None:
            raise RuntimeError("meta already destroyed")
        return self._handle

    def view(self) -> dict:
        """Device tensors aliasing B: cu_seqlens, max_seqlen, status, seq_id, pos, fwd/bwd items."""
        torch = _torch()
        v = _lib.MetaView()
        _lib.check("pk_meta_view", lib().pk_meta_view(self.handle, ctypes.byref(v)))
        base = self.buf.data_ptr()
        as32 = self.buf.view(torch.int32)

        def sl(ptr, n):
            off = (ptr - base) // 4
            return as32[off:off + n]

        return {
            "cu_seqlens": sl(v.cu_seqlens, v.n_seqs + 1),
            "max_seqlen": sl(v.max_seqlen, 1),
            "status": sl(v.status, 1),
            "seq_id": sl(v.seq_id, v.total_tokens),
            "pos": sl(v.pos, v.total_tokens),
            "fwd_items": sl(v.fwd_items, v.n_items * 8).view(v.n_items, 8),
            "bwd_items": sl(v.bwd_items, v.n_items * 8).view(v.n_items, 8),
            "n_items": v.n_items,
            "ds_off": sl(v.ds_off, v.n_items + 1),
        }

    def check(self, stream=None) -> Tuple[int, int]:
        """(status word, max_seqlen).  SYNCHRONISES the stream: debugging and tests only."""
        st, mx = ctypes.c_int32(0), ctypes.c_int32(0)
        rc = lib().pk_meta_check(self.handle, _stream_ptr(stream), ctypes.byref(st), ctypes.byref(mx))
        if rc not in (_lib.PK_OK, _lib.PK_ERR_DEVICE):
            _lib.check("pk_meta_check", rc)
        return int(st.value), int(mx.value)

    def close(self) -> None:
        if self._handle is not None:
            lib().pk_meta_destroy(self._handle)
            self._handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def build_meta(lengths, total_tokens: Optional[int] = None, stream=None,
               max_seqlen: Optional[int] = None) -> PackedMeta:
    """Build B on the device from int32 `lengths` (a CUDA tensor).  `total_tokens` is T, the
    token count of the pack as the caller's q/k/v hold it (never read back from the device).
    `max_seqlen`, when the caller knows it, is a host-side bound on the longest sequence that
    the backward uses to size its dS store (a wrong bound is safe: the device then falls back to
    recomputing)."""
    torch = _torch()
    if lengths.dtype != torch.int32 or not lengths.is_cuda or lengths.dim() != 1:
        raise ValueError("lengths must be a 1-D int32 CUDA tensor")
    lengths = lengths.contiguous()
    n = int(lengths.numel())
    if total_tokens is None:
        raise ValueError("total_tokens must be given (it is host-known: q.shape[0])")
    nbytes = int(lib().pk_meta_bytes(n, int(total_tokens)))
    if nbytes == 0:
        raise PkError("pk_meta_bytes", _lib.PK_ERR_INVALID)
    buf = torch.empty(nbytes, dtype=torch.uint8, device=lengths.device)
    h = ctypes.c_void_p()
    rc = lib().pk_build_meta(_ptr(lengths), n, int(total_tokens), _ptr(buf), nbytes,
                             _stream_ptr(stream), ctypes.byref(h))
    _lib.check("pk_build_meta", rc)
    return PackedMeta(h, buf, lengths, int(total_tokens), n,
                      None if max_seqlen is None else int(max_seqlen))


def _dims(q, k):
    t, hq, d = q.shape
    return int(t), int(hq), int(k.shape[1]), int(d)


def fwd_workspace(meta: PackedMeta, hq: int, hkv: int, d: int):
    torch = _torch()
    n = int(lib().pk_attn_fwd_workspace_bytes(meta.handle, hq, hkv, d))
    return torch.empty(max(n, 256), dtype=torch.uint8, device=meta.device)


def bwd_workspace(meta: PackedMeta, hq: int, hkv: int, d: int, store: bool = True,
                  max_seqlen: Optional[int] = None):
    """Backward workspace; with `store` and a max_seqlen bound (given here, or the meta's), it
    includes the dS store sized by pk_attn_bwd_workspace_bytes_ds."""
    torch = _torch()
    bound = meta.max_seqlen_bound if max_seqlen is None else max_seqlen
    if store and bound is not None:
        n = int(lib().pk_attn_bwd_workspace_bytes_ds(meta.handle, hq, hkv, d, int(bound)))
    else:
        n = int(lib().pk_attn_bwd_workspace_bytes(meta.handle, hq, hkv, d))
    return torch.empty(max(n, 256), dtype=torch.uint8, device=meta.device)


def _check_inputs(meta, *tensors):
    torch = _torch()
    for t in tensors:
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("tensors must be contiguous CUDA tensors")
        if t.device != meta.device:
            raise ValueError("tensor on %s, meta on %s" % (t.device, meta.device))


def _check_out(name, t, shape, dtype, device):
    """A caller-supplied output: exactly the shape, dtype and device the call writes, contiguous
    (the library writes through the raw pointer, so nothing else may be passed)."""
    if (t.dtype != dtype or tuple(t.shape) != tuple(int(x) for x in shape) or not t.is_contiguous()
            or t.device != device):
        raise ValueError("%s must be a contiguous %s tensor of shape %s on %s"
                         % (name, dtype, tuple(shape), device))


def _ws_bytes(ws, device) -> int:
    """Byte size of a caller-supplied workspace (any dtype; contiguous, on the call's device)."""
    if not ws.is_cuda or not ws.is_contiguous() or ws.device != device:
        raise ValueError("workspace must be a contiguous tensor on %s" % device)
    return int(ws.numel()) * int(ws.element_size())


def attn_fwd(meta: PackedMeta, q, k, v, softmax_scale: Optional[float] = None,
             rope_base: float = 10000.0, out=None, lse=None, workspace=None, stream=None):
    """(out bf16 [T,hq,d], lse float32 [hq,T]) for bf16 q [T,hq,d], k, v [T,hkv,d]."""
    torch = _torch()
    t, hq, hkv, d = _dims(q, k)
    _check_inputs(meta, q, k, v)
    if q.dtype != torch.bfloat16 or k.dtype != torch.bfloat16 or v.dtype != torch.bfloat16:
        raise ValueError("q, k, v must be bfloat16")
    if t != meta.total_tokens or k.shape != v.shape or k.shape[0] != t or k.shape[2] != d:
        raise ValueError("shape mismatch with the pack")
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((hq, t), dtype=torch.float32, device=q.device) if lse is None else lse
    _check_out("out", out, q.shape, torch.bfloat16, q.device)
    _check_out("lse", lse, (hq, t), torch.float32, q.device)
    ws = fwd_workspace(meta, hq, hkv, d) if workspace is None else workspace
    rc = lib().pk_attn_fwd(meta.handle, _ptr(q), _ptr(k), _ptr(v), hq, hkv, d, scale,
                           float(rope_base), _ptr(out), _ptr(lse), _ptr(ws), _ws_bytes(ws, q.device),
                           _stream_ptr(stream))
    _lib.check("pk_attn_fwd", rc)
    return out, lse


def attn_fwd_noalloc(meta: PackedMeta, q, k, v, out, lse, softmax_scale: Optional[float] = None,
                     rope_base: float = 10000.0, stream=None):
    """pk_attn_fwd_noalloc: the forward with the library's fixed per-device workspace, for
    callers that cannot allocate; out (bf16 [T,hq,d]) and lse (float32 [hq,T]) are the caller's
    and nothing is allocated here either.  Calls that overlap on one device race."""
    torch = _torch()
    t, hq, hkv, d = _dims(q, k)
    _check_inputs(meta, q, k, v)
    if q.dtype != torch.bfloat16 or k.dtype != torch.bfloat16 or v.dtype != torch.bfloat16:
        raise ValueError("q, k, v must be bfloat16")
    if t != meta.total_tokens or k.shape != v.shape or k.shape[0] != t or k.shape[2] != d:
        raise ValueError("shape mismatch with the pack")
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    _check_out("out", out, q.shape, torch.bfloat16, q.device)
    _check_out("lse", lse, (hq, t), torch.float32, q.device)
    rc = lib().pk_attn_fwd_noalloc(meta.handle, _ptr(q), _ptr(k), _ptr(v), hq, hkv, d, scale,
                                   float(rope_base), _ptr(out), _ptr(lse), _stream_ptr(stream))
    _lib.check("pk_attn_fwd_noalloc", rc)
    return out, lse


def _check_bwd_inputs(q, k, v, out, lse, dout, t, hq, d):
    torch = _torch()
    for name, x in (("q", q), ("k", k), ("v", v), ("out", out), ("dout", dout)):
        if x.dtype != torch.bfloat16:
            raise ValueError("%s must be bfloat16" % name)
    if k.shape != v.shape or k.dim() != 3 or k.shape[0] != t or k.shape[2] != d:
        raise ValueError("k and v must be [T, hkv, d] like each other")
    _check_out("lse", lse, (hq, t), torch.float32, q.device)


def _check_grads(dq, dk, dv, q, k):
    torch = _torch()
    _check_out("dq", dq, q.shape, torch.float32, q.device)
    _check_out("dk", dk, k.shape, torch.float32, q.device)
    _check_out("dv", dv, k.shape, torch.float32, q.device)


def attn_bwd(meta: PackedMeta, q, k, v, out, lse, dout, softmax_scale: Optional[float] = None,
             rope_base: float = 10000.0, dq=None, dk=None, dv=None, workspace=None, stream=None):
    """(dq, dk, dv) float32 for the loss sum(out * dout)."""
    torch = _torch()
    t, hq, hkv, d = _dims(q, k)
    _check_inputs(meta, q, k, v, out, lse, dout)
    if t != meta.total_tokens or out.shape != q.shape or dout.shape != q.shape:
        raise ValueError("shape mismatch with the pack")
    _check_bwd_inputs(q, k, v, out, lse, dout, t, hq, d)
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    dq = torch.empty(q.shape, dtype=torch.float32, device=q.device) if dq is None else dq
    dk = torch.empty(k.shape, dtype=torch.float32, device=q.device) if dk is None else dk
    dv = torch.empty(v.shape, dtype=torch.float32, device=q.device) if dv is None else dv
    _check_grads(dq, dk, dv, q, k)
    ws = bwd_workspace(meta, hq, hkv, d) if workspace is None else workspace
    rc = lib().pk_attn_bwd(meta.handle, _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(dout),
                           hq, hkv, d, scale, float(rope_base), _ptr(dq), _ptr(dk), _ptr(dv),
                           _ptr(ws), _ws_bytes(ws, q.device), _stream_ptr(stream))
    _lib.check("pk_attn_bwd", rc)
    return dq, dk, dv


def dense_mask(meta: PackedMeta, out=None, stream=None):
    """The pack's T x T keep pattern as a torch.bool tensor (True: key visible to query), the
    materialised structure the pages' uncached path rebuilds per layer."""
    torch = _torch()
    t = meta.total_tokens
    out = torch.empty((t, t), dtype=torch.bool, device=meta.device) if out is None else out
    _check_out("out", out, (t, t), torch.bool, meta.device)
    rc = lib().pk_dense_mask(meta.handle, _ptr(out), out.numel(), _stream_ptr(stream))
    _lib.check("pk_dense_mask", rc)
    return out


def rope_apply(meta: PackedMeta, x, rope_base: float = 10000.0, inverse: bool = False, out=None,
               stream=None):
    """Rotate-half RoPE of bf16 x [T, h, d] at positions inside each packed sequence (the
    transpose rotation when inverse).  out=x rotates in place."""
    torch = _torch()
    _check_inputs(meta, x)
    if x.dtype != torch.bfloat16 or x.dim() != 3 or x.shape[0] != meta.total_tokens:
        raise ValueError("x must be bf16 [T, h, d] with T the pack's token count")
    out = torch.empty_like(x) if out is None else out
    _check_out("out", out, x.shape, x.dtype, x.device)
    rc = lib().pk_rope_apply(meta.handle, _ptr(x), int(x.shape[1]), int(x.shape[2]),
                             float(rope_base), 1 if inverse else 0, _ptr(out), _stream_ptr(stream))
    _lib.check("pk_rope_apply", rc)
    return out


def moe_workspace(n_assign: int, n_experts: int, device):
    torch = _torch()
    n = int(lib().pk_moe_group_workspace_bytes(int(n_assign), int(n_experts)))
    if n == 0:
        raise PkError("pk_moe_group_workspace_bytes", _lib.PK_ERR_UNSUPPORTED)
    return torch.empty(n, dtype=torch.uint8, device=device)


def moe_group(router_indices, n_experts: int, workspace=None, stream=None):
    """Group int32 router indices [n_tokens, top_k] (CUDA) by expert in one pass.  Returns a dict
    of int32 device tensors: counts [E], offsets [E+1], perm [M] (flat assignment token*top_k+slot
    at each grouped position, ascending inside a group), inv [M] (grouped position of each flat
    assignment) and status [1] (PK_MOE_BAD_EXPERT for an index outside [0, E)).  Nothing is
    read back to the host."""
    torch = _torch()
    if router_indices.dtype != torch.int32 or not router_indices.is_cuda or router_indices.dim() != 2:
        raise ValueError("router_indices must be a 2-D int32 CUDA tensor")
    idx = router_indices.contiguous()
    n_tok, top_k = int(idx.shape[0]), int(idx.shape[1])
    m = n_tok * top_k
    dev = idx.device
    mk = lambda n: torch.empty(n, dtype=torch.int32, device=dev)
    res = {"counts": mk(n_experts), "offsets": mk(n_experts + 1), "perm": mk(m), "inv": mk(m),
           "status": mk(1)}
    ws = moe_workspace(m, n_experts, dev) if workspace is None else workspace
    rc = lib().pk_moe_group(_ptr(idx), n_tok, top_k, int(n_experts), _ptr(res["counts"]),
                            _ptr(res["offsets"]), _ptr(res["perm"]), _ptr(res["inv"]),
                            _ptr(res["status"]), _ptr(ws), _ws_bytes(ws, dev), _stream_ptr(stream))
    _lib.check("pk_moe_group", rc)
    return res


class ReloadPipeline:
    """Two-slot reload of tensors from pinned host memory on a library-owned copy stream
    (pk_reload_*): fetch(slot, dst, src) copies host -> device after the slot's last release;
    acquire(slot) makes the current stream wait for the slot's copies; release(slot) marks the
    current stream's work so far as the slot's last use."""

    def __init__(self):
        h = ctypes.c_void_p()
        _lib.check("pk_reload_create", lib().pk_reload_create(ctypes.byref(h)))
        self._h = h

    def fetch(self, slot: int, dst, src) -> None:
        if not dst.is_cuda or src.is_cuda or not dst.is_contiguous() or not src.is_contiguous():
            raise ValueError("dst must be a contiguous CUDA tensor and src a contiguous host tensor")
        if not src.is_pinned():
            raise ValueError("src must be in pinned host memory (torch.empty(..., pin_memory=True)), "
                             "or the copy cannot overlap the compute")
        n = dst.numel() * dst.element_size()
        if src.numel() * src.element_size() != n:
            raise ValueError("size mismatch")
        _lib.check("pk_reload_fetch", lib().pk_reload_fetch(self._h, int(slot), _ptr(dst), _ptr(src), n))

    def acquire(self, slot: int, stream=None) -> None:
        _lib.check("pk_reload_acquire", lib().pk_reload_acquire(self._h, int(slot), _stream_ptr(stream)))

    def release(self, slot: int, stream=None) -> None:
        _lib.check("pk_reload_release", lib().pk_reload_release(self._h, int(slot), _stream_ptr(stream)))

    def close(self) -> None:
        if self._h is not None:
            lib().pk_reload_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def peak_mfma_tflops(workgroups: Optional[int] = None, iters: int = 20000, reps: int = 3) -> float:
    """Measured dense fp16 matrix-core rate (TFLOP/s): best of `reps` timed launches of
    pk_peak_mfma, by default with eight workgroups (32 waves) per compute unit (the highest of
    2, 3, 4 and 8 per compute unit when measured on the part)."""
    torch = _torch()
    if workgroups is None:
        workgroups = 8 * torch.cuda.get_device_properties(torch.cuda.current_device()).multi_processor_count
    sink = torch.empty(4 * workgroups, dtype=torch.float32, device="cuda")
    flops = workgroups * 4 * 4 * iters * 32 * 32 * 16 * 2
    best = 0.0
    for r in range(reps + 1):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        _lib.check("pk_peak_mfma", lib().pk_peak_mfma(_ptr(sink), workgroups, iters, _stream_ptr(None)))
        e1.record()
        e1.synchronize()
        if r:   # the first launch warms up
            best = max(best, flops / (e0.elapsed_time(e1) * 1e-3) / 1e12)
    return best


def peak_hbm_gbps(nbytes: int = 2 << 30, reps: int = 3) -> dict:
    """Measured HBM bandwidth (GB/s) of a plain read, write and copy of `nbytes` (best of reps)."""
    torch = _torch()
    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    sink = torch.zeros(1, dtype=torch.float32, device="cuda")
    out = {}
    for mode, name, moved in ((0, "read", nbytes), (1, "write", nbytes), (2, "copy", 2 * nbytes)):
        best = 0.0
        for r in range(reps + 1):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            _lib.check("pk_peak_hbm", lib().pk_peak_hbm(mode, _ptr(src), _ptr(dst), nbytes, _ptr(sink),
                                                        _stream_ptr(None)))
            e1.record()
            e1.synchronize()
            if r:
                best = max(best, moved / (e0.elapsed_time(e1) * 1e-3) / 1e9)
        out[name] = round(best, 1)
    return out


def lora_workspace(t: int, k: int, n: int, r: int, device):
    torch = _torch()
    nb = int(lib().pk_lora_qkv_workspace_bytes(int(t), int(k), int(n), int(r)))
    if nb == 0:
        raise PkError("pk_lora_qkv_workspace_bytes", _lib.PK_ERR_UNSUPPORTED)
    return torch.empty(nb, dtype=torch.uint8, device=device)


def lora_qkv(x, wt, at, bt, scale: float = 1.0, out=None, workspace=None, stream=None):
    """y = x (W + scale A B) for bf16 x [T, K], wt = W^T [N, K], at = A^T [r, K], bt = B^T [N, r]
    (a linear layer's weight layout); returns y bf16 [T, N]."""
    torch = _torch()
    for z in (x, wt, at, bt):
        if not z.is_cuda or not z.is_contiguous() or z.dtype != torch.bfloat16 or z.dim() != 2:
            raise ValueError("x, wt, at, bt must be contiguous 2-D bf16 CUDA tensors")
    t, k = int(x.shape[0]), int(x.shape[1])
    n, r = int(wt.shape[0]), int(at.shape[0])
    if wt.shape[1] != k or at.shape[1] != k or tuple(bt.shape) != (n, r):
        raise ValueError("shape mismatch")
    if any(z.device != x.device for z in (wt, at, bt)):
        raise ValueError("x, wt, at, bt must be on one device")
    out = torch.empty((t, n), dtype=torch.bfloat16, device=x.device) if out is None else out
    _check_out("out", out, (t, n), torch.bfloat16, x.device)
    ws = lora_workspace(t, k, n, r, x.device) if workspace is None else workspace
    rc = lib().pk_lora_qkv(_ptr(x), _ptr(wt), _ptr(at), _ptr(bt), t, k, n, r, float(scale), _ptr(out),
                           _ptr(ws), _ws_bytes(ws, x.device), _stream_ptr(stream))
    _lib.check("pk_lora_qkv", rc)
    return out


def attn_bwd_prep(meta: PackedMeta, q, k, v, out, lse, dout, workspace,
                  softmax_scale: Optional[float] = None, rope_base: float = 10000.0, stream=None):
    """First half of attn_bwd: the backward's operands into `workspace` (pk_attn_bwd_prep)."""
    torch = _torch()
    t, hq, hkv, d = _dims(q, k)
    _check_inputs(meta, q, k, v, out, lse, dout, workspace)
    if t != meta.total_tokens or out.shape != q.shape or dout.shape != q.shape:
        raise ValueError("shape mismatch with the pack")
    _check_bwd_inputs(q, k, v, out, lse, dout, t, hq, d)
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    rc = lib().pk_attn_bwd_prep(meta.handle, _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(dout),
                                hq, hkv, d, scale, float(rope_base), _ptr(workspace),
                                _ws_bytes(workspace, q.device), _stream_ptr(stream))
    _lib.check("pk_attn_bwd_prep", rc)


def attn_bwd_main(meta: PackedMeta, hq: int, hkv: int, d: int, workspace, dq, dk, dv,
                  softmax_scale: Optional[float] = None, stream=None):
    """Second half of attn_bwd: dq, dk, dv from the operands attn_bwd_prep left in `workspace`."""
    torch = _torch()
    _check_inputs(meta, workspace, dq, dk, dv)
    t = meta.total_tokens
    _check_out("dq", dq, (t, hq, d), torch.float32, meta.device)
    _check_out("dk", dk, (t, hkv, d), torch.float32, meta.device)
    _check_out("dv", dv, (t, hkv, d), torch.float32, meta.device)
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    rc = lib().pk_attn_bwd_main(meta.handle, int(hq), int(hkv), int(d), scale, _ptr(dq), _ptr(dk), _ptr(dv),
                                _ptr(workspace), _ws_bytes(workspace, meta.device), _stream_ptr(stream))
    _lib.check("pk_attn_bwd_main", rc)
    return dq, dk, dv


def prof_enable(on: bool = True, kinds=None) -> None:
    """Record HIP events around launches of the given kernel kinds (names of KERNEL_KINDS;
    all when None), or stop recording (on=False)."""
    mask = 0
    if on:
        mask = _lib.PK_PROF_ALL if kinds is None else sum(1 << _lib.KERNEL_KINDS[k] for k in set(kinds))
    _lib.check("pk_prof_enable", lib().pk_prof_enable(mask))


def prof_reset() -> None:
    _lib.check("pk_prof_reset", lib().pk_prof_reset())


def prof_query(kind: str) -> Tuple[float, int]:
    """(total ms, launches) of one kernel kind since the last reset (synchronises on events)."""
    ms, n = ctypes.c_double(0.0), ctypes.c_int64(0)
    _lib.check("pk_prof_query", lib().pk_prof_query(_lib.KERNEL_KINDS[kind], ctypes.byref(ms), ctypes.byref(n)))
    return float(ms.value), int(n.value)


class PackedCausalAttention:
    """torch.autograd.Function over pk_attn_fwd / pk_attn_bwd (gradients cast to the inputs'
    bfloat16 by torch).  Use `PackedCausalAttention.apply(q, k, v, meta, scale, rope_base)`."""

    _fn = None

    @classmethod
    def apply(cls, q, k, v, meta: PackedMeta, softmax_scale=None, rope_base: float = 10000.0):
        if cls._fn is None:
            torch = _torch()

            class _F(torch.autograd.Function):
                @staticmethod
                def forward(ctx, q, k, v, meta, softmax_scale, rope_base):
                    out, lse = attn_fwd(meta, q, k, v, softmax_scale, rope_base)
                    ctx.save_for_backward(q, k, v, out, lse)
                    ctx.meta, ctx.scale, ctx.base = meta, softmax_scale, rope_base
                    return out

                @staticmethod
                def backward(ctx, dout):
                    q, k, v, out, lse = ctx.saved_tensors
                    dq, dk, dv = attn_bwd(ctx.meta, q, k, v, out, lse,
                                          dout.to(torch.bfloat16).contiguous(), ctx.scale, ctx.base)
                    return dq.to(q.dtype), dk.to(k.dtype), dv.to(v.dtype), None, None, None

            cls._fn = _F
        return cls._fn.apply(q, k, v, meta, softmax_scale, rope_base)
