"""ctypes declarations of libpk.so (include/pk.h).  Loading never touches the GPU."""
from __future__ import annotations

import ctypes
import os

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libpk.so")

PK_OK = 0
PK_ERR_INVALID = -1
PK_ERR_UNSUPPORTED = -2
PK_ERR_CAPACITY = -3
PK_ERR_HIP = -4
PK_ERR_DEVICE = -5

PK_META_BAD_LENGTH = 1
PK_META_BAD_TOTAL = 2

PK_K_META, PK_K_FWD_PREP, PK_K_FWD, PK_K_BWD_PREP, PK_K_BWD, PK_K_BWD_DQ = range(6)
PK_K_MASK, PK_K_ROPE, PK_K_MOE, PK_K_LORA = 6, 7, 8, 9
KERNEL_KINDS = {"meta": PK_K_META, "fwd_prep": PK_K_FWD_PREP, "fwd": PK_K_FWD,
                "bwd_prep": PK_K_BWD_PREP, "bwd": PK_K_BWD, "bwd_dq": PK_K_BWD_DQ,
                "mask": PK_K_MASK, "rope": PK_K_ROPE, "moe": PK_K_MOE, "lora": PK_K_LORA}

PK_MASK_MAX_TOKENS = 65536
PK_MOE_MAX_EXPERTS = 1024
PK_MOE_MAX_ASSIGN = 1 << 26
PK_MOE_BAD_EXPERT = 1
PK_LORA_MAX_RANK = 64
PK_NOALLOC_SCRATCH_BYTES = 128 << 20
PK_DS_BLOCK_ROWS = 64
PK_PROF_ALL = (1 << len(KERNEL_KINDS)) - 1

# every function pk.h declares, with (restype, argtypes)
_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_f32 = ctypes.c_float
_sz = ctypes.c_size_t


class MetaView(ctypes.Structure):
    _fields_ = [
        ("cu_seqlens", _vp), ("max_seqlen", _vp), ("status", _vp), ("seq_id", _vp), ("pos", _vp),
        ("fwd_items", _vp), ("bwd_items", _vp),
        ("n_seqs", _i32), ("n_items", _i32), ("total_tokens", _i64), ("device", _i32),
        ("ds_off", _vp),
    ]


SIGNATURES = {
    "pk_tile_rows": (_i32, []),
    "pk_meta_bytes": (_sz, [_i32, _i64]),
    "pk_build_meta": (_i32, [_vp, _i32, _i64, _vp, _sz, _vp, ctypes.POINTER(_vp)]),
    "pk_meta_view": (_i32, [_vp, ctypes.POINTER(MetaView)]),
    "pk_meta_check": (_i32, [_vp, _vp, ctypes.POINTER(_i32), ctypes.POINTER(_i32)]),
    "pk_meta_destroy": (_i32, [_vp]),
    "pk_attn_fwd_workspace_bytes": (_sz, [_vp, _i32, _i32, _i32]),
    "pk_attn_fwd": (_i32, [_vp, _vp, _vp, _vp, _i32, _i32, _i32, _f32, _f32, _vp, _vp, _vp, _sz, _vp]),
    "pk_attn_fwd_noalloc": (_i32, [_vp, _vp, _vp, _vp, _i32, _i32, _i32, _f32, _f32, _vp, _vp, _vp]),
    "pk_attn_bwd_workspace_bytes": (_sz, [_vp, _i32, _i32, _i32]),
    "pk_attn_bwd_workspace_bytes_ds": (_sz, [_vp, _i32, _i32, _i32, _i64]),
    "pk_attn_bwd": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _f32, _f32,
                           _vp, _vp, _vp, _vp, _sz, _vp]),
    "pk_dense_mask": (_i32, [_vp, _vp, _sz, _vp]),
    "pk_rope_apply": (_i32, [_vp, _vp, _i32, _i32, _f32, _i32, _vp, _vp]),
    "pk_moe_group_workspace_bytes": (_sz, [_i64, _i32]),
    "pk_moe_group": (_i32, [_vp, _i64, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "pk_lora_qkv_workspace_bytes": (_sz, [_i64, _i32, _i32, _i32]),
    "pk_lora_qkv": (_i32, [_vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _f32, _vp, _vp, _sz, _vp]),
    "pk_reload_create": (_i32, [ctypes.POINTER(_vp)]),
    "pk_reload_fetch": (_i32, [_vp, _i32, _vp, _vp, _sz]),
    "pk_reload_acquire": (_i32, [_vp, _i32, _vp]),
    "pk_reload_release": (_i32, [_vp, _i32, _vp]),
    "pk_reload_destroy": (_i32, [_vp]),
    "pk_peak_mfma": (_i32, [_vp, _i32, _i32, _vp]),
    "pk_peak_hbm": (_i32, [_i32, _vp, _vp, _sz, _vp, _vp]),
    "pk_attn_bwd_prep": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _f32, _f32,
                                _vp, _sz, _vp]),
    "pk_attn_bwd_main": (_i32, [_vp, _i32, _i32, _i32, _f32, _vp, _vp, _vp, _vp, _sz, _vp]),
    "pk_status_str": (ctypes.c_char_p, [_i32]),
    "pk_prof_enable": (_i32, [_i32]),
    "pk_prof_reset": (_i32, []),
    "pk_prof_query": (_i32, [_i32, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(_i64)]),
}

_LIB = None


class PkError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__("%s failed: %s (%d)" % (fn, status_str(status), status))


def lib() -> ctypes.CDLL:
    """The loaded library.  Raises if it has not been built: there is no fallback path."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libpk.so is missing (%s); build it with "
                               "`python -m packed_sequence_causal_pk_amd.build`" % LIB_PATH)
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = handle
    return _LIB


def status_str(status: int) -> str:
    return lib().pk_status_str(status).decode()


def check(fn: str, status: int) -> None:
    if status != PK_OK:
        raise PkError(fn, status)
