"""The C-ABI library loads on a machine without a GPU, exports every symbol pk.h declares, and
rejects bad arguments on the host before touching the device (CPU only)."""
import ctypes
import os
import re

import pytest

from oracle import pk_oracle as O
from packed_sequence_causal_pk_amd import _lib

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "pk.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pk_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libpk.so is not built: run python -m packed_sequence_causal_pk_amd.build")
    return _lib.lib()


def test_exports_every_declared_symbol(lib):
    names = _declared_functions()
    assert len(names) >= 14
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_lib.SIGNATURES), "binding and header disagree"


def test_tile_rows_and_sizes(lib):
    assert lib.pk_tile_rows() == O.TILE_ROWS == 128
    small = lib.pk_meta_bytes(4, 256)
    assert small > 0 and small % 256 == 0
    assert lib.pk_meta_bytes(3814, 65536) > lib.pk_meta_bytes(10, 16384) > small
    assert lib.pk_meta_bytes(0, 0) > 0
    assert lib.pk_meta_bytes(-1, 10) == 0
    assert lib.pk_meta_bytes(5, 4) == 0            # more sequences than tokens
    assert lib.pk_meta_bytes(1, (1 << 20) + 1) == 0


def test_host_side_rejections(lib):
    h = ctypes.c_void_p()
    fake = ctypes.c_void_p(0x10000)  # never dereferenced: every case fails before any launch
    assert lib.pk_build_meta(fake, 4, 256, fake, 1 << 20, None, None) == _lib.PK_ERR_INVALID
    assert lib.pk_build_meta(fake, -1, 256, fake, 1 << 20, None, ctypes.byref(h)) == _lib.PK_ERR_INVALID
    assert lib.pk_build_meta(fake, 4, 1 << 21, fake, 1 << 30, None, ctypes.byref(h)) == _lib.PK_ERR_UNSUPPORTED
    assert lib.pk_build_meta(None, 4, 256, fake, 1 << 20, None, ctypes.byref(h)) == _lib.PK_ERR_INVALID
    assert lib.pk_build_meta(fake, 4, 256, None, 1 << 20, None, ctypes.byref(h)) == _lib.PK_ERR_INVALID
    unaligned = ctypes.c_void_p(0x10004)
    assert lib.pk_build_meta(fake, 4, 256, unaligned, 1 << 20, None, ctypes.byref(h)) == _lib.PK_ERR_INVALID
    assert lib.pk_build_meta(fake, 4, 256, fake, 16, None, ctypes.byref(h)) == _lib.PK_ERR_CAPACITY
    assert lib.pk_build_meta(fake, 300, 256, fake, 1 << 20, None, ctypes.byref(h)) == _lib.PK_ERR_INVALID
    assert h.value is None
    args_fwd = [None, fake, fake, fake, 2, 1, 64, 0.125, 1e4, fake, fake, fake, 1 << 20, None]
    assert lib.pk_attn_fwd(*args_fwd) == _lib.PK_ERR_INVALID
    assert lib.pk_attn_fwd_noalloc(None, fake, fake, fake, 2, 1, 64, 0.125, 1e4, fake, fake, None) == _lib.PK_ERR_INVALID
    args_bwd = [None, fake, fake, fake, fake, fake, fake, 2, 1, 64, 0.125, 1e4, fake, fake, fake, fake, 1 << 20, None]
    assert lib.pk_attn_bwd(*args_bwd) == _lib.PK_ERR_INVALID
    args_prep = [None, fake, fake, fake, fake, fake, fake, 2, 1, 64, 0.125, 1e4, fake, 1 << 20, None]
    assert lib.pk_attn_bwd_prep(*args_prep) == _lib.PK_ERR_INVALID
    assert lib.pk_attn_bwd_main(None, 2, 1, 64, 0.125, fake, fake, fake, fake, 1 << 20, None) == _lib.PK_ERR_INVALID
    assert lib.pk_attn_fwd_workspace_bytes(None, 2, 1, 64) == 0
    assert lib.pk_attn_bwd_workspace_bytes(None, 2, 1, 64) == 0
    assert lib.pk_meta_destroy(None) == _lib.PK_ERR_INVALID
    assert lib.pk_meta_view(None, None) == _lib.PK_ERR_INVALID
    assert lib.pk_meta_check(None, None, None, None) == _lib.PK_ERR_INVALID


def test_host_side_rejections_aux(lib):
    fake = ctypes.c_void_p(0x10000)  # never dereferenced: every case fails before any launch
    assert lib.pk_dense_mask(None, fake, 1 << 20, None) == _lib.PK_ERR_INVALID
    assert lib.pk_rope_apply(None, fake, 2, 64, 1e4, 0, fake, None) == _lib.PK_ERR_INVALID
    assert lib.pk_moe_group_workspace_bytes(0, 1) > 0
    assert lib.pk_moe_group_workspace_bytes(65536, 128) >= 128 * 16 * 4
    assert lib.pk_moe_group_workspace_bytes(-1, 8) == 0
    assert lib.pk_moe_group_workspace_bytes(16, 0) == 0
    assert lib.pk_moe_group_workspace_bytes(16, _lib.PK_MOE_MAX_EXPERTS + 1) == 0
    assert lib.pk_moe_group_workspace_bytes(_lib.PK_MOE_MAX_ASSIGN + 1, 8) == 0
    ws = lib.pk_moe_group_workspace_bytes(64, 8)
    ok = [fake, 16, 4, 8, fake, fake, fake, fake, fake, fake, ws, None]

    def call(**kw):
        a = list(ok)
        names = ["idx", "n_tok", "top_k", "n_exp", "counts", "offsets", "perm", "inv", "status",
                 "ws", "ws_bytes", "stream"]
        for k, v in kw.items():
            a[names.index(k)] = v
        return lib.pk_moe_group(*a)

    assert call(n_tok=-1) == _lib.PK_ERR_INVALID
    assert call(top_k=0) == _lib.PK_ERR_INVALID
    assert call(n_exp=0) == _lib.PK_ERR_UNSUPPORTED
    assert call(n_exp=_lib.PK_MOE_MAX_EXPERTS + 1) == _lib.PK_ERR_UNSUPPORTED
    assert call(n_tok=_lib.PK_MOE_MAX_ASSIGN) == _lib.PK_ERR_UNSUPPORTED
    assert call(idx=None) == _lib.PK_ERR_INVALID
    assert call(perm=None) == _lib.PK_ERR_INVALID
    assert call(counts=None) == _lib.PK_ERR_INVALID
    assert call(status=None) == _lib.PK_ERR_INVALID
    assert call(ws=ctypes.c_void_p(0x10004)) == _lib.PK_ERR_INVALID
    assert call(ws_bytes=ws - 1) == _lib.PK_ERR_CAPACITY


def test_host_side_rejections_peak_and_reload(lib):
    fake = ctypes.c_void_p(0x10000)  # never dereferenced: every case fails before any launch
    assert lib.pk_peak_mfma(None, 512, 100, None) == _lib.PK_ERR_INVALID
    assert lib.pk_peak_mfma(fake, 0, 100, None) == _lib.PK_ERR_INVALID
    assert lib.pk_peak_mfma(fake, 512, 0, None) == _lib.PK_ERR_INVALID
    assert lib.pk_peak_hbm(3, fake, fake, 1 << 20, fake, None) == _lib.PK_ERR_INVALID
    assert lib.pk_peak_hbm(0, fake, fake, 1000, fake, None) == _lib.PK_ERR_INVALID     # not a multiple of 16
    assert lib.pk_peak_hbm(0, None, fake, 1 << 20, fake, None) == _lib.PK_ERR_INVALID
    assert lib.pk_peak_hbm(1, fake, None, 1 << 20, fake, None) == _lib.PK_ERR_INVALID
    assert lib.pk_peak_hbm(0, ctypes.c_void_p(0x10008), fake, 1 << 20, fake, None) == _lib.PK_ERR_INVALID
    assert lib.pk_reload_create(None) == _lib.PK_ERR_INVALID
    assert lib.pk_reload_fetch(None, 0, fake, fake, 16) == _lib.PK_ERR_INVALID
    assert lib.pk_reload_acquire(None, 0, None) == _lib.PK_ERR_INVALID
    assert lib.pk_reload_release(None, 1, None) == _lib.PK_ERR_INVALID
    assert lib.pk_reload_destroy(None) == _lib.PK_ERR_INVALID


def test_status_strings_and_profiler_queries(lib):
    for code in (0, -1, -2, -3, -4, -5):
        assert _lib.status_str(code)
    assert _lib.status_str(-99) == "unknown status"
    ms, n = ctypes.c_double(1.0), ctypes.c_int64(1)
    assert lib.pk_prof_query(99, ctypes.byref(ms), ctypes.byref(n)) == _lib.PK_ERR_INVALID
    assert lib.pk_prof_enable(-1) == _lib.PK_ERR_INVALID
    assert lib.pk_prof_enable(_lib.PK_PROF_ALL + 1) == _lib.PK_ERR_INVALID
    assert lib.pk_prof_enable(0) == 0
    assert lib.pk_prof_reset() == 0
    assert lib.pk_prof_query(_lib.PK_K_FWD, ctypes.byref(ms), ctypes.byref(n)) == 0
    assert ms.value == 0.0 and n.value == 0
