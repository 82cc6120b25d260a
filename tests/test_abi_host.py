"""Host-side checks of the C interface: the library loads, exports every
function ``include/spense.h`` declares, and rejects bad arguments on the host
before any HIP call (so these run without a GPU)."""

import ctypes
import os
import re

import numpy as np
import pytest

import sparse_dense_gemm_amd as sdg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE_PTR = 1 << 20  # never dereferenced: validation fails before any HIP call


def header_functions():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if not fn.endswith(".h"):
            continue
        src = open(os.path.join(ROOT, "include", fn)).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        for m in re.finditer(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(spense_[a-z0-9_]+)\s*\(", src, re.M):
            names.add(m.group(1))
    return sorted(names)


def test_library_exports_every_declared_function():
    names = header_functions()
    assert {"spense_pack", "spense_linear", "spense_free", "spense_export", "spense_info"} <= set(names)
    lib = ctypes.CDLL(sdg.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_abi_version_and_strerror():
    assert sdg.spense_abi_version() == 6
    lib = sdg._lib()
    for code in (0, -1, -2, -3, -4, -5):
        assert lib.spense_strerror(code) and lib.spense_strerror(code) != b"unknown status"
    assert lib.spense_strerror(12345) == b"unknown status"


def _pack(W=FAKE_PTR, wdt=sdg.DT_FP8, N=64, K=128, ldw=None, scales=FAKE_PTR, cols=None, frac=0.25):
    lib = sdg._lib()
    h = ctypes.c_void_p()
    cols_ptr, n = None, 0
    keep = None
    if cols is not None:
        keep = np.ascontiguousarray(np.asarray(cols, dtype=np.int32))
        cols_ptr, n = (keep.ctypes.data if keep.size else np.zeros(1, np.int32).ctypes.data), keep.size
    st = lib.spense_pack(W, wdt, N, K, K if ldw is None else ldw, scales, cols_ptr, n, frac, None, ctypes.byref(h))
    return st, h.value


@pytest.mark.parametrize("kw", [
    dict(W=None),                               # null weights
    dict(wdt=7),                                # unknown dtype
    dict(N=0), dict(K=0), dict(ldw=100),        # sizes
    dict(scales=None),                          # e4m3 needs scales
    dict(wdt=sdg.DT_BF16),                      # bf16 must not get scales
    dict(frac=1.5), dict(frac=-0.1), dict(frac=float("nan")),
    dict(K=130, frac=0.0),                      # K_s % 4 != 0
    dict(cols=[1, 2, 3]),                       # K - 3 not a multiple of 4
    dict(cols=[1, 1, 2, 3]),                    # duplicate
    dict(cols=[-1, 1, 2, 3]), dict(cols=[128, 1, 2, 3]),  # out of range
])
def test_pack_rejects_bad_arguments(kw):
    st, h = _pack(**kw)
    assert st == sdg.SPENSE_EINVAL and not h


def _pack_rows(W=FAKE_PTR, wdt=sdg.DT_FP8, N=64, K=128, ldw=None, scales=FAKE_PTR, rows=None, frac=0.25):
    lib = sdg._lib()
    h = ctypes.c_void_p()
    rows_ptr, n = None, 0
    keep = None
    if rows is not None:
        keep = np.ascontiguousarray(np.asarray(rows, dtype=np.int32))
        rows_ptr, n = (keep.ctypes.data if keep.size else np.zeros(1, np.int32).ctypes.data), keep.size
    st = lib.spense_pack_rows(W, wdt, N, K, K if ldw is None else ldw, scales, rows_ptr, n, frac, None,
                              ctypes.byref(h))
    return st, h.value


@pytest.mark.parametrize("kw,want", [
    (dict(W=None), sdg.SPENSE_EINVAL),
    (dict(wdt=7), sdg.SPENSE_EINVAL),
    (dict(N=0), sdg.SPENSE_EINVAL), (dict(K=0), sdg.SPENSE_EINVAL), (dict(ldw=100), sdg.SPENSE_EINVAL),
    (dict(scales=None), sdg.SPENSE_EINVAL),
    (dict(frac=1.5), sdg.SPENSE_EINVAL), (dict(frac=float("nan")), sdg.SPENSE_EINVAL),
    (dict(K=130, frac=0.5), sdg.SPENSE_EINVAL),      # sparse rows need K % 4 == 0
    (dict(rows=[3, 3]), sdg.SPENSE_EINVAL),          # duplicate row
    (dict(rows=[64]), sdg.SPENSE_EINVAL), (dict(rows=[-1]), sdg.SPENSE_EINVAL),
    (dict(wdt=sdg.DT_F32, scales=None), sdg.SPENSE_EUNSUPPORTED),  # no fp32 output-split
])
def test_pack_rows_rejects_bad_arguments(kw, want):
    st, h = _pack_rows(**kw)
    assert st == want and not h


def test_linear_rejects_bad_arguments():
    lib = sdg._lib()
    assert lib.spense_linear(None, FAKE_PTR, sdg.DT_BF16, 1, 128, FAKE_PTR, sdg.DT_F32, 64, None) == sdg.SPENSE_EINVAL
    assert lib.spense_linear_noalloc(None, FAKE_PTR, sdg.DT_BF16, 1, 128, FAKE_PTR, sdg.DT_F32, 64,
                                     None) == sdg.SPENSE_EINVAL
    assert lib.spense_free(None) == sdg.SPENSE_EINVAL
    assert lib.spense_info(None, None) == sdg.SPENSE_EINVAL
    assert lib.spense_export(None, None, None, None, None, None, None) == sdg.SPENSE_EINVAL
    assert lib.spense_export_rows(None, None, None, None, None, None, None) == sdg.SPENSE_EINVAL


def test_binding_fails_loudly_without_library(monkeypatch):
    monkeypatch.setattr(sdg, "_lib_handle", None)
    monkeypatch.setattr(sdg, "LIB_PATH", "/nonexistent/libspense.so")
    with pytest.raises(RuntimeError, match="not built"):
        sdg.spense_abi_version()


def _pack_glu(Wgu=FAKE_PTR, Wd=FAKE_PTR, wdt=sdg.DT_FP8, H=128, I=256, ldgu=None, ldd=None, sgu=FAKE_PTR,
              sd=FAKE_PTR, idx=None, frac=0.25):
    lib = sdg._lib()
    h = ctypes.c_void_p()
    idx_ptr, n = None, 0
    keep = None
    if idx is not None:
        keep = np.ascontiguousarray(np.asarray(idx, dtype=np.int32))
        idx_ptr, n = (keep.ctypes.data if keep.size else np.zeros(1, np.int32).ctypes.data), keep.size
    st = lib.spense_pack_glu(Wgu, Wd, wdt, H, I, H if ldgu is None else ldgu, I if ldd is None else ldd, sgu, sd,
                             idx_ptr, n, frac, None, ctypes.byref(h))
    return st, h.value


@pytest.mark.parametrize("kw,want", [
    (dict(Wgu=None), sdg.SPENSE_EINVAL), (dict(Wd=None), sdg.SPENSE_EINVAL),
    (dict(wdt=sdg.DT_F32, sgu=None, sd=None), sdg.SPENSE_EUNSUPPORTED),
    (dict(H=0), sdg.SPENSE_EINVAL), (dict(I=0), sdg.SPENSE_EINVAL),
    (dict(ldgu=100), sdg.SPENSE_EINVAL), (dict(ldd=200), sdg.SPENSE_EINVAL),
    (dict(sgu=None), sdg.SPENSE_EINVAL), (dict(sd=None), sdg.SPENSE_EINVAL),
    (dict(wdt=sdg.DT_BF16), sdg.SPENSE_EINVAL),            # bf16 must not get scales
    (dict(idx=[1, 2, 3]), sdg.SPENSE_EINVAL),              # I - 3 not a multiple of 4
    (dict(idx=[5, 5, 6, 7]), sdg.SPENSE_EINVAL),           # duplicate index
    (dict(H=130, frac=0.5), sdg.SPENSE_EINVAL),            # 2:4 gate/up rows need H % 4 == 0
    (dict(frac=2.0), sdg.SPENSE_EINVAL),
])
def test_pack_glu_rejects_bad_arguments(kw, want):
    st, h = _pack_glu(**kw)
    assert st == want and not h


def test_glu_rejects_bad_arguments():
    lib = sdg._lib()
    assert lib.spense_glu(None, FAKE_PTR, 1, 128, FAKE_PTR, 256, FAKE_PTR, sdg.DT_F32, 128, None) == sdg.SPENSE_EINVAL


def test_score_and_select_reject_bad_arguments():
    lib = sdg._lib()
    P = FAKE_PTR
    # null pointers, bad sizes, scale mismatch, fp32 weights
    assert lib.spense_score_glu(None, P, sdg.DT_FP8, 64, 128, 64, 128, P, P, P, 4, 64, P, 128, P, None) == sdg.SPENSE_EINVAL
    assert lib.spense_score_glu(P, P, sdg.DT_FP8, 0, 128, 64, 128, P, P, P, 4, 64, P, 128, P, None) == sdg.SPENSE_EINVAL
    assert lib.spense_score_glu(P, P, sdg.DT_FP8, 64, 128, 64, 128, P, P, P, 0, 64, P, 128, P, None) == sdg.SPENSE_EINVAL
    assert lib.spense_score_glu(P, P, sdg.DT_FP8, 64, 128, 64, 128, P, P, P, 4, 32, P, 128, P, None) == sdg.SPENSE_EINVAL
    assert lib.spense_score_glu(P, P, sdg.DT_FP8, 64, 128, 64, 128, None, P, P, 4, 64, P, 128, P, None) == sdg.SPENSE_EINVAL
    assert lib.spense_score_glu(P, P, sdg.DT_BF16, 64, 128, 64, 128, P, P, P, 4, 64, P, 128, P, None) == sdg.SPENSE_EINVAL
    assert (lib.spense_score_glu(P, P, sdg.DT_F32, 64, 128, 64, 128, None, None, P, 4, 64, P, 128, P, None)
            == sdg.SPENSE_EUNSUPPORTED)
    out = np.zeros(4, dtype=np.int32)
    assert lib.spense_select_dense(None, 8, 2, out.ctypes.data, None) == sdg.SPENSE_EINVAL
    assert lib.spense_select_dense(P, 8, 9, out.ctypes.data, None) == sdg.SPENSE_EINVAL
    assert lib.spense_select_dense(P, 8, -1, out.ctypes.data, None) == sdg.SPENSE_EINVAL
    assert lib.spense_select_dense(P, 8, 2, None, None) == sdg.SPENSE_EINVAL


def test_w8a8_entry_points_reject_bad_arguments():
    lib = sdg._lib()
    P = FAKE_PTR
    E = sdg.SPENSE_EINVAL
    assert lib.spense_quantize_tokens(None, 4, 64, 64, P, 64, P, None) == E
    assert lib.spense_quantize_tokens(P, 4, 64, 64, None, 64, P, None) == E
    assert lib.spense_quantize_tokens(P, 4, 64, 64, P, 64, None, None) == E
    assert lib.spense_quantize_tokens(P, 0, 64, 64, P, 64, P, None) == E
    assert lib.spense_quantize_tokens(P, 4, 0, 64, P, 64, P, None) == E
    assert lib.spense_quantize_tokens(P, 4, 64, 63, P, 64, P, None) == E
    assert lib.spense_quantize_tokens(P, 4, 64, 64, P, 32, P, None) == E
    assert lib.spense_quantize_tokens(P, (1 << 24) + 1, 64, 64, P, 64, P, None) == E
    assert lib.spense_linear_w8a8(None, P, 1, 128, P, sdg.DT_F32, 64, 0, None) == E
