"""Host-side checks of the C ABI (no kernel is launched; runs without a GPU).

The library must load, export every entry point the header declares, and
reject bad arguments with the documented status codes before touching the
device.
"""
from __future__ import annotations

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ffn_sparse.h")


@pytest.fixture(scope="module")
def L():
    from activation_sparse_gated_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("library not built (run __graft_entry__.build())")
    return _lib


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(ffn_sparse_[a-z_]+)\s*\(", text)))


def cfg(L, **kw):
    base = dict(d_model=2048, d_ff=8192, rank=0, dtype=1, act=0, sel=0, tile_w=128, ell_w=64,
                wdown_out_major=1, max_m=16)
    base.update(kw)
    return L.Config(**base)


def test_exports_every_declared_symbol(L):
    lib = L.load()
    names = declared_symbols()
    assert len(names) >= 14
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(L.EXPORTS)
    assert lib.ffn_sparse_abi_version() == 1


def test_status_strings(L):
    lib = L.load()
    for code in (0, -1, -2, -3, -4):
        assert lib.ffn_sparse_status_string(code).decode()


@pytest.mark.parametrize("kw,want", [
    ({}, 0),
    (dict(rank=512, d_model=4096, d_ff=14336, sel=1), 0),
    (dict(sel=2, act=1, ell_w=128, d_ff=11008, d_model=4096), 0),
    (dict(dtype=0, d_model=256, d_ff=1024, tile_w=64, ell_w=64), 0),
    (dict(tile_w=1024, ell_w=128, max_m=4096), 0),
    (dict(d_ff=8000), -1),                 # d_ff not a multiple of tile_w
    (dict(ell_w=129), -1),                 # E > T
    (dict(ell_w=-1), -1),
    (dict(dtype=7), -1),
    (dict(max_m=0), -1),
    (dict(max_m=70000), -2),
    (dict(d_model=2000), -2),              # d_model not a multiple of 64
    (dict(d_model=8192), -2),              # beyond the register-resident row length
    (dict(act=1), -2),                     # bias selection needs a ReLU gate
    (dict(sel=2, act=1, ell_w=64), -2),    # top-k needs E == T
    (dict(sel=2, act=1, ell_w=128, rank=64), -2),
    (dict(rank=48), -2),
    (dict(tile_w=24, d_ff=8184, ell_w=8), -2),
])
def test_check_config(L, kw, want):
    lib = L.load()
    c = cfg(L, **kw)
    assert lib.ffn_sparse_check_config(ctypes.byref(c)) == want
    nbytes = lib.ffn_sparse_workspace_bytes(ctypes.byref(c))
    assert (nbytes > 0) == (want == 0)


def test_pack_bytes(L):
    lib = L.load()
    c = cfg(L)
    nt, E = 8192 // 128, 64

    def a(v):
        return (v + 255) // 256 * 256

    for m in (0, 1, 16):
        want = a(m * nt * 4) + a(m * nt * E * 2) * 2 + a(m) + a(m * 4) + a(4)
        assert lib.ffn_sparse_pack_bytes(ctypes.byref(c), m) == want
    assert lib.ffn_sparse_pack_bytes(ctypes.byref(c), -1) == 0


def test_init_rejects_bad_pointers_before_launch(L):
    lib = L.load()
    c = cfg(L)
    h = ctypes.c_void_p()
    assert lib.ffn_sparse_init(ctypes.byref(c), None, None, 16, 16, 16, 1 << 30, None, ctypes.byref(h)) == -1
    assert lib.ffn_sparse_init(ctypes.byref(c), 17, None, 16, 16, 16, 1 << 30, None, ctypes.byref(h)) == -1
    low = cfg(L, rank=512, d_model=4096, d_ff=14336, sel=1)
    assert lib.ffn_sparse_init(ctypes.byref(low), 16, None, 16, 16, 16, 1 << 30, None, ctypes.byref(h)) == -1
    assert lib.ffn_sparse_init(ctypes.byref(c), 16, None, 16, 16, 16, 1 << 30, None, None) == -1


def test_calls_reject_null_handle(L):
    lib = L.load()
    p = L.Pack()
    assert lib.ffn_sparse_gate_pack(None, 16, 1, None, 0.0, None, 0, ctypes.byref(p), None, None, None) == -1
    assert lib.ffn_sparse_updown(None, 16, 1, ctypes.byref(p), 16, None) == -1
    assert lib.ffn_sparse_forward(None, 16, 1, None, 0.0, None, 0, ctypes.byref(p), 16, None) == -1
    assert lib.ffn_sparse_dense_forward(None, 16, 1, None, 0.0, None, 16, None) == -1
    assert lib.ffn_sparse_timing_enable(None, 1, 4) == -1
    assert lib.ffn_sparse_forward_path(None, 1) == -1
    lib.ffn_sparse_destroy(None)
