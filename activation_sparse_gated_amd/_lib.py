"""ctypes view of the C ABI in include/ffn_sparse.h and include/ffn_gsi.h (no computation here)."""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_double, c_float, c_int32, c_size_t, c_void_p

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libffn_sparse.so")

FFN_OK, FFN_E_INVALID, FFN_E_UNSUPPORTED, FFN_E_WORKSPACE, FFN_E_HIP = 0, -1, -2, -3, -4
DTYPES = {"f32": 0, "bf16": 1}
ACTS = {"relu": 0, "silu": 1}
SELS = {"bias": 0, "thresh": 1, "topk": 2}
KERNEL_KINDS = {"gate": 0, "lowrank_v": 1, "topk": 2, "updown": 3, "reduce": 4, "fallback": 5, "dense": 6,
                "route": 7, "up": 8, "bw_gate": 9, "bw_neuron": 10, "bw_dx": 11}

EXPORTS = [
    "ffn_sparse_abi_version", "ffn_sparse_status_string", "ffn_sparse_check_config",
    "ffn_sparse_workspace_bytes", "ffn_sparse_pack_bytes", "ffn_sparse_init", "ffn_sparse_gate_pack",
    "ffn_sparse_updown", "ffn_sparse_dense_fallback", "ffn_sparse_forward", "ffn_sparse_dense_forward",
    "ffn_sparse_forward_path", "ffn_sparse_timing_enable", "ffn_sparse_timing_read", "ffn_sparse_destroy",
    "ffn_sparse_device_status", "ffn_sparse_debug_waits", "ffn_sparse_forward_noalloc",
    "ffn_sparse_noalloc_scratch_bytes", "ffn_sparse_moe_workspace_bytes", "ffn_sparse_moe_forward",
    "ffn_sparse_backward_workspace_bytes", "ffn_sparse_backward",
    "ffn_gsi_check_config", "ffn_gsi_workspace_bytes", "ffn_gsi_init", "ffn_gsi_forward",
    "ffn_gsi_dense_forward", "ffn_gsi_image", "ffn_gsi_timing_enable", "ffn_gsi_timing_read",
    "ffn_gsi_destroy",
]
GSI_KERNEL_KINDS = {"proj": 0, "resid": 1, "out": 2, "dense": 3}


class Config(ctypes.Structure):
    _fields_ = [("d_model", c_int32), ("d_ff", c_int32), ("rank", c_int32), ("dtype", c_int32),
                ("act", c_int32), ("sel", c_int32), ("tile_w", c_int32), ("ell_w", c_int32),
                ("wdown_out_major", c_int32), ("max_m", c_int32), ("in_keep", c_int32)]


class GsiConfig(ctypes.Structure):
    _fields_ = [("d_in", c_int32), ("d_out", c_int32), ("k", c_int32), ("max_m", c_int32)]


class Pack(ctypes.Structure):
    _fields_ = [("cnt", c_void_p), ("idx", c_void_p), ("val", c_void_p), ("route", c_void_p),
                ("dense_list", c_void_p), ("n_dense", c_void_p)]


class FFNError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} ({status})")


_LIB = None


def load() -> ctypes.CDLL:
    """Load the built HIP library; raises if it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                           "(there is no CPU fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    P = POINTER
    sig = {
        "ffn_sparse_abi_version": (c_int32, []),
        "ffn_sparse_status_string": (ctypes.c_char_p, [c_int32]),
        "ffn_sparse_check_config": (c_int32, [P(Config)]),
        "ffn_sparse_workspace_bytes": (c_size_t, [P(Config)]),
        "ffn_sparse_pack_bytes": (c_size_t, [P(Config), c_int32]),
        "ffn_sparse_init": (c_int32, [P(Config), c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                      c_size_t, c_void_p, P(c_void_p)]),
        "ffn_sparse_gate_pack": (c_int32, [c_void_p, c_void_p, c_int32, c_void_p, c_float, c_void_p,
                                           c_int32, P(Pack), c_void_p, c_void_p, c_void_p]),
        "ffn_sparse_updown": (c_int32, [c_void_p, c_void_p, c_int32, P(Pack), c_void_p, c_void_p]),
        "ffn_sparse_dense_fallback": (c_int32, [c_void_p, c_void_p, c_int32, c_void_p, c_float, c_void_p,
                                                c_int32, P(Pack), c_void_p, c_void_p]),
        "ffn_sparse_forward": (c_int32, [c_void_p, c_void_p, c_int32, c_void_p, c_float, c_void_p,
                                         c_int32, P(Pack), c_void_p, c_void_p]),
        "ffn_sparse_dense_forward": (c_int32, [c_void_p, c_void_p, c_int32, c_void_p, c_float, c_void_p,
                                               c_void_p, c_void_p]),
        "ffn_sparse_forward_path": (c_int32, [c_void_p, c_int32]),
        "ffn_sparse_timing_enable": (c_int32, [c_void_p, c_int32, c_int32]),
        "ffn_sparse_timing_read": (c_int32, [c_void_p, c_int32, P(c_int32), P(c_double)]),
        "ffn_sparse_destroy": (None, [c_void_p]),
        "ffn_sparse_device_status": (c_int32, [c_void_p, c_void_p]),
        "ffn_sparse_forward_noalloc": (c_int32, [c_void_p, c_void_p, c_int32, c_void_p, c_float, c_void_p,
                                                 c_int32, P(Pack), c_void_p, c_void_p]),
        "ffn_sparse_noalloc_scratch_bytes": (c_size_t, []),
        "ffn_sparse_debug_waits": (c_int32, [c_void_p, ctypes.c_uint32, ctypes.c_uint32, c_void_p]),
        "ffn_sparse_moe_workspace_bytes": (c_size_t, [P(Config), c_int32, c_int32]),
        "ffn_sparse_backward_workspace_bytes": (c_size_t, [P(Config), c_int32]),
        "ffn_sparse_backward": (c_int32, [c_void_p, c_void_p, c_int32, c_void_p, c_float, c_void_p, P(Pack),
                                          c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t,
                                          c_void_p]),
        "ffn_sparse_moe_forward": (c_int32, [P(c_void_p), c_int32, c_void_p, c_int32, c_int32, P(c_int32),
                                             P(c_float), c_void_p, c_float, c_void_p, c_int32, c_int32,
                                             c_void_p, c_size_t, c_void_p, c_void_p]),
        "ffn_gsi_check_config": (c_int32, [P(GsiConfig)]),
        "ffn_gsi_workspace_bytes": (c_size_t, [P(GsiConfig)]),
        "ffn_gsi_init": (c_int32, [P(GsiConfig), c_void_p, c_void_p, c_void_p, c_size_t, c_void_p,
                                   P(c_void_p)]),
        "ffn_gsi_forward": (c_int32, [c_void_p, c_void_p, c_int32, c_float, c_void_p, c_void_p, c_void_p,
                                      c_void_p, c_void_p]),
        "ffn_gsi_dense_forward": (c_int32, [c_void_p, c_void_p, c_int32, c_void_p, c_void_p]),
        "ffn_gsi_image": (c_void_p, [c_void_p]),
        "ffn_gsi_timing_enable": (c_int32, [c_void_p, c_int32, c_int32]),
        "ffn_gsi_timing_read": (c_int32, [c_void_p, c_int32, P(c_int32), P(c_double)]),
        "ffn_gsi_destroy": (None, [c_void_p]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _LIB = lib
    return lib


def status_string(status: int) -> str:
    try:
        return load().ffn_sparse_status_string(status).decode()
    except Exception:
        return "status"


def check(status: int, where: str) -> None:
    if status != FFN_OK:
        raise FFNError(status, where)
