"""Python binding of the sparse gated FFN library.

Argument marshalling only: PyTorch provides device memory and the current
stream, and every step of the computation runs in the HIP kernels behind the
C ABI (include/ffn_sparse.h). Method names follow the C entry points.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass

import torch

from . import _lib
from ._lib import Config, Pack, check


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream_ptr(stream=None) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


@dataclass
class TwellPack:
    """Device tensors of one TwELL pack (layout documented in the C header)."""
    cnt: torch.Tensor
    idx: torch.Tensor
    val: torch.Tensor
    route: torch.Tensor
    dense_list: torch.Tensor
    n_dense: torch.Tensor

    def c_struct(self) -> Pack:
        return Pack(self.cnt.data_ptr(), self.idx.data_ptr(), self.val.data_ptr(),
                    self.route.data_ptr(), self.dense_list.data_ptr(), self.n_dense.data_ptr())


class SparseFFN:
    """One FFN layer bound to borrowed device weights and an owned workspace.

    Weights: w_gate [d_ff, d_model] (rank 0) or u [d_ff, rank] + v [rank, d_model];
    w_up [d_ff, d_model]; w_down [d_model, d_ff] (wdown_out_major) or
    [d_ff, d_model]. dtype 'bf16' tensors are torch.bfloat16, 'f32' torch.float32.
    """

    def __init__(self, *, d_model: int, d_ff: int, w_up: torch.Tensor, w_down: torch.Tensor,
                 tile_w: int, ell_w: int, max_m: int, rank: int = 0, dtype: str = "bf16",
                 act: str = "relu", sel: str = "bias", w_gate: torch.Tensor | None = None,
                 u: torch.Tensor | None = None, v: torch.Tensor | None = None,
                 wdown_out_major: bool = True, in_keep: int = 0, stream=None):
        self.lib = _lib.load()
        self.cfg = Config(d_model, d_ff, rank, _lib.DTYPES[dtype], _lib.ACTS[act], _lib.SELS[sel],
                          tile_w, ell_w, 1 if wdown_out_major else 0, max_m, in_keep)
        check(self.lib.ffn_sparse_check_config(ctypes.byref(self.cfg)), "ffn_sparse_check_config")
        self.dtype = dtype
        self.torch_dtype = torch.bfloat16 if dtype == "bf16" else torch.float32
        self.device = w_up.device
        self._weights = (w_gate, u, v, w_up, w_down)   # borrowed by the library: keep alive
        nbytes = self.lib.ffn_sparse_workspace_bytes(ctypes.byref(self.cfg))
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        h = ctypes.c_void_p()
        gate = w_gate if rank == 0 else u
        check(self.lib.ffn_sparse_init(ctypes.byref(self.cfg), _ptr(gate), _ptr(v), _ptr(w_up),
                                       _ptr(w_down), self.workspace.data_ptr(), nbytes,
                                       _stream_ptr(stream), ctypes.byref(h)), "ffn_sparse_init")
        self.handle = h

    # ------------------------------------------------------------------ buffers
    @property
    def ntiles(self) -> int:
        return self.cfg.d_ff // self.cfg.tile_w

    def new_pack(self, m: int) -> TwellPack:
        dev, nt, E = self.device, self.ntiles, self.cfg.ell_w
        m1 = max(m, 1)
        return TwellPack(
            cnt=torch.empty((m1, nt), dtype=torch.int32, device=dev),
            idx=torch.empty((m1, nt, max(E, 1)), dtype=torch.int16, device=dev),
            val=torch.empty((m1, nt, max(E, 1)), dtype=self.torch_dtype, device=dev),
            route=torch.empty((m1,), dtype=torch.uint8, device=dev),
            dense_list=torch.empty((m1,), dtype=torch.int32, device=dev),
            n_dense=torch.empty((1,), dtype=torch.int32, device=dev))

    def new_output(self, m: int) -> torch.Tensor:
        return torch.empty((max(m, 1), self.cfg.d_model), dtype=self.torch_dtype, device=self.device)

    # ------------------------------------------------------------------ entry points
    def gate_pack(self, x, m=None, *, bias=None, bias_scalar=0.0, tau=None, k=0, pack=None,
                  g_debug=None, s_debug=None, stream=None) -> TwellPack:
        m = x.shape[0] if m is None else m
        pack = self.new_pack(m) if pack is None else pack
        ps = pack.c_struct()
        check(self.lib.ffn_sparse_gate_pack(self.handle, _ptr(x), m, _ptr(bias), float(bias_scalar),
                                            _ptr(tau), int(k), ctypes.byref(ps), _ptr(g_debug),
                                            _ptr(s_debug), _stream_ptr(stream)), "ffn_sparse_gate_pack")
        return pack

    def updown(self, x, pack: TwellPack, y=None, m=None, stream=None) -> torch.Tensor:
        m = x.shape[0] if m is None else m
        y = self.new_output(m) if y is None else y
        ps = pack.c_struct()
        check(self.lib.ffn_sparse_updown(self.handle, _ptr(x), m, ctypes.byref(ps), _ptr(y),
                                         _stream_ptr(stream)), "ffn_sparse_updown")
        return y

    def dense_fallback(self, x, pack: TwellPack, y, m=None, *, bias=None, bias_scalar=0.0, tau=None,
                       k=0, stream=None) -> torch.Tensor:
        m = x.shape[0] if m is None else m
        ps = pack.c_struct()
        check(self.lib.ffn_sparse_dense_fallback(self.handle, _ptr(x), m, _ptr(bias), float(bias_scalar),
                                                 _ptr(tau), int(k), ctypes.byref(ps), _ptr(y),
                                                 _stream_ptr(stream)), "ffn_sparse_dense_fallback")
        return y

    def backward(self, x, dy, pack: TwellPack, m=None, *, bias=None, bias_scalar=0.0, tau=None, dx=None,
                 dw_gate=None, dw_up=None, dw_down_nm=None, workspace=None, stream=None):
        """Gradients of <dy, y> through the forward pass that wrote `pack`
        (ffn_sparse_backward). dx is written (allocated here unless given);
        the fp32 weight-gradient buffers [d_ff, d_model] are added to when given."""
        m = x.shape[0] if m is None else m
        if dx is None:
            dx = torch.empty((max(m, 1), self.cfg.d_model), dtype=self.torch_dtype, device=self.device)
        if workspace is None:
            nb = self.lib.ffn_sparse_backward_workspace_bytes(ctypes.byref(self.cfg), max(m, 1))
            workspace = torch.empty(max(nb, 256), dtype=torch.uint8, device=self.device)
        ps = pack.c_struct()
        check(self.lib.ffn_sparse_backward(self.handle, _ptr(x), m, _ptr(bias), float(bias_scalar), _ptr(tau),
                                           ctypes.byref(ps), _ptr(dy), _ptr(dx), _ptr(dw_gate), _ptr(dw_up),
                                           _ptr(dw_down_nm), workspace.data_ptr(), workspace.numel(),
                                           _stream_ptr(stream)), "ffn_sparse_backward")
        return dx

    def forward(self, x, m=None, *, bias=None, bias_scalar=0.0, tau=None, k=0, pack=None, y=None,
                stream=None):
        m = x.shape[0] if m is None else m
        pack = self.new_pack(m) if pack is None else pack
        y = self.new_output(m) if y is None else y
        ps = pack.c_struct()
        check(self.lib.ffn_sparse_forward(self.handle, _ptr(x), m, _ptr(bias), float(bias_scalar),
                                          _ptr(tau), int(k), ctypes.byref(ps), _ptr(y),
                                          _stream_ptr(stream)), "ffn_sparse_forward")
        return y, pack

    def forward_noalloc(self, x, pack: TwellPack, y, m=None, *, bias=None, bias_scalar=0.0, tau=None, k=0,
                        stream=None):
        """forward() through the allocation-free entry point: the caller passes
        the pack and y; the library's per-GPU scratch array holds the rest."""
        m = x.shape[0] if m is None else m
        ps = pack.c_struct()
        check(self.lib.ffn_sparse_forward_noalloc(self.handle, _ptr(x), m, _ptr(bias), float(bias_scalar),
                                                  _ptr(tau), int(k), ctypes.byref(ps), _ptr(y),
                                                  _stream_ptr(stream)), "ffn_sparse_forward_noalloc")
        return y, pack

    def dense_forward(self, x, m=None, *, bias=None, bias_scalar=0.0, tau=None, y=None, stream=None):
        m = x.shape[0] if m is None else m
        y = self.new_output(m) if y is None else y
        check(self.lib.ffn_sparse_dense_forward(self.handle, _ptr(x), m, _ptr(bias), float(bias_scalar),
                                                _ptr(tau), _ptr(y), _stream_ptr(stream)),
              "ffn_sparse_dense_forward")
        return y

    def forward_path(self, m: int) -> str:
        """Kernel sequence forward() runs for m tokens: 'general',
        'decode-chunk' / 'decode-part' / 'decode-split', (top-k selection)
        'topk-list' / 'topk-masked-dense', 'input-gate' (input-side gate
        selection) or 'masked-dense' (17..127 tokens, up to 256 for packs the
        XCD-sliced kernels cannot hold; see the C header)."""
        r = self.lib.ffn_sparse_forward_path(self.handle, int(m))
        if r < 0:
            raise ValueError(f"invalid token count {m}")
        return {0: "general", 1: "decode-chunk", 2: "decode-part", 3: "decode-split",
                4: "topk-list", 5: "topk-masked-dense", 6: "input-gate", 7: "masked-dense"}[r]

    def device_status(self, stream=None) -> int:
        """FFN_OK, or FFN_E_HIP when a launch failed or a bounded wait gave up
        (synchronises the stream; see ffn_sparse_device_status)."""
        return self.lib.ffn_sparse_device_status(self.handle, _stream_ptr(stream))

    def debug_waits(self, epoch_skew: int, spin_limit: int, stream=None) -> None:
        check(self.lib.ffn_sparse_debug_waits(self.handle, int(epoch_skew), int(spin_limit), _stream_ptr(stream)),
              "ffn_sparse_debug_waits")

    def reinit(self, stream=None) -> None:
        """Re-initialise the handle on the same weights and workspace."""
        w_gate, u, v, w_up, w_down = self._weights
        self.close()
        h = ctypes.c_void_p()
        gate = w_gate if self.cfg.rank == 0 else u
        check(self.lib.ffn_sparse_init(ctypes.byref(self.cfg), _ptr(gate), _ptr(v), _ptr(w_up), _ptr(w_down),
                                       self.workspace.data_ptr(), self.workspace.numel(), _stream_ptr(stream),
                                       ctypes.byref(h)), "ffn_sparse_init")
        self.handle = h

    # ------------------------------------------------------------------ timing
    def timing_enable(self, enable: bool = True, capacity: int = 4096) -> None:
        check(self.lib.ffn_sparse_timing_enable(self.handle, 1 if enable else 0, capacity),
              "ffn_sparse_timing_enable")

    def timing_read(self, kind: str) -> tuple[int, float]:
        n = ctypes.c_int32()
        ms = ctypes.c_double()
        check(self.lib.ffn_sparse_timing_read(self.handle, _lib.KERNEL_KINDS[kind], ctypes.byref(n),
                                              ctypes.byref(ms)), "ffn_sparse_timing_read")
        return n.value, ms.value

    def close(self) -> None:
        if getattr(self, "handle", None):
            self.lib.ffn_sparse_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def moe_forward(experts, x, expert_ids, weights, *, tau=None, bias=None, bias_scalar=0.0, k=0, y=None,
                workspace=None, dense=False, stream=None) -> torch.Tensor:
    """Mixture-of-experts layer over SparseFFN experts of one shape
    (ffn_sparse_moe_forward). expert_ids and weights are host arrays
    [m, topk] (numpy or lists); tau / bias device tensors [m, topk] or None."""
    import numpy as np
    lib = experts[0].lib
    ids = np.ascontiguousarray(np.asarray(expert_ids, dtype=np.int32))
    wts = np.ascontiguousarray(np.asarray(weights, dtype=np.float32))
    m, topk = ids.shape
    cfg = experts[0].cfg
    if y is None:
        y = torch.empty((max(m, 1), cfg.d_model), dtype=experts[0].torch_dtype, device=experts[0].device)
    nbytes = lib.ffn_sparse_moe_workspace_bytes(ctypes.byref(cfg), max(m, 1), topk)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=experts[0].device)
    hs = (ctypes.c_void_p * len(experts))(*[e.handle.value for e in experts])
    check(lib.ffn_sparse_moe_forward(hs, len(experts), _ptr(x), m, topk,
                                     ids.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                     wts.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), _ptr(bias),
                                     float(bias_scalar), _ptr(tau), int(k), 1 if dense else 0, workspace.data_ptr(),
                                     workspace.numel(), _ptr(y), _stream_ptr(stream)), "ffn_sparse_moe_forward")
    return y
