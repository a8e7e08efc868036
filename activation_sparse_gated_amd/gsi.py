"""Python binding of the gated subspace (GSI) linear map (include/ffn_gsi.h).

Argument marshalling only: PyTorch provides device memory and the current
stream; every step runs in the HIP kernels behind the C ABI. Method names
follow the C entry points.
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib
from ._lib import GsiConfig, check


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream_ptr(stream=None) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


class GsiLinear:
    """y = W x with the gated subspace fast path, bound to borrowed bf16 device
    tensors w [d_out, d_in] and vk [d_in, k] and an owned workspace."""

    def __init__(self, w: torch.Tensor, vk: torch.Tensor, *, max_m: int, stream=None):
        self.lib = _lib.load()
        d_out, d_in = w.shape
        self.cfg = GsiConfig(d_in, d_out, vk.shape[1], max_m)
        check(self.lib.ffn_gsi_check_config(ctypes.byref(self.cfg)), "ffn_gsi_check_config")
        self.device = w.device
        self._weights = (w, vk)          # borrowed by the library: keep alive
        nbytes = self.lib.ffn_gsi_workspace_bytes(ctypes.byref(self.cfg))
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        h = ctypes.c_void_p()
        check(self.lib.ffn_gsi_init(ctypes.byref(self.cfg), _ptr(w), _ptr(vk), self.workspace.data_ptr(), nbytes,
                                    _stream_ptr(stream), ctypes.byref(h)), "ffn_gsi_init")
        self.handle = h

    def new_output(self, m: int) -> torch.Tensor:
        return torch.empty((max(m, 1), self.cfg.d_out), dtype=torch.bfloat16, device=self.device)

    def forward(self, x, eps: float, m=None, *, y=None, rho=None, slow_list=None, n_slow=None, stream=None):
        """Returns (y, rho, slow_list, n_slow); the last three are device
        tensors allocated here unless passed in."""
        m = x.shape[0] if m is None else m
        y = self.new_output(m) if y is None else y
        dev = self.device
        rho = torch.empty((max(m, 1),), dtype=torch.float32, device=dev) if rho is None else rho
        slow_list = torch.empty((max(m, 1),), dtype=torch.int32, device=dev) if slow_list is None else slow_list
        n_slow = torch.empty((4,), dtype=torch.int32, device=dev) if n_slow is None else n_slow
        check(self.lib.ffn_gsi_forward(self.handle, _ptr(x), m, float(eps), _ptr(y), _ptr(rho), _ptr(slow_list),
                                       _ptr(n_slow), _stream_ptr(stream)), "ffn_gsi_forward")
        return y, rho, slow_list, n_slow

    def forward_raw(self, x, eps: float, y, m=None, rho=None, slow_list=None, n_slow=None, stream=None) -> int:
        """The C call with caller buffers (any of rho / slow_list / n_slow may be None); returns the status."""
        m = x.shape[0] if m is None else m
        return self.lib.ffn_gsi_forward(self.handle, _ptr(x), m, float(eps), _ptr(y), _ptr(rho), _ptr(slow_list),
                                        _ptr(n_slow), _stream_ptr(stream))

    def dense_forward(self, x, m=None, *, y=None, stream=None) -> torch.Tensor:
        m = x.shape[0] if m is None else m
        y = self.new_output(m) if y is None else y
        check(self.lib.ffn_gsi_dense_forward(self.handle, _ptr(x), m, _ptr(y), _stream_ptr(stream)),
              "ffn_gsi_dense_forward")
        return y

    def image(self) -> torch.Tensor:
        """The cached image M = W V_k [d_out, k] (bf16) as a view of the workspace."""
        addr = self.lib.ffn_gsi_image(self.handle)
        off = addr - self.workspace.data_ptr()
        n = self.cfg.d_out * self.cfg.k * 2
        return self.workspace[off:off + n].view(torch.bfloat16).view(self.cfg.d_out, self.cfg.k)

    def timing_enable(self, enable: bool = True, capacity: int = 4096) -> None:
        check(self.lib.ffn_gsi_timing_enable(self.handle, 1 if enable else 0, capacity), "ffn_gsi_timing_enable")

    def timing_read(self, kind: str):
        n, ms = ctypes.c_int32(), ctypes.c_double()
        check(self.lib.ffn_gsi_timing_read(self.handle, _lib.GSI_KERNEL_KINDS[kind], ctypes.byref(n),
                                           ctypes.byref(ms)), "ffn_gsi_timing_read")
        return n.value, ms.value

    def close(self) -> None:
        if getattr(self, "handle", None) is not None and self.handle.value:
            self.lib.ffn_gsi_destroy(self.handle)
            self.handle = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
