"""Activation-sparse gated FFN for AMD MI355X (gfx950).

The compute path is the HIP library libffn_sparse.so (C ABI in
include/ffn_sparse.h and include/ffn_gsi.h); this package only binds it. Importing works without a
GPU; calling an entry point needs the built library and a GPU.
"""
from ._lib import FFNError, load  # noqa: F401
from .ffn import SparseFFN, TwellPack, moe_forward  # noqa: F401
from .gsi import GsiLinear  # noqa: F401

__all__ = ["SparseFFN", "TwellPack", "GsiLinear", "moe_forward", "FFNError", "load"]
