"""MoGA (Mixture-of-Groups Attention) forward path for AMD MI355X (gfx950).

The compute runs in hand-written HIP kernels behind the C ABI declared in
include/moga.h (libmoga.so, built in this directory).  This package is the
thin Python binding: it checks tensors, marshals pointers and the current
stream, and calls the library.  There is no CPU or PyTorch fallback: if the
library is missing every entry point raises.
"""
from .metrics import attention_flops, moga_pairs  # noqa: F401

__all__ = ["attention_flops", "moga_pairs"]
