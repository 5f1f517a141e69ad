"""MI355X (gfx950) causal prefill attention forward: FP8 e4m3 and BF16.

The compute path is the C-ABI library ``libattn_prefill.so`` (hand-written HIP
kernels, declared in ``include/attn_prefill.h``); ``ops`` is a thin ctypes
binding over it that passes raw device pointers and the current HIP stream.
Importing this package does not load the library; the first call does, and it
raises if the library has not been built.
"""

from .workloads import WORKLOADS, Workload, make_inputs  # noqa: F401

__all__ = ["WORKLOADS", "Workload", "make_inputs"]
