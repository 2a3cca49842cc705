"""MI355X-native RWKV-6 WKV forward operator.

The computation runs in hand-written HIP kernels for gfx950 inside
``libwkv6.so`` (C ABI declared in ``include/wkv6.h``).  This package holds
the thin ctypes binding (``linear_attention_rnn_amd.wkv6``), the build step
(``linear_attention_rnn_amd.build``) and the seeded synthetic-input generator
(``linear_attention_rnn_amd.inputs``).  Importing the package does not load
the library; the binding loads it on first use and raises if it is missing.
"""

__all__ = ["inputs", "wkv6", "build"]
