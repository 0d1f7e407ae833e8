"""Collective KV-cache reuse kernels for AMD MI355X (gfx950).

The compute lives in ``libtdx.so`` (hand-written HIP); ``tdx`` is its ctypes
binding.  ``build`` compiles the library in-tree with hipcc.
"""

from . import tdx  # noqa: F401
