"""MI355X-native fused Transformer encoder layer (forward + backward).

The compute path is a C-ABI shared library (``libtel.so``) of hand-written
gfx950 HIP kernels; this package is its thin Python binding.  Importing the
package does not load the library: ``binding.lib()`` does, on first use, and
raises if the library has not been built.
"""
from . import synthetic  # noqa: F401

__all__ = ["synthetic"]
