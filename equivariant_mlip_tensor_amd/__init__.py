"""MI355X-native Clebsch-Gordan tensor-product convolution.

The library is ``libtpconv.so`` (C ABI in ``include/tpconv.h``); ``tpconv``
is its ctypes binding.  Build with ``python -m equivariant_mlip_tensor_amd.build``.
"""

__all__ = ["tpconv"]
