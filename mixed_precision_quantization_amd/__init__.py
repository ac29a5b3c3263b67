"""MI355X-native stochastic-computing (SC) bipolar XNOR matmul with dynamic
mixed precision.

The compute path is the C-ABI library ``libscmp.so`` (HIP kernels for gfx950,
declared in ``include/scmp.h``); ``scmp`` is its thin ctypes binding.  Import
``mixed_precision_quantization_amd.scmp`` to load the library; importing this
package alone loads nothing.
"""

__all__ = ["scmp", "workloads"]
