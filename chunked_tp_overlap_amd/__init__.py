"""MI355X-native chunked tensor-parallel overlap GEMMs over a capacity UserBuffer.

The hot path lives in a C-ABI shared library (``include/ub.h``) built from the HIP and
C++ sources under ``csrc/``.  ``chunked_tp_overlap_amd.ub`` is the thin ctypes binding
with the same entry-point names; ``chunked_tp_overlap_amd.workloads`` draws seeded
synthetic inputs.  Importing this package loads nothing: the library is opened on first
use of the binding, and an import of the binding fails loudly when it is not built.
"""

__all__ = ["ub", "workloads"]
