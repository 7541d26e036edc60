"""MI355X-native CSA2 sparse-attention layer.

The compute path is the HIP library ``libcsa2.so`` (hand-written gfx950
kernels behind a C ABI); :mod:`.binding` marshals arguments to it with
ctypes and :mod:`.workloads` prepares seeded synthetic inputs.  Importing
the package loads nothing; the library is opened on first use and a missing
library is an error, never a fallback.
"""

__all__ = ["binding", "workloads"]
