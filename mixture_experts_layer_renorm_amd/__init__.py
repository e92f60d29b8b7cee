"""MI355X-native forward pass of a sparse Mixture-of-Experts feed-forward layer.

The computation runs in hand-written HIP kernels for gfx950 behind the C ABI declared in
``include/moe.h`` (library ``libmoe.so``).  This package holds the thin ctypes binding to that
library (``abi``), the seeded synthetic-layer generator (``synth``) and the analytic cost model
used for roofline reporting (``costmodel``).
"""

__all__ = ["abi", "synth", "costmodel"]
