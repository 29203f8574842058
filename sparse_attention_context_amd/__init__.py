"""MI355X-native In-context Sparse Attention (ISA) forward hot path.

The compute lives in hand-written HIP kernels for gfx950 behind the C-ABI
library ``libisa.so`` (declared in include/isa.h).  ``isa`` is the thin
ctypes binding to it; ``synth`` draws seeded synthetic inputs and
``configs`` lists the benchmark workloads.  Importing the package does not
load the library; the first call through ``isa`` does, and raises if the
library has not been built.
"""

__all__ = ["isa", "synth", "configs"]
