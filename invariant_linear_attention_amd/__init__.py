"""MI355X (gfx950) batch-invariant Gated DeltaNet recurrent forward.

The compute lives in ``libgdn.so`` (HIP kernels behind the C ABI of include/gdn.h);
``gdn`` is its thin ctypes binding and ``synth`` draws seeded synthetic workloads.
Importing the package does not load the library; the first call does, and fails
loudly if it has not been built.
"""
from . import gdn  # noqa: F401
from .gdn import gdn_decode_step, gdn_fwd_varlen, load_library  # noqa: F401
