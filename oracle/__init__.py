"""fp64 CPU oracle for the Gated DeltaNet recurrent forward (test infrastructure only)."""
from .oracle import gdn_backward, gdn_forward, gdn_forward_fused, preprocess, short_conv, build, max_threads  # noqa: F401
