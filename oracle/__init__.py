"""fp64 CPU oracle for the Gated DeltaNet recurrent forward (test infrastructure only)."""
from .oracle import (gdn_backward, gdn_forward, gdn_forward_fused, preprocess, preprocess_backward,  # noqa: F401
                     short_conv, short_conv_backward, build, max_threads)
