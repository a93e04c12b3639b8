"""fp64 CPU oracle of fused linear cross-entropy (test infrastructure only).

Only the tests, the package entry point's smoke check and the benchmark's
CPU-baseline leg may import this package.  The GPU library never does.
"""
from .flce_oracle import (flce_reference, gradient_samples, row_argmax_ids, row_statistics,  # noqa: F401
                          streaming_reference, transform_derivative, transform_logits)
