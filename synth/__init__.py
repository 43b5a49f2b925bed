"""Seeded synthetic workloads for the lightning indexer.

Shared by the tests, the smoke check and the benchmark.  This package only
draws random inputs and marshals tensors to NumPy bit patterns; it holds
none of the indexer's arithmetic.
"""

from .workloads import (  # noqa: F401
    WORKLOADS,
    v4_inputs,
    v4_exact_inputs,
    v41_inputs,
    v41_exact_inputs,
    document_starts,
    upstream_gradient,
    bits,
)
