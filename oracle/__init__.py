"""CPU fp64 oracle for the quintic Newton–Schulz orthogonalization.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this package:
only the test suite, the smoke check and the CPU-baseline leg of the
benchmark may call it.  It shares no code with the HIP library.
"""

from .ns_oracle import (  # noqa: F401
    DEFAULT_COEFFS,
    DEFAULT_STEPS,
    EPS,
    frobenius_normalize,
    ns_iteration,
    gram_matrix,
    poly_matrix,
    apply_update,
    newton_schulz,
    newton_schulz_batched,
    dense_equivalent_flops,
)
