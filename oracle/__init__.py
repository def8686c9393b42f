"""Float64 CPU oracle for the theta-bundle projection (test infrastructure only).

Only the test suite, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg may import this package.  It shares no code with the HIP
library.
"""

from .theta_bundle import (  # noqa: F401
    band_sizes,
    band_map,
    band_index,
    bf16_bits_to_f64,
    reconstruct_weight,
    forward,
    forward_dense,
    relative_frobenius_error,
    mean_error,
    shared_block,
    row_scale,
    truncated_factors,
    orthonormal_basis,
    randomized_factors,
    decompose,
    ATTENTION_FAMILIES,
    MLP_FAMILIES,
    decompose_model,
    refine_shared_block,
    als_decompose,
    decomposition_error,
)
