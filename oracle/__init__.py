"""fp64 CPU oracle for the MRU prefix-scan path (test infrastructure only).

Imported by tests, the smoke check and the benchmark's CPU-baseline leg; never
by the product path.  See ``mru_oracle`` for the definitions and citations.
"""
from .mru_oracle import (  # noqa: F401
    FP32_DOMAIN_LIMIT,
    ORTHO_METHODS,
    build_orthogonal_ref,
    build_ref,
    build_vjp_ref,
    bwd_ref,
    flatten_ref,
    loss_ref,
    rel_fro_err,
    representable,
    scaled_ref,
    scan_ref,
)
