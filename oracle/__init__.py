"""fp64 CPU oracle of the MLA forward hot path.

Test infrastructure only: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the library or its binding.
"""
from .mla_oracle import (  # noqa: F401
    rope_theta, rope_rotate, weight_slices, visibility_mask, explicit_fwd,
    absorbed_fwd, decode_absorbed, lse_merge, chunk_bounds, brute_force_explicit,
)
