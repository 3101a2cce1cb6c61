"""fp64 CPU oracle for hierarchical video sparse attention.

Test infrastructure: only the tests, the package smoke check and the
benchmark's CPU-baseline leg use it.  It shares no code with the HIP path.
"""
from .vsa_oracle import (  # noqa: F401
    CUBE_TOKENS, backward, backward_sampled, coarse_attention, cube_attention_mass, cube_members,
    fine_attention,
    forward, forward_with_sets, lists_from_csr, lists_from_sel, pool,
    query_cube_output, select_mass, select_topk, token_cube_map,
)
