"""MI355X (gfx950) hierarchical video sparse attention: VSA and the
variable-length key lists of VSA2, as a C-ABI HIP library (libvsa.so) with
a thin PyTorch binding."""
from .ops import (  # noqa: F401
    block_sparse_attn_varlen, block_sparse_attn_varlen_attention, block_sparse_attn_varlen_backward,
    pack_lists,
    saved_bytes, vsa_backward, vsa_coarse_select_mass, vsa_coarse_topk, vsa_cube_max_pool,
    vsa_cube_permute_pool,
    vsa_attention, vsa_fine_forward, vsa_fine_order, vsa_forward, vsa_forward_mass, validate_lists,
)
