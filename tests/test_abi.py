"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every entry point include/vsa.h declares, sizes its buffers, and rejects bad
arguments with the documented status before touching the GPU."""
import ctypes
import os
import re

import pytest

from trainable_block_sparse_cube_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vsa.h")

OK, INVALID, UNSUPPORTED, WORKSPACE = (_lib.VSA_OK, _lib.VSA_ERR_INVALID_ARG,
                                       _lib.VSA_ERR_UNSUPPORTED, _lib.VSA_ERR_WORKSPACE)


def declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\**\s+\**([A-Za-z_][A-Za-z0-9_]*)\s*\(",
                       text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("libvsa.so not built")
    return _lib.load()


def test_header_declares_the_required_entry_points():
    names = declared_functions()
    for need in ("vsa_forward", "vsa_backward", "block_sparse_attn_varlen",
                 "block_sparse_attn_varlen_backward", "vsa_forward_workspace_bytes",
                 "vsa_backward_workspace_bytes", "vsa_saved_bytes", "vsa_status_string",
                 "vsa_cube_permute_pool", "vsa_coarse_topk", "vsa_fine_forward",
                 "vsa_forward_mass", "vsa_forward_mass_workspace_bytes", "vsa_coarse_select_mass",
                 "vsa_pack_lists", "vsa_cube_max_pool", "vsa_fine_order", "vsa_validate_lists"):
        assert need in names


def test_library_exports_every_declared_symbol(lib):
    names = declared_functions()
    for name in names:
        assert hasattr(lib, name), name
        assert name in _lib.SIGNATURES, f"{name} missing from the Python binding"


def test_status_strings(lib):
    for s in range(5):
        assert lib.vsa_status_string(s)
    assert lib.vsa_status_string(99) == b"unknown status"


def test_workspace_sizes(lib):
    # forward: K and V bf16 tile copies + three fp32 means + coarse output/lse
    B, nh, D, T, H, W = 1, 12, 128, 20, 48, 64
    N, nc = T * H * W, T * H * W // 64
    fw = lib.vsa_forward_workspace_bytes(B, nh, D, T, H, W, _lib.VSA_BF16)
    assert fw >= 2 * B * nh * N * D * 2 + 4 * B * nh * nc * D * 4
    sv = lib.vsa_saved_bytes(B, nh, D, T, H, W, _lib.VSA_BF16)
    # coarse output, both log-sum-exps, fine output; K and V tiles; three means
    assert sv >= 4 * (B * nh * nc * D + B * nh * nc + B * nh * N + B * nh * N * D) \
        + 2 * 2 * B * nh * N * D + 3 * 4 * B * nh * nc * D
    sv32 = lib.vsa_saved_bytes(B, nh, D, T, H, W, _lib.VSA_F32)
    assert sv32 >= sv + 2 * 2 * B * nh * N * D
    assert lib.vsa_saved_bytes(B, nh, D, T, H, W, 7) == 0
    bw = lib.vsa_backward_workspace_bytes(B, nh, D, T, H, W, _lib.VSA_BF16, B * nh * nc * 32)
    assert bw > fw
    # the coarse stage holds at most 3584 cubes (8 rows of logits in LDS,
    # 56 chunks of 64 per row in registers)
    assert lib.vsa_forward_workspace_bytes(1, 1, 128, 4, 4, 4 * 3584, _lib.VSA_BF16) > 0
    assert lib.vsa_forward_workspace_bytes(1, 1, 128, 4, 4, 4 * 3585, _lib.VSA_BF16) == 0
    # invalid shapes size to 0
    assert lib.vsa_forward_workspace_bytes(B, nh, D, 6, H, W, _lib.VSA_BF16) == 0
    assert lib.vsa_forward_workspace_bytes(B, nh, 96, T, H, W, _lib.VSA_BF16) == 0
    assert lib.vsa_backward_workspace_bytes(B, nh, D, T, H, W, _lib.VSA_BF16, -1) == 0


FAKE = 0x1000  # a non-null pointer value; never dereferenced by failing calls


def fwd(lib, T=8, H=8, W=8, D=64, topk=2, dtype=_lib.VSA_BF16, null_out=False, ws=FAKE, ws_bytes=1 << 40):
    return lib.vsa_forward(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 2, D, T, H, W, topk, dtype,
                           None if null_out else FAKE, FAKE, None, ws, ws_bytes, None)


def test_saved_state_size_follows_the_element_type():
    """The forward keeps its K and V tiles in the saved state, so its size
    grows with the element size (host only: no GPU work)."""
    import torch
    from trainable_block_sparse_cube_amd import ops
    B, nh, D, grid = 1, 2, 64, (8, 8, 8)
    N = 8 * 8 * 8
    bf, f32 = ops.saved_bytes(B, nh, D, grid, torch.bfloat16), ops.saved_bytes(B, nh, D, grid, torch.float32)
    assert f32 - bf >= 2 * 2 * B * nh * N * D  # two tiles, 2 more bytes per element
    with pytest.raises(TypeError):
        ops.saved_bytes(B, nh, D, grid, torch.float16)


def test_forward_rejects_bad_arguments(lib):
    assert fwd(lib, T=6) == INVALID          # grid not made of 4x4x4 cubes
    assert fwd(lib, H=0) == INVALID
    assert fwd(lib, topk=0) == INVALID
    assert fwd(lib, topk=9) == INVALID       # 8 cubes
    assert fwd(lib, D=96) == UNSUPPORTED
    assert fwd(lib, dtype=7) == UNSUPPORTED
    assert fwd(lib, null_out=True) == INVALID
    assert fwd(lib, ws=None) == INVALID
    assert fwd(lib, ws_bytes=16) == WORKSPACE
    # B * heads is a grid dimension: at most 65535 (batch, head) pairs
    assert lib.vsa_forward(FAKE, FAKE, FAKE, FAKE, FAKE, 256, 256, 64, 8, 8, 8, 2, _lib.VSA_BF16,
                           FAKE, FAKE, None, FAKE, 1 << 40, None) == UNSUPPORTED
    # (batch, head, cube) units: at most 2^24 - 8 (1-D grids of 256-thread
    # workgroups); 65535 pairs of 256 cubes pass, of 257 do not
    assert lib.vsa_forward_workspace_bytes(1, 65535, 64, 4, 16, 256, _lib.VSA_BF16) > 0
    assert lib.vsa_forward_workspace_bytes(1, 65535, 64, 4, 4, 4 * 257, _lib.VSA_BF16) == 0
    assert lib.vsa_forward(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 65535, 64, 4, 4, 4 * 257, 2, _lib.VSA_BF16,
                           FAKE, FAKE, None, FAKE, 1 << 60, None) == UNSUPPORTED


def test_varlen_and_backward_reject_bad_arguments(lib):
    st = lib.block_sparse_attn_varlen(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 2, 64, 8, 8, 8,
                                      None, FAKE, 4, _lib.VSA_BF16, FAKE, None, FAKE, 1 << 40, None)
    assert st == INVALID  # no offsets
    st = lib.block_sparse_attn_varlen(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 2, 64, 8, 8, 8,
                                      FAKE, FAKE, -1, _lib.VSA_BF16, FAKE, None, FAKE, 1 << 40, None)
    assert st == INVALID  # negative entry count
    st = lib.vsa_backward(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 1, 2, 64, 8, 8, 8, 2,
                          _lib.VSA_BF16, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40, None)
    assert st == INVALID  # no saved state
    st = lib.vsa_backward(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 2, 64, 8, 8, 8, 2,
                          _lib.VSA_F32, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 16, None)
    assert st == WORKSPACE  # fp32 is accepted: it gets as far as the workspace check
    st = lib.vsa_backward(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 2, 64, 8, 8, 8, 2,
                          7, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40, None)
    assert st == UNSUPPORTED  # unknown dtype
    st = lib.vsa_backward(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 2, 64, 8, 8, 8, 2,
                          _lib.VSA_BF16, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 16, None)
    assert st == WORKSPACE


def test_stage_calls_reject_bad_arguments(lib):
    BF = _lib.VSA_BF16
    assert lib.vsa_coarse_topk(FAKE, FAKE, FAKE, 1, 1, 64, 8, 9, BF, FAKE, FAKE, FAKE, None) == INVALID
    assert lib.vsa_coarse_topk(FAKE, FAKE, FAKE, 1, 1, 64, 8, 2, BF, FAKE, FAKE, None, None) == INVALID
    assert lib.vsa_coarse_topk(FAKE, FAKE, FAKE, 1, 1, 64, 8, 2, 7, FAKE, FAKE, FAKE, None) == INVALID
    assert lib.vsa_coarse_topk(FAKE, FAKE, FAKE, 1, 1, 64, 100000, 2, BF, FAKE, FAKE, FAKE,
                               None) == UNSUPPORTED
    assert lib.vsa_fine_forward(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 64, 8, 8, 8,
                                None, FAKE, 0, 2, _lib.VSA_BF16, FAKE, FAKE, None, None, None) == INVALID
    # CSR lists: a negative entry count, or more entries than every list full
    assert lib.vsa_fine_forward(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 64, 8, 8, 8,
                                FAKE, FAKE, -1, 0, _lib.VSA_BF16, FAKE, None, None, None, None) == INVALID
    assert lib.vsa_fine_forward(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 64, 8, 8, 8,
                                FAKE, FAKE, 65, 0, _lib.VSA_BF16, FAKE, None, None, None, None) == INVALID
    assert lib.vsa_fine_order(None, FAKE, 0, 0, 1, 1, 8, FAKE, None) == INVALID  # topk 0 without offsets
    assert lib.vsa_fine_order(None, FAKE, 0, 2, 1, 1, 8, None, None) == INVALID
    assert lib.vsa_fine_order(FAKE, FAKE, 10, 0, 1, 1, 5000, FAKE, None) == UNSUPPORTED
    assert lib.vsa_fine_order(FAKE, FAKE, 65, 0, 1, 1, 8, FAKE, None) == INVALID
    assert lib.vsa_cube_permute_pool(FAKE, FAKE, FAKE, 1, 1, 64, 8, 8, 5, _lib.VSA_BF16,
                                     FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == INVALID


def test_mass_rule_calls_reject_bad_arguments(lib):
    BF = _lib.VSA_BF16
    B, nh, D, T, H, W = 1, 2, 64, 8, 8, 8  # 8 cubes
    fw = lib.vsa_forward_workspace_bytes(B, nh, D, T, H, W, BF)
    mw = lib.vsa_forward_mass_workspace_bytes(B, nh, D, T, H, W, BF, 4)
    # forward workspace + B*heads*Nc counts + B*heads*Nc*k_max padded ids
    assert mw >= fw + 4 * (B * nh * 8) + 4 * (B * nh * 8 * 4)
    assert lib.vsa_forward_mass_workspace_bytes(B, nh, D, T, H, W, BF, 0) == 0
    assert lib.vsa_forward_mass_workspace_bytes(B, nh, D, T, H, W, BF, 9) == 0  # k_max > Nc

    def fwd(mass, k_min, k_max, ws=1 << 40, offs=FAKE, ids=FAKE):
        return lib.vsa_forward_mass(FAKE, FAKE, FAKE, FAKE, FAKE, B, nh, D, T, H, W, mass, k_min,
                                    k_max, BF, FAKE, offs, ids, None, FAKE, ws, None)
    assert fwd(0.0, 1, 4) == INVALID
    assert fwd(1.5, 1, 4) == INVALID
    assert fwd(float("nan"), 1, 4) == INVALID
    assert fwd(0.5, 0, 4) == INVALID
    assert fwd(0.5, 5, 4) == INVALID
    assert fwd(0.5, 1, 9) == INVALID
    assert fwd(0.5, 1, 4, offs=None) == INVALID
    assert fwd(0.5, 1, 4, ids=None) == INVALID
    assert fwd(0.5, 1, 4, ws=16) == WORKSPACE

    def coarse(mass, k_min, k_max, dtype=BF, counts=FAKE):
        return lib.vsa_coarse_select_mass(FAKE, FAKE, FAKE, 1, 1, 64, 8, mass, k_min, k_max, dtype,
                                          FAKE, FAKE, counts, FAKE, None)
    assert coarse(0.5, 1, 9) == INVALID
    assert coarse(-0.1, 1, 4) == INVALID
    assert coarse(0.5, 1, 4, dtype=7) == INVALID
    assert coarse(0.5, 1, 4, counts=None) == INVALID
    assert lib.vsa_pack_lists(FAKE, FAKE, -1, 4, FAKE, FAKE, None) == INVALID
    assert lib.vsa_pack_lists(FAKE, FAKE, 4, 0, FAKE, FAKE, None) == INVALID
    assert lib.vsa_pack_lists(FAKE, FAKE, 4, 4, None, FAKE, None) == INVALID
    assert lib.vsa_pack_lists(FAKE, FAKE, 1 << 20, 1 << 12, FAKE, FAKE, None) == UNSUPPORTED
    assert lib.vsa_cube_max_pool(FAKE, FAKE, FAKE, 1, 1, 64, 8, 8, 6, BF, FAKE, FAKE, FAKE, None) == INVALID
    assert lib.vsa_cube_max_pool(FAKE, FAKE, FAKE, 1, 1, 64, 8, 8, 8, BF, FAKE, None, FAKE, None) == INVALID


def test_validate_lists_rejects_bad_arguments(lib):
    v = lib.vsa_validate_lists
    assert v(FAKE, FAKE, 10, 0, 4, 8, None, None) == INVALID      # no result buffer
    assert v(FAKE, FAKE, 10, 0, -1, 8, FAKE, None) == INVALID     # negative row count
    assert v(FAKE, FAKE, 10, 0, 4, 0, FAKE, None) == INVALID      # no cubes
    assert v(FAKE, FAKE, -1, 0, 4, 8, FAKE, None) == INVALID      # negative entry count
    assert v(FAKE, None, 10, 0, 4, 8, FAKE, None) == INVALID      # entries but no ids
    assert v(FAKE, FAKE, 10, 0, 4, 5000, FAKE, None) == UNSUPPORTED
    # fixed length: n_list_entries must be n_rows * topk
    assert v(None, FAKE, 10, 3, 4, 8, FAKE, None) == INVALID
    assert v(None, FAKE, 12, 0, 4, 8, FAKE, None) == INVALID
