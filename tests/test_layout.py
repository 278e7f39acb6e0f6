"""Fragment order of the expert weights (a byte order the kernels read as whole cache lines): the
CPU reference's two forms agree with each other and with hand positions, the order is a bijection,
and the ABI rejects bad sizes and pointers before touching a device."""
import ctypes

import numpy as np
import pytest

import sparse_moe_layer_top_amd as bm
from sparse_moe_layer_top_amd import binding as B
from tests import fragment_order as F

FAKE = ctypes.c_void_p(0x10000)


def test_hand_positions():
    # a 16 x 128-byte matrix: two 64-byte slices of one block
    pos = F.positions(16, 128)
    assert pos[0, 0] == 0
    assert pos[0, 16] == 16 * 16            # row 0, quarter 1: lane 16
    assert pos[1, 0] == 16                  # row 1, quarter 0: lane 1
    assert pos[5, 70] == 1024 + 16 * 5 + 6  # slice 1, quarter 0, byte 6 of row 5
    assert pos[15, 127] == 2047             # the last byte: slice 1, lane 15 + 48, byte 15
    # a second block starts after 16 whole rows
    pos = F.positions(32, 64)
    assert pos[16, 0] == 16 * 64
    assert pos[17, 63] == 16 * 64 + 16 * (1 + 48) + 15


def test_scale_order_hand_positions():
    # MXFP4 scales: 16-byte slices, a slice holds the 16 rows' bytes [16g, +16) row after row
    pos = F.positions(16, 160, 16)
    assert pos[0, 0] == 0
    assert pos[1, 0] == 16
    assert pos[0, 16] == 256               # slice 1
    assert pos[3, 37] == 2 * 256 + 16 * 3 + 5
    pos = F.positions(32, 32, 16)
    assert pos[16, 0] == 16 * 32           # block 1 after 16 rows of 32 bytes
    assert pos[31, 31] == 16 * 32 + 256 + 16 * 15 + 15


def test_positions_are_a_bijection():
    for R, B, W in ((16, 64, 64), (48, 192, 64), (32, 1280, 64), (16, 16, 16), (48, 160, 16)):
        p = F.positions(R, B, W).ravel()
        assert np.array_equal(np.sort(p), np.arange(R * B))


@pytest.mark.parametrize("dtype,shape", [(np.uint16, (3, 48, 256)), (np.uint8, (2, 32, 192)),
                                         (np.uint16, (16, 32)), (np.uint8, (64, 640))])
def test_two_forms_agree_and_invert(dtype, shape):
    rng = np.random.default_rng(7)
    w = rng.integers(0, np.iinfo(dtype).max, size=shape, dtype=dtype)
    a = F.pack_by_positions(w)
    b = F.pack_by_reshape(w)
    assert a.dtype == w.dtype and a.shape == w.shape
    assert np.array_equal(a, b)
    assert np.array_equal(F.unpack(a), w)
    if w.shape[-1] * w.itemsize % 16 == 0:
        a16 = F.pack_by_positions(w, 16)
        assert np.array_equal(a16, F.pack_by_reshape(w, 16))
        assert np.array_equal(F.unpack(a16, 16), w)


def test_slice_holds_a_matrix_core_operand():
    """Lane L of a slice holds 16 bytes of row L%16 at quarter L//16: for bf16 that is the 8 k values
    [32f + 8(L//16), +8) of that row, the B operand of a 16x16x32 MFMA lane."""
    R, H = 16, 128
    w = (np.arange(R)[:, None] * 1000 + np.arange(H)[None, :]).astype(np.uint16)   # value = 1000 r + k
    p = F.pack_by_reshape(w).reshape(-1, 64, 8)   # [slices, lanes, 8 bf16]
    for f in range(H // 32):
        for L in range(64):
            r, q = L % 16, L // 16
            assert list(p[f, L]) == [1000 * r + 32 * f + 8 * q + t for t in range(8)]


def test_mxfp4_fragment_order_needs_512():
    n = ctypes.c_size_t(0)
    for H, I in ((768, 512), (512, 768)):
        c = bm.Config(hidden=H, inter=I, weight_type=B.W_MXFP4, weight_layout=B.LAYOUT_FRAGMENTS).c()
        assert B.LIB.beam_moe_workspace_bytes(ctypes.byref(c), 64, B.OP_FORWARD, ctypes.byref(n)) == B.ERR_UNSUPPORTED
        c = bm.Config(hidden=H, inter=I, weight_type=B.W_MXFP4).c()           # row order: fine
        assert B.LIB.beam_moe_workspace_bytes(ctypes.byref(c), 64, B.OP_FORWARD, ctypes.byref(n)) == B.OK
        d = bm.DenseConfig(H, I, B.W_MXFP4, B.LAYOUT_FRAGMENTS).c()
        assert B.LIB.beam_dense_workspace_bytes(ctypes.byref(d), 64, ctypes.byref(n)) == B.ERR_UNSUPPORTED
    c = bm.Config(hidden=1024, inter=512, weight_type=B.W_MXFP4, weight_layout=B.LAYOUT_FRAGMENTS).c()
    assert B.LIB.beam_moe_workspace_bytes(ctypes.byref(c), 64, B.OP_FORWARD, ctypes.byref(n)) == B.OK


def test_bad_layout_rejected():
    n = ctypes.c_size_t(0)
    for lay in (-1, 2):
        c = bm.Config(weight_layout=lay).c()
        assert B.LIB.beam_moe_workspace_bytes(ctypes.byref(c), 64, B.OP_FORWARD, ctypes.byref(n)) == B.ERR_INVALID
        d = bm.DenseConfig(weight_layout=lay).c()
        assert B.LIB.beam_dense_workspace_bytes(ctypes.byref(d), 64, ctypes.byref(n)) == B.ERR_INVALID
    c = bm.Config(weight_layout=B.LAYOUT_FRAGMENTS).c()
    assert B.LIB.beam_moe_workspace_bytes(ctypes.byref(c), 64, B.OP_FORWARD, ctypes.byref(n)) == B.OK
    assert n.value == bm.beam_moe_workspace_bytes(bm.Config(), 64)   # the order changes no workspace


def test_pack_validation():
    L, f = B.LIB, FAKE
    other = ctypes.c_void_p(0x10000 + (1 << 30))
    assert L.beam_moe_pack_weights(24, 128, f, other, None) == B.ERR_INVALID        # rows % 16
    assert L.beam_moe_pack_weights(16, 96, f, other, None) == B.ERR_INVALID         # row bytes % 64
    assert L.beam_moe_pack_weights(16, 0, f, other, None) == B.ERR_INVALID
    assert L.beam_moe_pack_weights(-16, 64, f, other, None) == B.ERR_INVALID
    assert L.beam_moe_pack_weights(16, 64, None, other, None) == B.ERR_INVALID
    assert L.beam_moe_pack_weights(16, 64, f, None, None) == B.ERR_INVALID
    assert L.beam_moe_pack_weights(16, 64, ctypes.c_void_p(0x10008), other, None) == B.ERR_INVALID   # misaligned
    assert L.beam_moe_pack_weights(16, 64, f, ctypes.c_void_p(0x10000 + 512), None) == B.ERR_INVALID  # overlap
    assert L.beam_moe_pack_weights(16, 64, f, f, None) == B.ERR_INVALID                               # in place
    assert L.beam_moe_pack_weights(0, 64, None, None, None) == B.OK                                   # no-op
    # scales: 16-byte slices
    assert L.beam_moe_pack_scales(16, 24, f, other, None) == B.ERR_INVALID          # row bytes % 16
    assert L.beam_moe_pack_scales(8, 16, f, other, None) == B.ERR_INVALID           # rows % 16
    assert L.beam_moe_pack_scales(16, 16, f, ctypes.c_void_p(0x10000 + 128), None) == B.ERR_INVALID   # overlap
    assert L.beam_moe_pack_scales(16, 16, None, other, None) == B.ERR_INVALID
    assert L.beam_moe_pack_scales(0, 16, None, None, None) == B.OK


def test_binding_pack_checks_shapes_first():
    import torch
    with pytest.raises(ValueError, match="multiple of 16"):
        bm.beam_moe_pack_weights(torch.zeros(24, 64, dtype=torch.bfloat16))    # 24 rows
    with pytest.raises(ValueError, match="multiple of 16"):
        bm.beam_moe_pack_weights(torch.zeros(16, 16, dtype=torch.bfloat16))    # 32-byte rows
    with pytest.raises(ValueError, match="must be one of"):
        bm.beam_moe_pack_weights(torch.zeros(16, 64, dtype=torch.float32))
    with pytest.raises(ValueError, match="device tensor"):                     # a valid shape on the host
        bm.beam_moe_pack_weights(torch.zeros(16, 64, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="multiple of 16"):
        bm.beam_moe_pack_scales(torch.zeros(16, 8, dtype=torch.uint8))          # 8-byte scale rows
    with pytest.raises(ValueError, match="must be one of"):
        bm.beam_moe_pack_scales(torch.zeros(16, 16, dtype=torch.bfloat16))
