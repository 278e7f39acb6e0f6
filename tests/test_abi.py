"""The C ABI library: loads, exports every entry point the header declares, and
rejects invalid arguments before enqueuing anything (no GPU needed: every call
here fails validation before its first HIP call, or is the T = 0 no-op)."""
import ctypes
import os
import re

import pytest

import sparse_moe_layer_top_amd as bm
from sparse_moe_layer_top_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "beam_moe.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\s*\*)\s*(beam_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_three_entry_points():
    names = declared_functions()
    for n in ("beam_moe_route", "beam_moe_permute", "beam_moe_forward", "beam_moe_workspace_bytes",
              "beam_moe_status_string", "beam_moe_block_forward", "beam_dense_mlp_forward", "beam_mxfp4_quantize"):
        assert n in names


def test_every_declared_symbol_is_exported():
    lib = ctypes.CDLL(bm.LIB_PATH)
    for n in declared_functions():
        assert hasattr(lib, n), n


def test_status_strings():
    for st in (0, -1, -2, -3, -4):
        assert bm.status_string(st) and bm.status_string(st) != "unknown status"
    assert bm.status_string(7) == "unknown status"


def _cfg(**kw):
    return bm.Config(**kw).c()


BAD_CONFIGS = [
    (dict(n_experts=250), B.ERR_INVALID),                 # E % G != 0
    (dict(topk_groups=9), B.ERR_INVALID),                 # Gk > G
    (dict(top_k=0), B.ERR_INVALID),
    (dict(topk_groups=1, n_groups=64, top_k=8), B.ERR_INVALID),   # K > Gk*E/G = 4
    (dict(routed_scale=float("inf")), B.ERR_INVALID),
    (dict(weight_type=3), B.ERR_INVALID),
    (dict(hidden=5100), B.ERR_UNSUPPORTED),               # not a multiple of 128
    (dict(hidden=5248, weight_type=B.W_MXFP4), B.ERR_UNSUPPORTED),   # MXFP4: not a multiple of 256
    (dict(inter=2688, weight_type=B.W_MXFP4), B.ERR_UNSUPPORTED),
    (dict(n_experts=512, n_groups=8), B.ERR_UNSUPPORTED),
    (dict(top_k=9, topk_groups=4), B.ERR_UNSUPPORTED),
    (dict(n_groups=128, n_experts=256, topk_groups=8), B.ERR_UNSUPPORTED),
    # one expert per group: a group score is the sum of a group's two best scores
    (dict(n_experts=32, n_groups=32, topk_groups=8), B.ERR_INVALID),
    (dict(n_experts=8, n_groups=8, topk_groups=8, top_k=8), B.ERR_INVALID),
]


@pytest.mark.parametrize("kw,status", BAD_CONFIGS)
def test_bad_config_rejected(kw, status):
    n = ctypes.c_size_t(0)
    assert B.LIB.beam_moe_workspace_bytes(ctypes.byref(_cfg(**kw)), 64, B.OP_FORWARD, ctypes.byref(n)) == status
    assert B.LIB.beam_moe_route(ctypes.byref(_cfg(**kw)), 64, None, None, None, None, None, None, 0, None) == status


FAKE = ctypes.c_void_p(0x10000)   # aligned, never dereferenced: each call below fails validation first


def test_null_and_negative():
    c = ctypes.byref(_cfg())
    assert B.LIB.beam_moe_route(None, 4, FAKE, FAKE, None, FAKE, FAKE, FAKE, 1 << 30, None) == B.ERR_INVALID
    assert B.LIB.beam_moe_route(c, -1, FAKE, FAKE, None, FAKE, FAKE, FAKE, 1 << 30, None) == B.ERR_INVALID
    assert B.LIB.beam_moe_route(c, B.MAX_TOKENS + 1, FAKE, FAKE, None, FAKE, FAKE, FAKE, 1 << 30, None) == B.ERR_INVALID
    assert B.LIB.beam_moe_route(c, 4, None, FAKE, None, FAKE, FAKE, FAKE, 1 << 30, None) == B.ERR_INVALID
    assert B.LIB.beam_moe_permute(c, 4, FAKE, None, FAKE, FAKE, FAKE, 1 << 30, None) == B.ERR_INVALID
    args = [FAKE] * 6
    assert B.LIB.beam_moe_forward(c, 4, None, *args[:5], None, None, None, FAKE, None, None, FAKE, 1 << 30, None) == B.ERR_INVALID


def test_misaligned_pointer():
    c = ctypes.byref(_cfg())
    odd = ctypes.c_void_p(0x10008)
    assert B.LIB.beam_moe_route(c, 4, odd, FAKE, None, FAKE, FAKE, FAKE, 1 << 30, None) == B.ERR_INVALID


def test_scale_pointers_must_match_weight_type():
    c_bf16 = ctypes.byref(_cfg())
    c_fp8 = ctypes.byref(_cfg(weight_type=B.W_FP8_E4M3))
    f = FAKE
    # bf16 with scales, fp8 without: invalid
    assert B.LIB.beam_moe_forward(c_bf16, 4, f, f, None, f, f, f, f, f, f, f, None, None, f, 1 << 30, None) == B.ERR_INVALID
    assert B.LIB.beam_moe_forward(c_fp8, 4, f, f, None, f, f, f, None, None, None, f, None, None, f, 1 << 30, None) == B.ERR_INVALID


def test_workspace_too_small():
    c = ctypes.byref(_cfg())
    f = FAKE
    need = bm.beam_moe_workspace_bytes(bm.Config(), 64, B.OP_ROUTE)
    assert need > 0
    assert B.LIB.beam_moe_route(c, 64, f, f, None, f, f, f, need - 1, None) == B.ERR_WORKSPACE
    assert B.LIB.beam_moe_route(c, 64, f, f, None, f, f, None, need, None) == B.ERR_WORKSPACE
    need = bm.beam_moe_workspace_bytes(bm.Config(), 64, B.OP_FORWARD)
    assert B.LIB.beam_moe_forward(c, 64, f, f, None, f, f, f, None, None, None, f, None, None, f, need - 1, None) == B.ERR_WORKSPACE
    need = bm.beam_moe_workspace_bytes(bm.Config(), 64, B.OP_PERMUTE)
    assert B.LIB.beam_moe_permute(c, 64, f, f, f, f, f, need - 1, None) == B.ERR_WORKSPACE


def test_zero_tokens_is_a_noop():
    c = ctypes.byref(_cfg())
    assert B.LIB.beam_moe_route(c, 0, None, None, None, None, None, None, 0, None) == B.OK
    assert B.LIB.beam_moe_permute(c, 0, None, None, None, None, None, 0, None) == B.OK
    assert B.LIB.beam_moe_forward(c, 0, *([None] * 13), 0, None) == B.OK
    assert bm.beam_moe_workspace_bytes(bm.Config(), 0) == 0


def test_workspace_grows_with_T():
    cfg = bm.Config()
    sizes = [bm.beam_moe_workspace_bytes(cfg, T) for T in (1, 64, 1000, 8192)]
    assert sizes == sorted(sizes)
    # forward workspace holds at least h [T*K, I] and y [T*K, H] in bf16
    assert sizes[-1] >= 8192 * 8 * (2560 + 5120) * 2
    for op in (B.OP_ROUTE, B.OP_PERMUTE):
        assert bm.beam_moe_workspace_bytes(cfg, 8192, op) < sizes[-1]


def test_header_declares_norm_and_block_entry_points():
    names = declared_functions()
    for n in ("beam_moe_rms_norm", "beam_moe_block_forward", "beam_moe_block_forward_timed"):
        assert n in names


def test_rms_norm_validation():
    f, g = FAKE, FAKE
    L = B.LIB
    assert L.beam_moe_rms_norm(0, 5120, None, None, 1e-6, None, None) == B.OK              # T = 0: no work
    assert L.beam_moe_rms_norm(-1, 5120, f, g, 1e-6, f, None) == B.ERR_INVALID
    assert L.beam_moe_rms_norm(4, 5121, f, g, 1e-6, f, None) == B.ERR_INVALID             # not a multiple of 8
    assert L.beam_moe_rms_norm(4, 0, f, g, 1e-6, f, None) == B.ERR_INVALID
    assert L.beam_moe_rms_norm(4, 5120, f, g, 0.0, f, None) == B.ERR_INVALID              # eps must be > 0
    assert L.beam_moe_rms_norm(4, 5120, f, g, float("nan"), f, None) == B.ERR_INVALID
    assert L.beam_moe_rms_norm(4, 5120, f, g, float("inf"), f, None) == B.ERR_INVALID
    assert L.beam_moe_rms_norm(4, B.MAX_NORM_HIDDEN + 8, f, g, 1e-6, f, None) == B.ERR_UNSUPPORTED
    assert L.beam_moe_rms_norm(4, 5120, None, g, 1e-6, f, None) == B.ERR_INVALID
    assert L.beam_moe_rms_norm(4, 5120, f, None, 1e-6, f, None) == B.ERR_INVALID
    assert L.beam_moe_rms_norm(4, 5120, ctypes.c_void_p(0x10008), g, 1e-6, f, None) == B.ERR_INVALID


def _block(cfg, T, step=5, eps=1e-6, stream_in=FAKE, gpre=FAKE, gpost=FAKE, scales=(None, None, None),
           stream_out=FAKE, moe_out=None, ws=FAKE, ws_bytes=1 << 40):
    f = FAKE
    return B.LIB.beam_moe_block_forward(ctypes.byref(cfg), T, step, eps, stream_in, gpre, gpost, f, None, f, f, f,
                                        *scales, stream_out, moe_out, None, None, ws, ws_bytes, None)


def test_block_validation():
    c = _cfg()
    assert _block(c, 0, stream_in=None, gpre=None, gpost=None, stream_out=None, ws=None, ws_bytes=0) == B.OK
    assert _block(c, 4, step=1) == B.ERR_INVALID                    # the embedding is step 1
    assert _block(c, 4, eps=0.0) == B.ERR_INVALID
    assert _block(c, 4, eps=float("nan")) == B.ERR_INVALID
    assert _block(c, 4, gpre=None) == B.ERR_INVALID
    assert _block(c, 4, gpost=None) == B.ERR_INVALID
    assert _block(c, 4, stream_out=None) == B.ERR_INVALID
    assert _block(c, 4, moe_out=ctypes.c_void_p(0x10008)) == B.ERR_INVALID
    assert _block(c, 4, scales=(FAKE, FAKE, FAKE)) == B.ERR_INVALID  # bf16 with scales
    assert _block(_cfg(hidden=8192 + 128), 4) == B.ERR_UNSUPPORTED
    need = bm.beam_moe_workspace_bytes(bm.Config(), 64, B.OP_BLOCK)
    assert _block(c, 64, ws_bytes=need - 1) == B.ERR_WORKSPACE
    assert _block(c, 64, ws=None) == B.ERR_WORKSPACE


def test_block_workspace_adds_the_normalised_input():
    cfg = bm.Config()
    for T in (1, 64, 8192):
        fwd = bm.beam_moe_workspace_bytes(cfg, T, B.OP_FORWARD)
        blk = bm.beam_moe_workspace_bytes(cfg, T, B.OP_BLOCK)
        assert blk >= fwd + T * cfg.hidden * 2
    n = ctypes.c_size_t(0)
    assert B.LIB.beam_moe_workspace_bytes(ctypes.byref(_cfg(hidden=8192 + 128)), 4, B.OP_BLOCK,
                                          ctypes.byref(n)) == B.ERR_UNSUPPORTED
    assert B.LIB.beam_moe_workspace_bytes(ctypes.byref(_cfg()), 4, 9, ctypes.byref(n)) == B.ERR_INVALID


def _dcfg(**kw):
    return bm.DenseConfig(**kw).c()


def test_dense_validation():
    L = B.LIB
    f = FAKE
    c = ctypes.byref(_dcfg())
    n = ctypes.c_size_t(0)
    assert L.beam_dense_workspace_bytes(ctypes.byref(_dcfg(hidden=5100)), 4, ctypes.byref(n)) == B.ERR_UNSUPPORTED
    assert L.beam_dense_workspace_bytes(ctypes.byref(_dcfg(inter=0)), 4, ctypes.byref(n)) == B.ERR_INVALID
    assert L.beam_dense_workspace_bytes(ctypes.byref(_dcfg(weight_type=5)), 4, ctypes.byref(n)) == B.ERR_INVALID
    assert L.beam_dense_workspace_bytes(c, -1, ctypes.byref(n)) == B.ERR_INVALID
    assert L.beam_dense_workspace_bytes(c, 0, ctypes.byref(n)) == B.OK and n.value == 0
    assert L.beam_dense_mlp_forward(c, 0, *([None] * 9), 0, None) == B.OK
    assert L.beam_dense_mlp_forward(None, 4, f, f, f, f, None, None, None, f, f, 1 << 40, None) == B.ERR_INVALID
    assert L.beam_dense_mlp_forward(c, 4, None, f, f, f, None, None, None, f, f, 1 << 40, None) == B.ERR_INVALID
    assert L.beam_dense_mlp_forward(c, 4, f, f, f, f, f, f, f, f, f, 1 << 40, None) == B.ERR_INVALID   # bf16 + scales
    c8 = ctypes.byref(_dcfg(weight_type=B.W_FP8_E4M3))
    assert L.beam_dense_mlp_forward(c8, 4, f, f, f, f, None, None, None, f, f, 1 << 40, None) == B.ERR_INVALID
    need = bm.beam_dense_workspace_bytes(bm.DenseConfig(), 64)
    assert L.beam_dense_mlp_forward(c, 64, f, f, f, f, None, None, None, f, f, need - 1, None) == B.ERR_WORKSPACE
    assert L.beam_dense_mlp_forward(c, 64, f, f, f, f, None, None, None, f, None, need, None) == B.ERR_WORKSPACE


def test_dense_workspace_holds_h_and_the_split_partials():
    cfg = bm.DenseConfig()
    small = bm.beam_dense_workspace_bytes(cfg, 64)
    assert small >= 64 * cfg.inter * 2 + 2 * 64 * cfg.hidden * 4       # h plus at least two fp32 parts
    assert bm.beam_dense_workspace_bytes(cfg, 8192) >= 8192 * cfg.inter * 2


def test_mxfp4_scales_required_and_aligned():
    c = ctypes.byref(_cfg(weight_type=B.W_MXFP4))
    f = FAKE
    need = bm.beam_moe_workspace_bytes(bm.Config(weight_type=B.W_MXFP4), 4)
    # MXFP4 without block scales: invalid
    assert B.LIB.beam_moe_forward(c, 4, f, f, None, f, f, f, None, None, None, f, None, None, f, need, None) == B.ERR_INVALID
    # MXFP4 scale rows are read in 16-byte pieces: a 16-byte aligned scale pointer passes validation
    # (the call then fails only at the workspace check), a 4-byte aligned one does not (fp8 accepts it)
    four = ctypes.c_void_p(0x10004)
    assert B.LIB.beam_moe_forward(c, 4, f, f, None, f, f, f, f, f, f, f, None, None, f, need - 1, None) == B.ERR_WORKSPACE
    assert B.LIB.beam_moe_forward(c, 4, f, f, None, f, f, f, four, four, four, f, None, None, f, need - 1, None) == B.ERR_INVALID
    c8 = ctypes.byref(_cfg(weight_type=B.W_FP8_E4M3))
    assert B.LIB.beam_moe_forward(c8, 4, f, f, None, f, f, f, four, four, four, f, None, None, f, need - 1, None) == B.ERR_WORKSPACE
    odd = ctypes.c_void_p(0x10001)
    assert B.LIB.beam_moe_forward(c8, 4, f, f, None, f, f, f, odd, odd, odd, f, None, None, f, need - 1, None) == B.ERR_INVALID
    cd = ctypes.byref(_dcfg(weight_type=B.W_MXFP4))
    assert B.LIB.beam_dense_mlp_forward(cd, 4, f, f, f, f, None, None, None, f, f, 1 << 40, None) == B.ERR_INVALID
    n = ctypes.c_size_t(0)
    assert B.LIB.beam_dense_workspace_bytes(ctypes.byref(_dcfg(inter=20480 + 128, weight_type=B.W_MXFP4)), 4,
                                            ctypes.byref(n)) == B.ERR_UNSUPPORTED


def test_mxfp4_quantize_validation():
    L, f = B.LIB, FAKE
    assert L.beam_mxfp4_quantize(4, 48, f, f, f, None) == B.ERR_INVALID          # cols % 32
    assert L.beam_mxfp4_quantize(-1, 64, f, f, f, None) == B.ERR_INVALID
    assert L.beam_mxfp4_quantize(4, -32, f, f, f, None) == B.ERR_INVALID
    assert L.beam_mxfp4_quantize(4, 64, None, f, f, None) == B.ERR_INVALID
    assert L.beam_mxfp4_quantize(4, 64, f, f, None, None) == B.ERR_INVALID
    assert L.beam_mxfp4_quantize(4, 64, ctypes.c_void_p(0x10008), f, f, None) == B.ERR_INVALID   # misaligned
    assert L.beam_mxfp4_quantize(0, 64, None, None, None, None) == B.OK                        # no-op
    assert L.beam_mxfp4_quantize(4, 0, None, None, None, None) == B.OK


def test_binding_checks_mxfp4_shapes():
    """The binding's shape checks run before any device work: CPU tensors fail on the device check, so a
    wrong shape must be reported first."""
    import torch
    E, H, I = 2, 256, 256
    cfg = bm.Config(hidden=H, inter=I, n_experts=E, n_groups=1, topk_groups=1, top_k=1, weight_type=B.W_MXFP4)
    wg = torch.empty(E, I, H, dtype=torch.uint8)                   # unpacked width: wrong for MXFP4
    with pytest.raises(ValueError, match=r"w_gate: expected shape \(2, 256, 128\)"):
        B._expert_weights(cfg.weight_type, (E,), H, I, wg, wg, wg, None, None, None, None)
    sc = torch.empty(E, I, H // 32, dtype=torch.float32)
    with pytest.raises(TypeError, match="expected torch.uint8"):
        B._need(sc, "s_gate", torch.uint8, (E, I, H // 32))


def test_noalloc_forward_validation():
    """The allocation-free forward checks its arguments like the forward, and rejects a layer whose
    workspace exceeds the fixed scratch array before enqueuing anything (or touching the GPU)."""
    c = ctypes.byref(_cfg())
    f = FAKE
    assert B.LIB.beam_moe_forward_noalloc(c, 0, *([None] * 12), None) == B.OK
    assert B.LIB.beam_moe_forward_noalloc(None, 4, *([f] * 12), None) == B.ERR_INVALID
    assert B.LIB.beam_moe_forward_noalloc(c, -1, *([f] * 12), None) == B.ERR_INVALID
    # x missing; scales given for bf16 weights
    assert B.LIB.beam_moe_forward_noalloc(c, 4, None, f, None, f, f, f, None, None, None, f, None, None, None) == B.ERR_INVALID
    assert B.LIB.beam_moe_forward_noalloc(c, 4, f, f, None, f, f, f, f, f, f, f, None, None, None) == B.ERR_INVALID
    # the scratch array's limit: the real-shape layer's forward workspace crosses 64 MiB between 256 and 512 tokens
    cfg = bm.Config()
    assert bm.NOALLOC_SCRATCH_BYTES == 64 << 20
    fits = [T for T in (1, 64, 128, 256, 512, 8192) if bm.beam_moe_workspace_bytes(cfg, T) <= bm.NOALLOC_SCRATCH_BYTES]
    assert fits == [1, 64, 128, 256]
    assert B.LIB.beam_moe_forward_noalloc(c, 512, f, f, None, f, f, f, None, None, None, f, None, None, None) == B.ERR_WORKSPACE
    assert B.LIB.beam_moe_forward_noalloc(c, 8192, f, f, None, f, f, f, None, None, None, f, None, None, None) == B.ERR_WORKSPACE
