"""Thin ctypes binding of libbeam_moe.so (the C ABI in include/beam_moe.h).

Argument marshalling only: dtype/shape/device checks on torch tensors, then the
raw device pointers and torch's current HIP stream go to the library, which
enqueues every step of the path in its own kernels.  There is no fallback: if
the library is not built, importing the binding raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libbeam_moe.so")

OK, ERR_INVALID, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = 0, -1, -2, -3, -4
W_BF16, W_FP8_E4M3, W_MXFP4 = 0, 1, 2
LAYOUT_ROWS, LAYOUT_FRAGMENTS = 0, 1
OP_ROUTE, OP_PERMUTE, OP_FORWARD, OP_BLOCK = 0, 1, 2, 3
MAX_TOKENS = 262144
MAX_NORM_HIDDEN = 8192


class BeamMoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {status_string(status)} ({status})")


class _Config(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("inter", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("n_groups", ctypes.c_int32), ("topk_groups", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("routed_scale", ctypes.c_float), ("weight_type", ctypes.c_int32), ("weight_layout", ctypes.c_int32)]


@dataclass(frozen=True)
class Config:
    """Layer shape: hidden H, inter I, E experts in G groups, keep Gk groups, top-K, scale alpha; the
    expert weights' type and byte order (LAYOUT_FRAGMENTS: as beam_moe_pack_weights writes them)."""
    hidden: int = 5120
    inter: int = 2560
    n_experts: int = 256
    n_groups: int = 8
    topk_groups: int = 4
    top_k: int = 8
    routed_scale: float = 2.5
    weight_type: int = W_BF16
    weight_layout: int = LAYOUT_ROWS

    def c(self) -> _Config:
        return _Config(self.hidden, self.inter, self.n_experts, self.n_groups, self.topk_groups, self.top_k,
                       self.routed_scale, self.weight_type, self.weight_layout)


class _DenseConfig(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("inter", ctypes.c_int32), ("weight_type", ctypes.c_int32),
                ("weight_layout", ctypes.c_int32)]


@dataclass(frozen=True)
class DenseConfig:
    """Dense SwiGLU MLP shape: hidden H, intermediate I (not given on the pages: a parameter)."""
    hidden: int = 5120
    inter: int = 20480
    weight_type: int = W_BF16
    weight_layout: int = LAYOUT_ROWS

    def c(self) -> _DenseConfig:
        return _DenseConfig(self.hidden, self.inter, self.weight_type, self.weight_layout)


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is not built; run python sparse_moe_layer_top_amd/build.py "
                          "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(_LIB_PATH)
    P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    cfgp = ctypes.POINTER(_Config)
    lib.beam_moe_status_string.argtypes = [ctypes.c_int]
    lib.beam_moe_status_string.restype = ctypes.c_char_p
    lib.beam_moe_workspace_bytes.argtypes = [cfgp, I32, I32, ctypes.POINTER(SZ)]
    lib.beam_moe_workspace_bytes.restype = ctypes.c_int
    lib.beam_moe_route.argtypes = [cfgp, I32, P, P, P, P, P, P, SZ, P]
    lib.beam_moe_route.restype = ctypes.c_int
    lib.beam_moe_permute.argtypes = [cfgp, I32, P, P, P, P, P, SZ, P]
    lib.beam_moe_permute.restype = ctypes.c_int
    lib.beam_moe_forward.argtypes = [cfgp, I32, P, P, P, P, P, P, P, P, P, P, P, P, P, SZ, P]
    lib.beam_moe_forward.restype = ctypes.c_int
    lib.beam_moe_forward_timed.argtypes = [cfgp, I32] + [P] * 13 + [SZ, P, P]
    lib.beam_moe_forward_timed.restype = ctypes.c_int
    lib.beam_moe_forward_noalloc.argtypes = [cfgp, I32] + [P] * 13
    lib.beam_moe_forward_noalloc.restype = ctypes.c_int
    F32 = ctypes.c_float
    lib.beam_moe_rms_norm.argtypes = [I32, I32, P, P, F32, P, P]
    lib.beam_moe_rms_norm.restype = ctypes.c_int
    lib.beam_moe_block_forward.argtypes = [cfgp, I32, I32, F32] + [P] * 16 + [SZ, P]
    lib.beam_moe_block_forward.restype = ctypes.c_int
    lib.beam_moe_block_forward_timed.argtypes = [cfgp, I32, I32, F32] + [P] * 16 + [SZ, P, P]
    lib.beam_moe_block_forward_timed.restype = ctypes.c_int
    dcfgp = ctypes.POINTER(_DenseConfig)
    lib.beam_dense_workspace_bytes.argtypes = [dcfgp, I32, ctypes.POINTER(SZ)]
    lib.beam_dense_workspace_bytes.restype = ctypes.c_int
    lib.beam_dense_mlp_forward.argtypes = [dcfgp, I32] + [P] * 9 + [SZ, P]
    lib.beam_dense_mlp_forward.restype = ctypes.c_int
    lib.beam_dense_mlp_forward_timed.argtypes = [dcfgp, I32] + [P] * 9 + [SZ, P, P]
    lib.beam_dense_mlp_forward_timed.restype = ctypes.c_int
    lib.beam_mxfp4_quantize.argtypes = [I32, I32, P, P, P, P]
    lib.beam_mxfp4_quantize.restype = ctypes.c_int
    lib.beam_moe_pack_weights.argtypes = [ctypes.c_int64, I32, P, P, P]
    lib.beam_moe_pack_weights.restype = ctypes.c_int
    lib.beam_moe_pack_scales.argtypes = [ctypes.c_int64, I32, P, P, P]
    lib.beam_moe_pack_scales.restype = ctypes.c_int
    return lib


LIB = _load()
LIB_PATH = _LIB_PATH


def status_string(status: int) -> str:
    return LIB.beam_moe_status_string(status).decode()


def _check(fn: str, st: int):
    if st != OK:
        raise BeamMoeError(fn, st)


def beam_moe_workspace_bytes(cfg: Config, T: int, op: int = OP_FORWARD) -> int:
    n = ctypes.c_size_t(0)
    _check("beam_moe_workspace_bytes", LIB.beam_moe_workspace_bytes(ctypes.byref(cfg.c()), T, op, ctypes.byref(n)))
    return n.value


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t: Optional[torch.Tensor], name: str, dtype, shape, device=None, optional=False):
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _expert_weights(weight_type, lead, H, I, w_gate, w_up, w_down, s_gate, s_up, s_down, dev):
    """Checks the gate/up [*lead, I, H] and down [*lead, H, I] weights and their scales for the weight type:
    bf16 (no scales); e4m3 codes (uint8, same shape) with fp32 per-output-row scales [*lead, rows];
    MXFP4 (uint8, two E2M1 codes a byte, low nibble first: [*lead, rows, cols/2]) with E8M0 scale bytes
    [*lead, rows, cols/32]."""
    lead = tuple(lead)
    mats = ((w_gate, s_gate, "gate", I, H), (w_up, s_up, "up", I, H), (w_down, s_down, "down", H, I))
    for w, sc, n, rows, cols in mats:
        if weight_type == W_BF16:
            _need(w, "w_" + n, torch.bfloat16, lead + (rows, cols), dev)
        elif weight_type == W_FP8_E4M3:
            _need(w, "w_" + n, torch.uint8, lead + (rows, cols), dev)
            _need(sc, "s_" + n, torch.float32, lead + (rows,), dev)
        elif weight_type == W_MXFP4:
            _need(w, "w_" + n, torch.uint8, lead + (rows, cols // 2), dev)
            _need(sc, "s_" + n, torch.uint8, lead + (rows, cols // 32), dev)
        else:
            raise ValueError(f"unknown weight_type {weight_type}")
    if weight_type == W_BF16 and any(t is not None for t in (s_gate, s_up, s_down)):
        raise ValueError("scales are only for fp8 and MXFP4 weights")


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _workspace(cfg, T, op, workspace, device):
    need = beam_moe_workspace_bytes(cfg, T, op)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=device)
    if workspace.dtype != torch.uint8 or workspace.device != device or workspace.numel() < need:
        raise ValueError(f"workspace must be a uint8 device tensor of at least {need} bytes")
    return workspace


def beam_moe_route(cfg: Config, x: torch.Tensor, w_router: torch.Tensor, b_router: Optional[torch.Tensor] = None,
                   topk_ids: Optional[torch.Tensor] = None, topk_w: Optional[torch.Tensor] = None,
                   workspace: Optional[torch.Tensor] = None):
    """Router + group-limited top-k.  x [T,H] bf16, w_router [H,E] fp32, b_router [E] fp32 or None.
    Returns (topk_ids [T,K] int32 ascending, topk_w [T,K] fp32)."""
    T, dev = x.shape[0], x.device
    _need(x, "x", torch.bfloat16, (T, cfg.hidden))
    _need(w_router, "w_router", torch.float32, (cfg.hidden, cfg.n_experts), dev)
    _need(b_router, "b_router", torch.float32, (cfg.n_experts,), dev, optional=True)
    if topk_ids is None:
        topk_ids = torch.empty(T, cfg.top_k, dtype=torch.int32, device=dev)
    if topk_w is None:
        topk_w = torch.empty(T, cfg.top_k, dtype=torch.float32, device=dev)
    _need(topk_ids, "topk_ids", torch.int32, (T, cfg.top_k), dev)
    _need(topk_w, "topk_w", torch.float32, (T, cfg.top_k), dev)
    ws = _workspace(cfg, T, OP_ROUTE, workspace, dev)
    _check("beam_moe_route", LIB.beam_moe_route(ctypes.byref(cfg.c()), T, _ptr(x), _ptr(w_router), _ptr(b_router),
                                                _ptr(topk_ids), _ptr(topk_w), _ptr(ws), ws.numel(), _stream(dev)))
    return topk_ids, topk_w


def beam_moe_permute(cfg: Config, topk_ids: torch.Tensor, expert_offsets=None, sorted_pairs=None,
                     pair_to_row=None, workspace: Optional[torch.Tensor] = None):
    """Token -> expert permutation.  Returns (expert_offsets [E+1], sorted_pairs [T*K], pair_to_row [T*K])."""
    T, dev = topk_ids.shape[0], topk_ids.device
    _need(topk_ids, "topk_ids", torch.int32, (T, cfg.top_k))
    n = T * cfg.top_k
    if expert_offsets is None:
        expert_offsets = torch.empty(cfg.n_experts + 1, dtype=torch.int32, device=dev)
    if sorted_pairs is None:
        sorted_pairs = torch.empty(n, dtype=torch.int32, device=dev)
    if pair_to_row is None:
        pair_to_row = torch.empty(n, dtype=torch.int32, device=dev)
    _need(expert_offsets, "expert_offsets", torch.int32, (cfg.n_experts + 1,), dev)
    _need(sorted_pairs, "sorted_pairs", torch.int32, (n,), dev)
    _need(pair_to_row, "pair_to_row", torch.int32, (n,), dev)
    ws = _workspace(cfg, T, OP_PERMUTE, workspace, dev)
    _check("beam_moe_permute", LIB.beam_moe_permute(ctypes.byref(cfg.c()), T, _ptr(topk_ids), _ptr(expert_offsets),
                                                    _ptr(sorted_pairs), _ptr(pair_to_row), _ptr(ws), ws.numel(),
                                                    _stream(dev)))
    return expert_offsets, sorted_pairs, pair_to_row


def beam_moe_forward(cfg: Config, x: torch.Tensor, w_router: torch.Tensor, b_router: Optional[torch.Tensor],
                     w_gate: torch.Tensor, w_up: torch.Tensor, w_down: torch.Tensor,
                     s_gate: Optional[torch.Tensor] = None, s_up: Optional[torch.Tensor] = None,
                     s_down: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                     topk_ids_out: Optional[torch.Tensor] = None, topk_w_out: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None, stage_events=None) -> torch.Tensor:
    """The whole MoE block.  Expert weights [E,I,H] / [E,H,I]: bf16, uint8 e4m3 codes with fp32 per-row
    scales, or MXFP4 codes with E8M0 block scales (see _expert_weights).

    stage_events: None, or 7 recorded torch.cuda.Event(enable_timing=True)
    that the library records before each stage and after the last
    (beam_moe_forward_timed)."""
    T, dev = x.shape[0], x.device
    E, H, I = cfg.n_experts, cfg.hidden, cfg.inter
    _need(x, "x", torch.bfloat16, (T, H))
    _need(w_router, "w_router", torch.float32, (H, E), dev)
    _need(b_router, "b_router", torch.float32, (E,), dev, optional=True)
    _expert_weights(cfg.weight_type, (E,), H, I, w_gate, w_up, w_down, s_gate, s_up, s_down, dev)
    if out is None:
        out = torch.empty(T, H, dtype=torch.bfloat16, device=dev)
    _need(out, "out", torch.bfloat16, (T, H), dev)
    _need(topk_ids_out, "topk_ids_out", torch.int32, (T, cfg.top_k), dev, optional=True)
    _need(topk_w_out, "topk_w_out", torch.float32, (T, cfg.top_k), dev, optional=True)
    ws = _workspace(cfg, T, OP_FORWARD, workspace, dev)
    args = [ctypes.byref(cfg.c()), T, _ptr(x), _ptr(w_router), _ptr(b_router), _ptr(w_gate), _ptr(w_up),
            _ptr(w_down), _ptr(s_gate), _ptr(s_up), _ptr(s_down), _ptr(out), _ptr(topk_ids_out),
            _ptr(topk_w_out), _ptr(ws), ws.numel(), _stream(dev)]
    if stage_events is None:
        _check("beam_moe_forward", LIB.beam_moe_forward(*args))
    else:
        if len(stage_events) != 7 or any(ev.cuda_event == 0 for ev in stage_events):
            raise ValueError("stage_events must be 7 torch.cuda.Event objects, each recorded once beforehand")
        arr = (ctypes.c_void_p * 7)(*[ev.cuda_event for ev in stage_events])
        _check("beam_moe_forward_timed", LIB.beam_moe_forward_timed(*args, arr))
    return out


NOALLOC_SCRATCH_BYTES = 64 << 20


def beam_moe_forward_noalloc(cfg: Config, x: torch.Tensor, w_router: torch.Tensor, b_router: Optional[torch.Tensor],
                             w_gate: torch.Tensor, w_up: torch.Tensor, w_down: torch.Tensor,
                             out: torch.Tensor, s_gate: Optional[torch.Tensor] = None,
                             s_up: Optional[torch.Tensor] = None, s_down: Optional[torch.Tensor] = None,
                             topk_ids_out: Optional[torch.Tensor] = None,
                             topk_w_out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """beam_moe_forward with the library's fixed device scratch array as its workspace (for callers that
    cannot allocate): the caller passes every input and output, `out` included; nothing is allocated.
    Calls on one device share the array, so they must not overlap."""
    T, dev = x.shape[0], x.device
    E, H, I = cfg.n_experts, cfg.hidden, cfg.inter
    _need(x, "x", torch.bfloat16, (T, H))
    _need(w_router, "w_router", torch.float32, (H, E), dev)
    _need(b_router, "b_router", torch.float32, (E,), dev, optional=True)
    _expert_weights(cfg.weight_type, (E,), H, I, w_gate, w_up, w_down, s_gate, s_up, s_down, dev)
    _need(out, "out", torch.bfloat16, (T, H), dev)
    _need(topk_ids_out, "topk_ids_out", torch.int32, (T, cfg.top_k), dev, optional=True)
    _need(topk_w_out, "topk_w_out", torch.float32, (T, cfg.top_k), dev, optional=True)
    _check("beam_moe_forward_noalloc",
           LIB.beam_moe_forward_noalloc(ctypes.byref(cfg.c()), T, _ptr(x), _ptr(w_router), _ptr(b_router),
                                        _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(s_gate), _ptr(s_up),
                                        _ptr(s_down), _ptr(out), _ptr(topk_ids_out), _ptr(topk_w_out),
                                        _stream(dev)))
    return out


def beam_moe_rms_norm(x: torch.Tensor, gamma: torch.Tensor, eps: float, out: Optional[torch.Tensor] = None):
    """RMSNorm of bf16 rows x [T,H] with fp32 gain gamma [H]: bf16((x * r) * gamma), r = 1/sqrt(mean(x^2)+eps),
    every step one correctly rounded fp32 operation (sum of squares over 64 contiguous channel blocks, each in
    channel order, then the block sums in block order).  out may be x."""
    T, H = x.shape
    dev = x.device
    _need(x, "x", torch.bfloat16, (T, H))
    _need(gamma, "gamma", torch.float32, (H,), dev)
    if out is None:
        out = torch.empty(T, H, dtype=torch.bfloat16, device=dev)
    _need(out, "out", torch.bfloat16, (T, H), dev)
    _check("beam_moe_rms_norm", LIB.beam_moe_rms_norm(T, H, _ptr(x), _ptr(gamma), ctypes.c_float(eps), _ptr(out),
                                                      _stream(dev)))
    return out


def beam_moe_block_forward(cfg: Config, step: int, eps: float, stream_in: torch.Tensor, gamma_pre: torch.Tensor,
                           gamma_post: torch.Tensor, w_router: torch.Tensor, b_router: Optional[torch.Tensor],
                           w_gate: torch.Tensor, w_up: torch.Tensor, w_down: torch.Tensor,
                           s_gate: Optional[torch.Tensor] = None, s_up: Optional[torch.Tensor] = None,
                           s_down: Optional[torch.Tensor] = None, stream_out: Optional[torch.Tensor] = None,
                           moe_out: Optional[torch.Tensor] = None, topk_ids_out: Optional[torch.Tensor] = None,
                           topk_w_out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                           stage_events=None) -> torch.Tensor:
    """Pre-norm, the MoE block, post-norm and the constant-scale residual mix at step `step` (>= 2).

    Returns stream_out [T,H] bf16 (may be stream_in itself).  moe_out, if given, receives the MoE output
    before the post-norm.  stage_events: None or 8 recorded torch.cuda.Event objects."""
    T, dev = stream_in.shape[0], stream_in.device
    E, H, I = cfg.n_experts, cfg.hidden, cfg.inter
    _need(stream_in, "stream_in", torch.bfloat16, (T, H))
    _need(gamma_pre, "gamma_pre", torch.float32, (H,), dev)
    _need(gamma_post, "gamma_post", torch.float32, (H,), dev)
    _need(w_router, "w_router", torch.float32, (H, E), dev)
    _need(b_router, "b_router", torch.float32, (E,), dev, optional=True)
    _expert_weights(cfg.weight_type, (E,), H, I, w_gate, w_up, w_down, s_gate, s_up, s_down, dev)
    if stream_out is None:
        stream_out = torch.empty(T, H, dtype=torch.bfloat16, device=dev)
    _need(stream_out, "stream_out", torch.bfloat16, (T, H), dev)
    _need(moe_out, "moe_out", torch.bfloat16, (T, H), dev, optional=True)
    _need(topk_ids_out, "topk_ids_out", torch.int32, (T, cfg.top_k), dev, optional=True)
    _need(topk_w_out, "topk_w_out", torch.float32, (T, cfg.top_k), dev, optional=True)
    ws = _workspace(cfg, T, OP_BLOCK, workspace, dev)
    args = [ctypes.byref(cfg.c()), T, step, ctypes.c_float(eps), _ptr(stream_in), _ptr(gamma_pre), _ptr(gamma_post),
            _ptr(w_router), _ptr(b_router), _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(s_gate), _ptr(s_up),
            _ptr(s_down), _ptr(stream_out), _ptr(moe_out), _ptr(topk_ids_out), _ptr(topk_w_out), _ptr(ws),
            ws.numel(), _stream(dev)]
    if stage_events is None:
        _check("beam_moe_block_forward", LIB.beam_moe_block_forward(*args))
    else:
        if len(stage_events) != 8 or any(ev.cuda_event == 0 for ev in stage_events):
            raise ValueError("stage_events must be 8 torch.cuda.Event objects, each recorded once beforehand")
        arr = (ctypes.c_void_p * 8)(*[ev.cuda_event for ev in stage_events])
        _check("beam_moe_block_forward_timed", LIB.beam_moe_block_forward_timed(*args, arr))
    return stream_out


def beam_dense_workspace_bytes(cfg: DenseConfig, T: int) -> int:
    n = ctypes.c_size_t(0)
    _check("beam_dense_workspace_bytes", LIB.beam_dense_workspace_bytes(ctypes.byref(cfg.c()), T, ctypes.byref(n)))
    return n.value


def beam_dense_mlp_forward(cfg: DenseConfig, x: torch.Tensor, w_gate: torch.Tensor, w_up: torch.Tensor,
                           w_down: torch.Tensor, s_gate: Optional[torch.Tensor] = None,
                           s_up: Optional[torch.Tensor] = None, s_down: Optional[torch.Tensor] = None,
                           out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                           stage_events=None) -> torch.Tensor:
    """Dense SwiGLU MLP: out = bf16(W_down bf16(SiLU(W_gate x) * (W_up x))).  Weights [I,H] / [H,I]: bf16,
    uint8 e4m3 codes with fp32 per-output scales, or MXFP4 (see _expert_weights).  stage_events: None or 4 recorded torch.cuda.Event objects."""
    T, dev = x.shape[0], x.device
    H, I = cfg.hidden, cfg.inter
    _need(x, "x", torch.bfloat16, (T, H))
    _expert_weights(cfg.weight_type, (), H, I, w_gate, w_up, w_down, s_gate, s_up, s_down, dev)
    if out is None:
        out = torch.empty(T, H, dtype=torch.bfloat16, device=dev)
    _need(out, "out", torch.bfloat16, (T, H), dev)
    need = beam_dense_workspace_bytes(cfg, T)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    if workspace.dtype != torch.uint8 or workspace.device != dev or workspace.numel() < need:
        raise ValueError(f"workspace must be a uint8 device tensor of at least {need} bytes")
    args = [ctypes.byref(cfg.c()), T, _ptr(x), _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(s_gate), _ptr(s_up),
            _ptr(s_down), _ptr(out), _ptr(workspace), workspace.numel(), _stream(dev)]
    if stage_events is None:
        _check("beam_dense_mlp_forward", LIB.beam_dense_mlp_forward(*args))
    else:
        if len(stage_events) != 4 or any(ev.cuda_event == 0 for ev in stage_events):
            raise ValueError("stage_events must be 4 torch.cuda.Event objects, each recorded once beforehand")
        arr = (ctypes.c_void_p * 4)(*[ev.cuda_event for ev in stage_events])
        _check("beam_dense_mlp_forward_timed", LIB.beam_dense_mlp_forward_timed(*args, arr))
    return out


def beam_mxfp4_quantize(w: torch.Tensor, codes: Optional[torch.Tensor] = None,
                        scales: Optional[torch.Tensor] = None):
    """MXFP4 encoding of bf16 rows w [..., cols] (cols % 32 == 0): returns (codes [..., cols/2] uint8,
    scales [..., cols/32] uint8), the layout the MXFP4 weight type reads."""
    if w.dim() < 1:
        raise ValueError("w must have at least one dimension")
    cols = w.shape[-1]
    rows = w.numel() // cols if cols else 0
    lead = tuple(w.shape[:-1])
    dev = w.device
    _need(w, "w", torch.bfloat16, tuple(w.shape))
    if cols % 32:
        raise ValueError("cols must be a multiple of 32")
    if codes is None:
        codes = torch.empty(lead + (cols // 2,), dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty(lead + (cols // 32,), dtype=torch.uint8, device=dev)
    _need(codes, "codes", torch.uint8, lead + (cols // 2,), dev)
    _need(scales, "scales", torch.uint8, lead + (cols // 32,), dev)
    _check("beam_mxfp4_quantize", LIB.beam_mxfp4_quantize(rows, cols, _ptr(w), _ptr(codes), _ptr(scales),
                                                          _stream(dev)))
    return codes, scales


def _pack(fn: str, w: torch.Tensor, slice_bytes: int, dtypes, out: Optional[torch.Tensor]) -> torch.Tensor:
    if w.dim() < 2:
        raise ValueError("w must have at least two dimensions")
    if w.dtype not in dtypes:
        raise ValueError(f"w must be one of {dtypes}, got {w.dtype}")
    row_bytes = w.shape[-1] * w.element_size()
    rows = w.numel() // w.shape[-1] if w.shape[-1] else 0
    if rows % 16 or row_bytes % slice_bytes or row_bytes == 0:
        raise ValueError(f"rows ({rows}) must be a multiple of 16 and row bytes ({row_bytes}) of {slice_bytes}")
    dev = w.device
    _need(w, "w", w.dtype, tuple(w.shape))
    if out is None:
        out = torch.empty_like(w)
    _need(out, "out", w.dtype, tuple(w.shape), dev)
    _check(fn, getattr(LIB, fn)(rows, row_bytes, _ptr(w), _ptr(out), _stream(dev)))
    return out


def beam_moe_pack_weights(w: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Fragment order of weight matrices w [..., rows, cols] (bf16, or uint8 for e4m3 and MXFP4 codes):
    the same shape and dtype with the bytes permuted as LAYOUT_FRAGMENTS describes (16-row blocks,
    1 KB lane-ordered 64-byte column slices).  All leading rows are taken together: a multiple of 16,
    each row a multiple of 64 bytes."""
    return _pack("beam_moe_pack_weights", w, 64, (torch.bfloat16, torch.uint8), out)


def beam_moe_pack_scales(s: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Fragment order of MXFP4 scale matrices s [..., rows, cols/32] (uint8 E8M0): 16-row blocks of
    256-byte slices (16 bytes of each row).  Rows a multiple of 16, each row a multiple of 16 bytes."""
    return _pack("beam_moe_pack_scales", s, 16, (torch.uint8,), out)
