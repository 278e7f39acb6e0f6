"""Seeded generators for the synthetic MoE-layer workloads.

Shapes and value distributions follow the Beam MoE block as the pages state it
(Reflection Beam 1.0 overview, agentlenshq.com, section "Mixture of Experts":
hidden 5120, 256 SwiGLU experts of intermediate size 2560 in 8 groups of 32,
top-4 groups, top-8 experts, weights scaled by 2.5).  No trained weights exist
in this setting, so every tensor is drawn from a fixed distribution:

    x        ~ N(0, 1)      -> bf16           [T, H]
    W_router ~ N(0, s_r)    fp32              [H, E]   (s_r = 0.05 tiny, 0.02 real shape)
    b_router                fp32              [E]      (zero, fitted-balanced, or N(0, 1.5))
    W_gate, W_up ~ N(0, 0.02) -> bf16         [E, I, H] (out, in: the reduction dim is contiguous)
    W_down       ~ N(0, 0.02) -> bf16         [E, H, I]
    fp8 workloads: the same fp32 draw, quantised per output channel to OCP e4m3
    with scale = max_in |w| / 448 (fp32).
    MXFP4 workloads: uniform random bytes as E2M1 code pairs, and E8M0 block
    scales 127 + floor(log2(0.02 / 2.25)) + {-1, 0, 1} (2.25 = mean |E2M1 value|),
    so the weights have about the bf16 draws' scale; nothing is quantised.
    norm gains (the norms around the block): 1 + N(0, 0.1^2), fp32 [2, H].

Every tensor comes from its own stream, numpy.random.default_rng(
[seed, workload_id, tensor_id, index]); tensor ids: 0 x, 1 W_router, 2 bias,
3 W_gate, 4 W_up, 5 W_down, 6 re-drawn x rows, 7 norm gains.  Expert matrices are drawn one
expert at a time, so any single expert can be regenerated on the CPU without
touching the rest.  All real-shape workloads share one layer's expert weights
(workload id 2 in their seed); the fp8 workloads quantise those same fp32
draws.

fp32 -> bf16 and fp32 -> e4m3 conversions use torch's CPU casts (round to
nearest even); they are input preparation, not the layer's arithmetic.
"""
from __future__ import annotations

import os
import threading
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace
from typing import Callable, Optional

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))

X_ID, WR_ID, B_ID, WG_ID, WU_ID, WD_ID, REDRAW_ID, GAIN_ID = 0, 1, 2, 3, 4, 5, 6, 7
E4M3_MAX = 448.0


@dataclass(frozen=True)
class Workload:
    name: str
    wid: int            # workload id used in the seed tuple
    T: int              # tokens
    hidden: int         # H
    inter: int          # I
    n_experts: int      # E
    n_groups: int       # G
    topk_groups: int    # Gk
    top_k: int          # K
    alpha: float        # routed scale
    sigma_router: float
    sigma_expert: float
    bias: str           # "zero" | "balanced" | "skew"
    weight: str         # "bf16" | "fp8" | "mxfp4"
    weights_id: int     # seed id of the expert weights: every real-shape workload shares one layer

    def with_T(self, T: int) -> "Workload":
        return replace(self, T=T)


def _real(name, wid, T, bias="zero", weight="bf16"):
    return Workload(name, wid, T, 5120, 2560, 256, 8, 4, 8, 2.5, 0.02, 0.02, bias, weight, 2)


WORKLOADS = {
    # tiny layer, same routing structure: 32 experts in 8 groups of 4
    "tiny": Workload("tiny", 1, 64, 256, 128, 32, 8, 4, 8, 2.5, 0.05, 0.02, "zero", "bf16", 1),
    # real shape, decode regime: weight streaming
    "decode": _real("decode", 2, 64),
    # real shape, prefill regime with near-balanced expert loads
    "prefill": _real("prefill", 3, 8192, bias="balanced"),
    # real shape, skewed routing from a per-expert logit offset ~ N(0, 1.5)
    "skew": _real("skew", 4, 4096, bias="skew"),
    # real shape, e4m3 expert weights + per-output-channel fp32 scales
    "fp8_decode": _real("fp8_decode", 5, 32, weight="fp8"),
    "fp8_prefill": _real("fp8_prefill", 5, 2048, weight="fp8"),
    # real shape, MXFP4 expert weights (E2M1 codes, one E8M0 scale per 32 inputs)
    "mxfp4_decode": _real("mxfp4_decode", 10, 64, weight="mxfp4"),
    "mxfp4_prefill": _real("mxfp4_prefill", 10, 2048, weight="mxfp4"),
    # tiny MXFP4 layers (the MXFP4 kernels need H and I to be multiples of 256)
    "tiny_mx": Workload("tiny_mx", 11, 64, 256, 256, 32, 8, 4, 8, 2.5, 0.05, 0.02, "zero", "mxfp4", 11),
    "dense_tiny_mx": Workload("dense_tiny_mx", 12, 64, 256, 512, 1, 1, 1, 1, 1.0, 0.05, 0.02, "zero", "mxfp4", 12),
    # speculative verification: 8 sequences x (1 + 15 drafted tokens) in one forward pass
    "spec_verify": _real("spec_verify", 6, 128),
    # dense SwiGLU MLP (the first layers): one "expert" of intermediate 20480 = 8 x 2560
    # (the pages do not give the dense width; this one does a routed layer's per-token work)
    "dense_tiny": Workload("dense_tiny", 7, 64, 256, 512, 1, 1, 1, 1, 1.0, 0.05, 0.02, "zero", "bf16", 7),
    "dense_decode": Workload("dense_decode", 8, 64, 5120, 20480, 1, 1, 1, 1, 1.0, 0.02, 0.02, "zero", "bf16", 8),
    "dense_prefill": Workload("dense_prefill", 9, 8192, 5120, 20480, 1, 1, 1, 1, 1.0, 0.02, 0.02, "zero", "bf16", 8),
}


def workload(name: str, T: Optional[int] = None) -> Workload:
    w = WORKLOADS[name]
    return w if T is None else w.with_T(T)


# ---------------------------------------------------------------- casts ----

def bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 array -> bf16 bit patterns (uint16), round to nearest even (torch CPU cast)."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def _e4m3_codes(a: np.ndarray) -> np.ndarray:
    """fp32 -> OCP e4m3fn bytes, round to nearest even, saturating at +-448."""
    t = torch.from_numpy(np.clip(a, -E4M3_MAX, E4M3_MAX).astype(np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _rng(seed, wid, tid, idx=0):
    return np.random.default_rng([seed, wid, tid, idx])


# ------------------------------------------------------- router inputs ----

def _draw_x_rows(w: Workload, seed: int, rows: np.ndarray, rnd: int) -> np.ndarray:
    out = np.empty((len(rows), w.hidden), np.float32)
    for i, r in enumerate(rows):
        out[i] = _rng(seed, w.wid, REDRAW_ID, rnd * 1_000_003 + int(r)).standard_normal(
            w.hidden, dtype=np.float32)
    return bf16_bits(out)


def balanced_bias_path(seed: int) -> str:
    return os.path.join(_HERE, f"prefill_bias_seed{seed}.txt")


def load_balanced_bias(seed: int, n_experts: int) -> np.ndarray:
    """The fitted bias column of the balanced prefill workload.

    The file holds fp32 bit patterns in hex, one per expert, written by
    oracle/fit_prefill_bias.py (which fits it with the oracle's routing).
    """
    path = balanced_bias_path(seed)
    if not os.path.exists(path):
        raise FileNotFoundError(
            f"no fitted balanced bias for seed {seed} ({path}); "
            "run python -m oracle.fit_prefill_bias --seed N")
    vals = [int(line.split()[0], 16) for line in open(path)
            if line.strip() and not line.startswith("#")]
    b = np.array(vals, np.uint32).view(np.float32)
    if b.shape != (n_experts,):
        raise ValueError(f"{path}: expected {n_experts} values, got {b.shape}")
    return b


def router_inputs(w: Workload, seed: int = 0, bias: Optional[np.ndarray] = None):
    """Return (x_bits uint16 [T,H], W_router fp32 [H,E], b_router fp32 [E])."""
    x = _rng(seed, w.wid, X_ID).standard_normal((w.T, w.hidden), dtype=np.float32)
    x_bits = bf16_bits(x)
    wr = _rng(seed, w.wid, WR_ID).standard_normal((w.hidden, w.n_experts), dtype=np.float32)
    wr *= np.float32(w.sigma_router)
    if bias is not None:
        b = np.asarray(bias, np.float32)
    elif w.bias == "zero":
        b = np.zeros(w.n_experts, np.float32)
    elif w.bias == "skew":
        b = _rng(seed, w.wid, B_ID).standard_normal(w.n_experts, dtype=np.float32)
        b *= np.float32(1.5)
    elif w.bias == "balanced":
        b = load_balanced_bias(seed, w.n_experts)
    else:
        raise ValueError(w.bias)
    return x_bits, wr, b


def redraw_rows(x_bits: np.ndarray, w: Workload, seed: int, rows, rnd: int) -> np.ndarray:
    """Replace the given token rows with fresh N(0,1) draws from the re-draw stream."""
    rows = np.asarray(rows, np.int64)
    out = x_bits.copy()
    if len(rows):
        out[rows] = _draw_x_rows(w, seed, rows, rnd)
    return out


def guarded_router_inputs(w: Workload, seed: int,
                          violations: Callable[[np.ndarray, np.ndarray, np.ndarray], np.ndarray],
                          max_rounds: int = 16, bias: Optional[np.ndarray] = None):
    """router_inputs() with rows re-drawn until `violations` returns none.

    `violations(x_bits, W_router, b)` is supplied by the caller (the tests pass
    the oracle's score-gap check); this module does not compute scores itself.
    Returns (x_bits, W_router, b, n_redrawn).
    """
    x_bits, wr, b = router_inputs(w, seed, bias)
    n = 0
    for rnd in range(max_rounds):
        bad = np.asarray(violations(x_bits, wr, b))
        if len(bad) == 0:
            return x_bits, wr, b, n
        n += len(bad)
        x_bits = redraw_rows(x_bits, w, seed, bad, rnd)
    raise RuntimeError(f"gap guard still violated after {max_rounds} re-draw rounds")


def norm_gains(w: Workload, seed: int = 0):
    """Per-channel fp32 gains of the norms before and after the block: 1 + N(0, 0.1^2) each."""
    g = _rng(seed, w.wid, GAIN_ID).standard_normal((2, w.hidden), dtype=np.float32)
    return (1.0 + 0.1 * g[0]).astype(np.float32), (1.0 + 0.1 * g[1]).astype(np.float32)


# ------------------------------------------------------ expert weights ----

def expert_matrix(w: Workload, seed: int, which: str, e: int):
    """One expert's matrix.

    which: "gate" | "up" -> [I, H]; "down" -> [H, I].
    bf16 workloads return uint16 bit patterns; fp8 workloads return
    (uint8 e4m3 codes, fp32 scale [out]) with scale = max|w| / 448 per row;
    mxfp4 workloads return (packed E2M1 codes [out, in/2], E8M0 scales [out, in/32]).
    """
    tid = {"gate": WG_ID, "up": WU_ID, "down": WD_ID}[which]
    shape = (w.inter, w.hidden) if which in ("gate", "up") else (w.hidden, w.inter)
    if w.weight == "mxfp4":
        # random E2M1 codes (two per byte) and random E8M0 block scales near sigma / 2.25
        # (2.25 = mean |value| of a uniform code): drawn directly, nothing is quantised here
        g = _rng(seed, w.weights_id, tid, e)
        packed = g.integers(0, 256, (shape[0], shape[1] // 2), dtype=np.uint8)
        e0 = 127 + int(np.floor(np.log2(w.sigma_expert / 2.25)))
        scales = (e0 + g.integers(-1, 2, (shape[0], shape[1] // 32))).astype(np.uint8)
        return packed, scales
    a = _rng(seed, w.weights_id, tid, e).standard_normal(shape, dtype=np.float32)
    a *= np.float32(w.sigma_expert)
    if w.weight == "bf16":
        return bf16_bits(a)
    amax = np.abs(a).max(axis=1)
    scale = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    q = _e4m3_codes(a / safe[:, None])
    return q, scale


class ExpertSource:
    """Lazily generated expert weights on the host, one expert at a time.

    get(which, e) returns what expert_matrix() returns; results are cached.
    prefetch(experts) generates a set of experts with a thread pool.
    """

    def __init__(self, w: Workload, seed: int = 0, threads: Optional[int] = None):
        self.w, self.seed = w, seed
        self.threads = threads or min(16, len(os.sched_getaffinity(0)))
        self._cache = {}
        self._lock = threading.Lock()

    def get(self, which: str, e: int):
        key = (which, int(e))
        with self._lock:
            if key in self._cache:
                return self._cache[key]
        v = expert_matrix(self.w, self.seed, which, int(e))
        with self._lock:
            self._cache[key] = v
        return v

    def prefetch(self, experts):
        keys = [(wh, int(e)) for e in experts for wh in ("gate", "up", "down")]
        with ThreadPoolExecutor(self.threads) as ex:
            list(ex.map(lambda k: self.get(*k), keys))

    def drop(self):
        self._cache.clear()


def device_expert_weights(w: Workload, seed: int, device, threads: Optional[int] = None, log=None):
    """All E experts' matrices as device tensors, generated on the host expert by expert.

    Returns dict(gate, up, down) of [E, out, in] tensors (bf16, or uint8 e4m3
    codes) and, for fp8, s_gate, s_up, s_down [E, out] fp32 scales; for mxfp4,
    [E, out, in/2] packed codes and [E, out, in/32] uint8 E8M0 scales.
    """
    E = w.n_experts
    fp8 = w.weight == "fp8"
    mx = w.weight == "mxfp4"
    wdt = torch.uint8 if (fp8 or mx) else torch.bfloat16
    div = 2 if mx else 1
    out = {"gate": torch.empty(E, w.inter, w.hidden // div, dtype=wdt, device=device),
           "up": torch.empty(E, w.inter, w.hidden // div, dtype=wdt, device=device),
           "down": torch.empty(E, w.hidden, w.inter // div, dtype=wdt, device=device)}
    scales = {}
    if mx:
        scales = {"s_gate": torch.empty(E, w.inter, w.hidden // 32, dtype=torch.uint8, device=device),
                  "s_up": torch.empty(E, w.inter, w.hidden // 32, dtype=torch.uint8, device=device),
                  "s_down": torch.empty(E, w.hidden, w.inter // 32, dtype=torch.uint8, device=device)}
    if fp8:
        scales = {"s_gate": torch.empty(E, w.inter, dtype=torch.float32, device=device),
                  "s_up": torch.empty(E, w.inter, dtype=torch.float32, device=device),
                  "s_down": torch.empty(E, w.hidden, dtype=torch.float32, device=device)}
    threads = threads or min(16, len(os.sched_getaffinity(0)))

    def one(key):
        which, e = key
        v = expert_matrix(w, seed, which, e)
        return key, v

    keys = [(wh, e) for e in range(E) for wh in ("gate", "up", "down")]
    done = 0
    with ThreadPoolExecutor(threads) as ex:
        for (which, e), v in ex.map(one, keys):
            if fp8 or mx:
                q, sc = v
                out[which][e].copy_(torch.from_numpy(q))
                scales["s_" + which][e].copy_(torch.from_numpy(sc))
            else:
                out[which][e].copy_(torch.from_numpy(v.view(np.int16)).view(torch.bfloat16))
            done += 1
            if log and done % 192 == 0:
                log(f"expert weights: {done}/{len(keys)} matrices")
    out.update(scales)
    return out
