"""Plain CPU definition of the Beam MoE block forward pass (test infrastructure only).

What the layer computes is stated on the pages (Reflection Beam 1.0 overview,
agentlenshq.com, section "Mixture of Experts: 256 experts, 8 routed per token";
repeated on the aixai.ru page, section "256 experts per layer", and on the
dothoosh.com page, section "Architecture and memory efficiency"):

  * each MoE layer has 256 experts, each a SwiGLU MLP of intermediate size 2560;
  * the router follows DeepSeek-V3's group-limited scheme: a sigmoid scores all
    256 experts, the experts are split into 8 groups of 32, each group is ranked
    by the sum of its two highest scores, the best 4 groups are kept, and the
    best 8 experts inside them are chosen;
  * there is no shared expert;
  * expert outputs are combined with normalised router weights and scaled by 2.5.

The same overview page (section "Residual stream ...") lists where the
implementation pins FP32: the router and the SwiGLU product among them.

Readings this oracle takes where the pages are silent:
  * router logits z = x . W_router + b with an optional fp32 bias column b
    (zero unless a workload supplies one); scores s = 1 / (1 + exp(-z));
  * groups are contiguous id ranges; ties at a selection boundary go to the
    lower group index / lower expert id (inputs are drawn so that no boundary
    gap is below 1e-6, so ties never decide a result);
  * the 8 weights are normalised over the 8 chosen scores, and the 2.5 scale is
    applied to the weights (so they sum to 2.5);
  * the 8 ids of a token are listed in ascending expert id; combine sums them in
    that order;
  * expert e computes down(SiLU(gate . x) * (up . x)), no biases, weights stored
    [out, in]; linear outputs are rounded to bf16 (the model dtype): h after the
    SwiGLU product, y after the down projection, and the combined output;
  * fp8 weights are OCP e4m3 codes with one fp32 scale per output channel; the
    oracle dequantises the same bytes as fp32(decode(q) * scale);
  * MXFP4 weights (the MI355X analogue of the pages' NVFP4 checkpoint) are E2M1
    codes, two per byte, with one E8M0 scale per 32 consecutive inputs of an
    output row; their values e2m1(q) * 2^(e-127) are exact (oracle/codecs.py).

Arithmetic: every dot product accumulates in float64 and is rounded once to
float32 (f32) at the point the layer rounds; bf16 values enter exactly.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Callable

import numpy as np

from .codecs import bf16_round_bits, bf16_to_f64, e4m3_decode, f32, mxfp4_dequant

GAP_GUARD = 1e-6


@dataclass(frozen=True)
class LayerSpec:
    hidden: int
    inter: int
    n_experts: int
    n_groups: int
    topk_groups: int
    top_k: int
    alpha: float
    weight: str = "bf16"   # "bf16" | "fp8" | "mxfp4"

    @staticmethod
    def of(w) -> "LayerSpec":
        return LayerSpec(w.hidden, w.inter, w.n_experts, w.n_groups, w.topk_groups,
                         w.top_k, w.alpha, w.weight)

    @property
    def group_size(self) -> int:
        return self.n_experts // self.n_groups


# ------------------------------------------------------------- router ------

def router_logits(x_bits, w_router, b_router) -> np.ndarray:
    """z[t,e] = f32( sum_h x[t,h] * W_router[h,e] + b[e] ), accumulated in fp64.

    The router is one of the places the pages pin to FP32 (overview page,
    section "Residual stream"); x (bf16) enters exactly.
    """
    x = bf16_to_f64(x_bits)
    z = x @ np.asarray(w_router, np.float64)
    if b_router is not None:
        z = z + np.asarray(b_router, np.float64)[None, :]
    return f32(z)


def router_scores(x_bits, w_router, b_router) -> np.ndarray:
    """s = f32( 1 / (1 + exp(-z)) ): the sigmoid over all experts (section "Mixture of Experts")."""
    z = router_logits(x_bits, w_router, b_router).astype(np.float64)
    return f32(1.0 / (1.0 + np.exp(-z)))


def _group_scores(s: np.ndarray, spec: LayerSpec) -> np.ndarray:
    """Group score = f32(top1 + top2) of the group's sigmoid scores (a group holds at least two experts)."""
    if spec.group_size < 2:
        raise ValueError("a group's score is the sum of its two best scores: groups need two experts or more")
    T = s.shape[0]
    sg = np.sort(s.reshape(T, spec.n_groups, spec.group_size).astype(np.float64), axis=2)
    return f32(sg[:, :, -1] + sg[:, :, -2])


def select_experts(s: np.ndarray, spec: LayerSpec):
    """Group-limited top-k (section "Mixture of Experts").

    Returns (ids [T,K] ascending expert id, kept_groups [T,Gk] by rank).
    Ranks use a stable sort of the negated keys, so an exact tie goes to the
    lower index.
    """
    T, E = s.shape
    gs = _group_scores(s, spec)
    kept = np.argsort(-gs.astype(np.float64), axis=1, kind="stable")[:, :spec.topk_groups]
    in_kept = np.zeros((T, spec.n_groups), bool)
    np.put_along_axis(in_kept, kept, True, axis=1)
    cand = np.repeat(in_kept, spec.group_size, axis=1)
    key = np.where(cand, s.astype(np.float64), -np.inf)
    chosen = np.argsort(-key, axis=1, kind="stable")[:, :spec.top_k]
    ids = np.sort(chosen, axis=1).astype(np.int32)
    return ids, kept


def combine_weights(s: np.ndarray, ids: np.ndarray, alpha: float) -> np.ndarray:
    """w_k = f32( f32(s_k / den) * alpha ), den = sequential f32 sum of the chosen scores.

    "Normalised router weights ... scaled by 2.5" (section "Mixture of Experts").
    """
    sel = np.take_along_axis(s, ids, axis=1).astype(np.float32)
    den = np.zeros(sel.shape[0], np.float32)
    for k in range(sel.shape[1]):
        den = f32(den.astype(np.float64) + sel[:, k])
    q = (sel / den[:, None]).astype(np.float32)          # IEEE binary32 division
    return (q * np.float32(alpha)).astype(np.float32)


def route(spec: LayerSpec, x_bits, w_router, b_router):
    """Router + group-limited selection + weights: (ids [T,K] int32, w [T,K] fp32)."""
    s = router_scores(x_bits, w_router, b_router)
    ids, _ = select_experts(s, spec)
    return ids, combine_weights(s, ids, spec.alpha)


def gap_violations(spec: LayerSpec, x_bits, w_router, b_router, guard: float = GAP_GUARD):
    """Token rows whose fp32 score gap at a selection boundary is below `guard`.

    The two boundaries: between the Gk-th and (Gk+1)-th group score, and between
    the K-th and (K+1)-th candidate score inside the kept groups.
    """
    s = router_scores(x_bits, w_router, b_router)
    gs = np.sort(_group_scores(s, spec).astype(np.float64), axis=1)[:, ::-1]
    bad = np.zeros(s.shape[0], bool)
    if spec.topk_groups < spec.n_groups:
        bad |= (gs[:, spec.topk_groups - 1] - gs[:, spec.topk_groups]) < guard
    _, kept = select_experts(s, spec)
    in_kept = np.zeros((s.shape[0], spec.n_groups), bool)
    np.put_along_axis(in_kept, kept, True, axis=1)
    cand = np.repeat(in_kept, spec.group_size, axis=1)
    key = np.sort(np.where(cand, s.astype(np.float64), -np.inf), axis=1)[:, ::-1]
    n_cand = spec.topk_groups * spec.group_size
    if spec.top_k < n_cand:
        bad |= (key[:, spec.top_k - 1] - key[:, spec.top_k]) < guard
    return np.nonzero(bad)[0]


# -------------------------------------------------------- permutation ------

def permute(ids: np.ndarray, n_experts: int):
    """Token -> expert permutation of the T*K (token, slot) pairs.

    On one GPU, "tokens move to their experts and the results are merged back"
    (breadlab.ai Beam inference post, section "Reading 23B active and 501B
    resident separately") becomes a grouping of the pairs by expert.  Pair
    p = t*K + k; pairs are grouped by expert id, ascending p inside an expert.
    Returns (expert_offsets [E+1], sorted_pairs [T*K], pair_to_row [T*K]).
    """
    flat = np.asarray(ids, np.int64).ravel()
    sorted_pairs = np.argsort(flat, kind="stable").astype(np.int32)
    counts = np.bincount(flat, minlength=n_experts)
    offsets = np.zeros(n_experts + 1, np.int32)
    offsets[1:] = np.cumsum(counts)
    pair_to_row = np.empty_like(sorted_pairs)
    pair_to_row[sorted_pairs] = np.arange(len(flat), dtype=np.int32)
    return offsets, sorted_pairs, pair_to_row


# --------------------------------------------------------- expert math -----

def _dequant(spec: LayerSpec, mat) -> np.ndarray:
    """Expert matrix as float64: bf16 bits exactly, fp32(decode(q) * scale) for fp8, e2m1 * 2^(e-127) for mxfp4."""
    if spec.weight == "bf16":
        return bf16_to_f64(mat)
    if spec.weight == "mxfp4":
        packed, e8 = mat
        return mxfp4_dequant(packed, e8)
    q, scale = mat
    return f32(e4m3_decode(q).astype(np.float32).astype(np.float64)
               * np.asarray(scale, np.float64)[:, None]).astype(np.float64)


def expert_rows(spec: LayerSpec, X: np.ndarray, wg, wu, wd) -> np.ndarray:
    """One SwiGLU expert on rows X (float64 values of bf16 inputs) -> bf16 bits.

    g = f32(X Wg^T), u = f32(X Wu^T); a = f32(SiLU(g)) with SiLU(g) = g/(1+e^-g);
    h = bf16(f32(a * u)) (the SwiGLU product in FP32); y = bf16(f32(h Wd^T)).
    """
    g = f32(X @ _dequant(spec, wg).T).astype(np.float64)
    u = f32(X @ _dequant(spec, wu).T).astype(np.float64)
    a = f32(g / (1.0 + np.exp(-g))).astype(np.float64)
    h = bf16_to_f64(bf16_round_bits(f32(a * u)))
    return bf16_round_bits(f32(h @ _dequant(spec, wd).T))


def combine(y_bits: np.ndarray, w: np.ndarray, pair_to_row: np.ndarray, T: int, K: int):
    """out[t] = bf16( sum_k f32(w[t,k] * y[row(t,k)]) ), summed in f32 in slot order."""
    y = bf16_to_f64(y_bits)
    acc = np.zeros((T, y.shape[1]), np.float32)
    rows = np.asarray(pair_to_row).reshape(T, K)
    for k in range(K):
        term = f32(np.asarray(w[:, k], np.float64)[:, None] * y[rows[:, k]])
        acc = f32(acc.astype(np.float64) + term)
    return bf16_round_bits(acc)


def forward(spec: LayerSpec, x_bits, w_router, b_router,
            weights: Callable[[str, int], object]):
    """The whole block: route, permute, experts, combine.

    weights(which, e) returns expert e's matrix for which in {"gate","up","down"}
    (bf16 bits, or (e4m3 codes, scales) for fp8), shaped [out, in].
    Returns a dict with ids, w, expert_offsets, sorted_pairs, pair_to_row, y
    (bf16 bits, permuted rows) and out (bf16 bits [T, H]).
    """
    x_bits = np.asarray(x_bits, np.uint16)
    T, K = x_bits.shape[0], spec.top_k
    ids, w = route(spec, x_bits, w_router, b_router)
    offsets, sorted_pairs, pair_to_row = permute(ids, spec.n_experts)
    y = np.zeros((T * K, spec.hidden), np.uint16)
    for e in range(spec.n_experts):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if lo == hi:
            continue
        tok = sorted_pairs[lo:hi] // K
        X = bf16_to_f64(x_bits[tok])
        y[lo:hi] = expert_rows(spec, X, weights("gate", e), weights("up", e), weights("down", e))
    out = combine(y, w, pair_to_row, T, K)
    return dict(ids=ids, w=w, expert_offsets=offsets, sorted_pairs=sorted_pairs,
                pair_to_row=pair_to_row, y=y, out=out)


def dense_mlp(x_bits, wg, wu, wd, weight: str = "bf16") -> np.ndarray:
    """The dense SwiGLU MLP of Beam's first 3 layers (Reflection Beam 1.0 overview,
    section "Architecture"): down(SiLU(gate x) * (up x)) on every row, with one
    expert's arithmetic and rounding points (expert_rows); no router, no combine.

    x_bits [T, H] bf16 bits; wg, wu [I, H], wd [H, I] as bf16 bits, or
    (e4m3 codes, scales) pairs when weight == "fp8", or (packed E2M1 codes,
    E8M0 scales) when weight == "mxfp4".  Returns bf16 bits [T, H].
    """
    x_bits = np.asarray(x_bits, np.uint16)
    H = x_bits.shape[1]
    I = (wg if weight == "bf16" else wg[0]).shape[0]
    spec = LayerSpec(H, I, 1, 1, 1, 1, 1.0, weight)
    return expert_rows(spec, bf16_to_f64(x_bits), wg, wu, wd)
