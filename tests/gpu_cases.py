"""Shared helpers for the GPU parity tests: upload seeded inputs, run the HIP
path through the binding, and compare with the oracle to the layer's bar:
ids and permutation bit-exact, weights within 1e-5 relative, and bf16 outputs
with

    max_i |d_i| / max(|ref_i|, rms(ref)) <= 2e-2     (max relative error)
    mean_i |d_i| / rms(ref)              <  1e-3     (mean absolute error)

where d = out_gpu - out_oracle.  The max error is relative to the element
itself, with the output RMS as its floor so that near-zero outputs (which come
from cancelling terms) are measured on the output's scale.  One bf16 ulp is at
most 2^-7 of the value, so rounding-order differences pass; an error measured
against the RMS alone would fail on a single ulp of an element a few times the
RMS."""
from __future__ import annotations

import sys
from concurrent.futures import ThreadPoolExecutor
import itertools
import os

import numpy as np
import torch

import oracle
from oracle import codecs
from synth import gen

OUT_MAX_REL = 2e-2
OUT_MEAN_REL = 1e-3
W_REL = 1e-5


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev():
    return torch.device("cuda:0")


def to_bf16(bits: np.ndarray, device=None):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device or dev())


def bits_of(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def cfg_of(w, layout=0):
    import sparse_moe_layer_top_amd as bm
    return bm.Config(w.hidden, w.inter, w.n_experts, w.n_groups, w.topk_groups, w.top_k, w.alpha,
                     {"bf16": bm.W_BF16, "fp8": bm.W_FP8_E4M3, "mxfp4": bm.W_MXFP4}[w.weight], layout)


def packed(W):
    """The expert weights W (row order) in fragment order, through the library's pack entry points:
    the weight matrices, and MXFP4 scale bytes (uint8); FP8 scales stay as they are."""
    import sparse_moe_layer_top_amd as bm
    P = dict(W)
    for k in ("gate", "up", "down"):
        P[k] = bm.beam_moe_pack_weights(W[k])
        s = W.get("s_" + k)
        if s is not None and s.dtype == torch.uint8:
            P["s_" + k] = bm.beam_moe_pack_scales(s)
    torch.cuda.synchronize()
    return P


def guarded(w, seed=0):
    spec = oracle.LayerSpec.of(w)
    x, wr, b, _ = gen.guarded_router_inputs(w, seed, lambda x, wr, b: oracle.gap_violations(spec, x, wr, b))
    return spec, x, wr, b


def router_tensors(x, wr, b):
    d = dev()
    return to_bf16(x), torch.from_numpy(wr).to(d), torch.from_numpy(b).to(d)


def host_expert_weights(w, seed=0):
    """Tiny layers: all experts stacked on the host and uploaded (plus the source for the oracle)."""
    src = gen.ExpertSource(w, seed)
    d = dev()
    if w.weight == "bf16":
        t = {k: to_bf16(np.stack([src.get(k, e) for e in range(w.n_experts)])) for k in ("gate", "up", "down")}
    else:
        t = {}
        for k in ("gate", "up", "down"):
            t[k] = torch.from_numpy(np.stack([src.get(k, e)[0] for e in range(w.n_experts)])).to(d)
            t["s_" + k] = torch.from_numpy(np.stack([src.get(k, e)[1] for e in range(w.n_experts)])).to(d)
    return t, src


def run_forward(w, xt, wrt, bt, W, layout=0):
    import sparse_moe_layer_top_amd as bm
    T = xt.shape[0]
    ids = torch.empty(T, w.top_k, dtype=torch.int32, device=dev())
    wts = torch.empty(T, w.top_k, dtype=torch.float32, device=dev())
    out = bm.beam_moe_forward(cfg_of(w, layout), xt, wrt, bt, W["gate"], W["up"], W["down"], W.get("s_gate"),
                              W.get("s_up"), W.get("s_down"), topk_ids_out=ids, topk_w_out=wts)
    torch.cuda.synchronize()
    return out, ids, wts


def check_ids_w(ids_gpu, w_gpu, ids_ref, w_ref):
    ids_gpu = np.asarray(ids_gpu)
    assert ids_gpu.shape == ids_ref.shape
    bad = np.nonzero((ids_gpu != ids_ref).any(axis=1))[0]
    assert len(bad) == 0, f"{len(bad)} tokens with different expert ids, first {bad[:5]}"
    rel = np.abs(np.asarray(w_gpu, np.float64) - w_ref) / np.abs(w_ref)
    assert rel.max() <= W_REL, f"weight rel err {rel.max():.3e}"


def out_errors(got_bits, ref_bits):
    """(max relative error with the RMS floor, mean abs error / RMS, max abs error / RMS)."""
    g = codecs.bf16_to_f64(got_bits)
    r = codecs.bf16_to_f64(ref_bits)
    rms = np.sqrt(np.mean(r * r))
    d = np.abs(g - r)
    return (d / np.maximum(np.abs(r), rms)).max(), d.mean() / rms, d.max() / rms


def check_out(got_bits, ref_bits, what="output"):
    """The output bar; every call logs both readings of the max error (element-relative with the
    RMS floor, and relative to the RMS alone) and the mean error."""
    assert np.all(np.isfinite(codecs.bf16_to_f64(got_bits)))
    mx, mn, mr = out_errors(got_bits, ref_bits)
    say(f"  {what}: {np.size(got_bits)} values, max|d|/max(|ref|,rms) {mx:.3e}, max|d|/rms {mr:.3e}, "
        f"mean|d|/rms {mn:.3e}")
    assert mx <= OUT_MAX_REL and mn < OUT_MEAN_REL, \
        f"max rel {mx:.3e}, mean|d|/rms {mn:.3e} (max|d|/rms {mr:.3e})"
    return mx, mn


def bf16_order(bits) -> np.ndarray:
    """bf16 bit patterns -> integers in the order of their values (+0 and -0 both 0), so the
    difference of two is their distance in bf16 steps."""
    b = np.asarray(bits, np.uint16).astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def check_within_ulp(got_bits, ref_bits, ulps=1, what="values"):
    """Every element within `ulps` bf16 steps of the reference; returns the fraction that is exact."""
    d = np.abs(bf16_order(got_bits) - bf16_order(ref_bits))
    assert d.max(initial=0) <= ulps, f"{what}: {int((d > ulps).sum())} elements more than {ulps} bf16 step(s) off"
    frac = float((d == 0).mean()) if d.size else 1.0
    say(f"  {what}: within {ulps} bf16 step(s), exact on {100 * frac:.4f}% of {d.size}")
    return frac


def bf16_spacing(x) -> np.ndarray:
    """Spacing of bf16 values at |x| (the smallest normal spacing for 0 and subnormals)."""
    a = np.maximum(np.abs(np.asarray(x, np.float64)), 2.0 ** -126)
    return np.exp2(np.floor(np.log2(a)) - 7)


def check_permutation(ids, offsets, sorted_pairs, pair_to_row, E):
    ref_off, ref_sp, ref_p2r = oracle.permute(ids, E)
    assert np.array_equal(offsets, ref_off), "expert offsets differ"
    assert np.array_equal(sorted_pairs, ref_sp), "sorted_pairs differ"
    assert np.array_equal(pair_to_row, ref_p2r), "pair_to_row differ"


def oracle_forward_threads(spec, x_bits, wr, b, weights, threads=None):
    """oracle.forward's steps (route, permute, one expert at a time, combine), with the experts
    handed to a thread pool: the same oracle functions on the same rows, only run side by side."""
    x_bits = np.asarray(x_bits, np.uint16)
    T, K = x_bits.shape[0], spec.top_k
    ids, w = oracle.route(spec, x_bits, wr, b)
    offsets, sorted_pairs, pair_to_row = oracle.permute(ids, spec.n_experts)
    y = np.zeros((T * K, spec.hidden), np.uint16)

    def one(e):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if lo == hi:
            return
        X = codecs.bf16_to_f64(x_bits[sorted_pairs[lo:hi] // K])
        y[lo:hi] = oracle.expert_rows(spec, X, weights("gate", e), weights("up", e), weights("down", e))

    with ThreadPoolExecutor(threads or min(16, len(os.sched_getaffinity(0)))) as ex:
        list(ex.map(one, range(spec.n_experts)))
    return dict(ids=ids, w=w, out=oracle.combine(y, w, pair_to_row, T, K))


def coverage_sample(rid, n_experts, n_min=128, span=576, seed=0):
    """Tokens for output parity at a real shape: every token of the most loaded expert up to `span`
    of its permuted rows, plus its last `span // 2` rows (so that the rows of one expert cover every
    position of a row tile of any height up to span / 2, the first tile and the last), the batch's
    first and last token, and seeded random tokens up to n_min in all.  Permuted row r of expert e
    is the r-th token, in ascending order, routed to e."""
    load = np.bincount(np.asarray(rid).ravel(), minlength=n_experts)
    e = int(load.argmax())
    toks = np.nonzero((rid == e).any(axis=1))[0]
    picks = [toks[:span], toks[-(span // 2):], [0, len(rid) - 1]]
    sample = np.unique(np.concatenate(picks))
    rng = np.random.default_rng(seed)
    while len(sample) < n_min:
        sample = np.unique(np.concatenate([sample, rng.choice(len(rid), n_min - len(sample), replace=False)]))
    return sample, e, int(load[e])


def check_valid_selection(spec, s, ids, wts, tol=1e-6):
    """Routing of near-tie tokens (score gaps below the guard), where several selections are correct:
    the ids are K distinct ascending experts inside some Gk groups that form a top-Gk of the oracle's
    group scores to within tol, they form a top-K of the oracle's scores among those groups' experts
    to within tol, and the weights are alpha * s / sum(s) over the chosen ids (to 1e-5)."""
    s = np.asarray(s, np.float32)
    T = s.shape[0]
    gsz, G, Gk, K = spec.group_size, spec.n_groups, spec.topk_groups, spec.top_k
    assert ids.shape == (T, K) and np.all(np.diff(ids, axis=1) > 0) and ids.min() >= 0 and ids.max() < spec.n_experts
    gs = oracle.moe._group_scores(s, spec).astype(np.float64)
    for t in range(T):
        used = sorted(set((ids[t] // gsz).tolist()))
        assert len(used) <= Gk, f"token {t}: ids span {len(used)} groups"
        rest = [g for g in range(G) if g not in used]
        ok = False
        for extra in itertools.combinations(rest, Gk - len(used)):
            kept = set(used) | set(extra)
            out = [g for g in range(G) if g not in kept]
            if out and min(gs[t, g] for g in kept) < max(gs[t, g] for g in out) - tol:
                continue                       # not a top-Gk of the group scores within tol
            cand = [e for g in sorted(kept) for e in range(g * gsz, (g + 1) * gsz) if e not in set(ids[t])]
            if cand and float(s[t, ids[t]].min()) < float(s[t, cand].max()) - tol:
                continue                       # not a top-K inside these groups within tol
            ok = True
            break
        assert ok, f"token {t}: ids {ids[t]} are no top-{K} inside any valid top-{Gk} groups"
    ref_w = oracle.combine_weights(s, ids.astype(np.int64), spec.alpha)
    rel = np.abs(np.asarray(wts, np.float64) - ref_w) / np.abs(ref_w)
    assert rel.max() <= W_REL, f"near-tie weight rel err {rel.max():.3e}"
