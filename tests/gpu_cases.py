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


def cfg_of(w):
    import sparse_moe_layer_top_amd as bm
    return bm.Config(w.hidden, w.inter, w.n_experts, w.n_groups, w.topk_groups, w.top_k, w.alpha,
                     {"bf16": bm.W_BF16, "fp8": bm.W_FP8_E4M3, "mxfp4": bm.W_MXFP4}[w.weight])


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


def run_forward(w, xt, wrt, bt, W):
    import sparse_moe_layer_top_amd as bm
    T = xt.shape[0]
    ids = torch.empty(T, w.top_k, dtype=torch.int32, device=dev())
    wts = torch.empty(T, w.top_k, dtype=torch.float32, device=dev())
    out = bm.beam_moe_forward(cfg_of(w), xt, wrt, bt, W["gate"], W["up"], W["down"], W.get("s_gate"),
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


def check_out(got_bits, ref_bits):
    assert np.all(np.isfinite(codecs.bf16_to_f64(got_bits)))
    mx, mn, mr = out_errors(got_bits, ref_bits)
    assert mx <= OUT_MAX_REL and mn < OUT_MEAN_REL, \
        f"max rel {mx:.3e}, mean|d|/rms {mn:.3e} (max|d|/rms {mr:.3e})"
    return mx, mn


def check_permutation(ids, offsets, sorted_pairs, pair_to_row, E):
    ref_off, ref_sp, ref_p2r = oracle.permute(ids, E)
    assert np.array_equal(offsets, ref_off), "expert offsets differ"
    assert np.array_equal(sorted_pairs, ref_sp), "sorted_pairs differ"
    assert np.array_equal(pair_to_row, ref_p2r), "pair_to_row differ"
