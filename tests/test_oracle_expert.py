"""Pins for the oracle's expert math and combine.

* naive loops with exactly rounded dot products (math.fsum) on the tiny layer;
* identical experts: the layer reduces to 2.5 x one dense SwiGLU MLP
  (the textbook form down(SiLU(gate x) * up x)), computed here with torch;
* every token routed to the same 8 experts: the grouped GEMM becomes 8 dense
  GEMMs;
* fp8 weights dequantised by torch's e4m3 cast.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import codecs
from synth import gen


def _bf16_bits_t(t32):
    return t32.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _bits_to_t(bits):
    return torch.from_numpy(codecs.bf16_to_f64(bits))


def _ulps_bf16(a, b):
    ia = a.astype(np.int32)
    ib = b.astype(np.int32)
    # map sign-magnitude to an ordered integer line
    ia = np.where(ia & 0x8000, 0x8000 - ia, ia)
    ib = np.where(ib & 0x8000, 0x8000 - ib, ib)
    return np.abs(ia - ib)


def _assert_rounds_to(out_bits, v, rel=1e-6):
    """out must be bf16(v); where v lies within `rel` of a bf16 rounding midpoint
    (fp32 summation noise decides those), either neighbour is accepted."""
    ref = codecs.bf16_round_bits(v.astype(np.float32))
    d = _ulps_bf16(out_bits, ref)
    r = codecs.bf16_to_f64(ref)
    ulp = np.abs(np.spacing(r.astype(np.float32)).astype(np.float64)) * 2 ** 16
    near_mid = np.abs(np.abs(v - r) - ulp / 2) <= rel * np.abs(v) + 1e-30
    assert d.max() <= 1
    assert np.all((d == 0) | near_mid), int(((d != 0) & ~near_mid).sum())


def _tiny_src(seed=0):
    w = gen.workload("tiny")
    return w, oracle.LayerSpec.of(w), gen.ExpertSource(w, seed)


def test_expert_naive_loops():
    w, spec, src = _tiny_src()
    x, _, _ = gen.router_inputs(w, 0)
    X = codecs.bf16_to_f64(x[:6])
    e = 5
    wg, wu, wd = (codecs.bf16_to_f64(src.get(k, e)) for k in ("gate", "up", "down"))
    y = oracle.expert_rows(spec, X, src.get("gate", e), src.get("up", e), src.get("down", e))
    ref = np.zeros_like(y)
    for r in range(X.shape[0]):
        h = []
        for i in range(spec.inter):
            g = float(np.float32(math.fsum(X[r, hh] * wg[i, hh] for hh in range(spec.hidden))))
            u = float(np.float32(math.fsum(X[r, hh] * wu[i, hh] for hh in range(spec.hidden))))
            a = float(np.float32(g / (1.0 + math.exp(-g))))
            h.append(float(codecs.bf16_to_f64(codecs.bf16_round_bits(np.float32(a * u)))))
        for n in range(spec.hidden):
            acc = np.float32(math.fsum(h[i] * wd[n, i] for i in range(spec.inter)))
            ref[r, n] = codecs.bf16_round_bits(np.array([acc], np.float32))[0]
    d = _ulps_bf16(y, ref)
    assert d.max() <= 1 and (d == 0).mean() > 0.99


def _identical_expert_weights(w, src, which_e=3):
    mats = {k: src.get(k, which_e) for k in ("gate", "up", "down")}
    return lambda which, e: mats[which]


@pytest.mark.parametrize("seed", [0, 1])
def test_identical_experts_equal_dense_mlp(seed):
    """With identical experts the combine weights sum to 2.5, so out = bf16(2.5 * y_dense)."""
    w, spec, src = _tiny_src(seed)
    x, wr, b = gen.router_inputs(w, seed)
    weights = _identical_expert_weights(w, src)
    res = oracle.forward(spec, x, wr, b, weights)
    X = _bits_to_t(x)
    Wg, Wu, Wd = (_bits_to_t(weights(k, 0)) for k in ("gate", "up", "down"))
    g = (X @ Wg.T).to(torch.float32)
    u = (X @ Wu.T).to(torch.float32)
    h = (F.silu(g.double()).to(torch.float32) * u).to(torch.bfloat16).double()
    y = (h @ Wd.T).to(torch.float32).to(torch.bfloat16).double()
    v = (2.5 * y).numpy()                       # exact: y has 8 significant bits
    _assert_rounds_to(res["out"], v)


def test_shared_route_is_dense_per_expert():
    """A large bias on 8 experts of 2 groups sends every token to them: each is a dense MLP over all T."""
    w, spec, src = _tiny_src(0)
    x, wr, _ = gen.router_inputs(w, 0)
    chosen = [0, 1, 2, 3, 8, 9, 10, 11]        # groups 0 and 2 of size 4
    b = np.full(spec.n_experts, -20.0, np.float32)
    b[chosen] = 20.0
    res = oracle.forward(spec, x, wr, b, src.get)
    assert (res["ids"] == np.array(chosen)).all()
    X = _bits_to_t(x)
    acc = torch.zeros(w.T, spec.hidden, dtype=torch.float32)
    wts = torch.from_numpy(res["w"])
    for k, e in enumerate(chosen):
        Wg, Wu, Wd = (_bits_to_t(src.get(n, e)) for n in ("gate", "up", "down"))
        g = (X @ Wg.T).to(torch.float32)
        u = (X @ Wu.T).to(torch.float32)
        h = (F.silu(g.double()).to(torch.float32) * u).to(torch.bfloat16).double()
        y = (h @ Wd.T).to(torch.float32).to(torch.bfloat16).to(torch.float32)
        acc = acc + wts[:, k:k + 1] * y
    d = _ulps_bf16(res["out"], _bf16_bits_t(acc))
    assert d.max() <= 1 and (d == 0).mean() > 0.98


def test_fp8_dequant_matches_torch_cast():
    w = gen.workload("fp8_decode")
    spec = oracle.LayerSpec.of(w)
    q, scale = gen.expert_matrix(w, 0, "down", 7)
    ref = (torch.from_numpy(q).view(torch.float8_e4m3fn).to(torch.float32)
           * torch.from_numpy(scale)[:, None]).double().numpy()
    got = oracle.moe._dequant(spec, (q, scale))
    assert np.array_equal(got, ref)
    # scale is the row max over 448: the largest code of each row decodes to 448
    assert np.all(np.abs(codecs.e4m3_decode(q)).max(axis=1) == 448.0)


def test_combine_fixed_order():
    """Combine sums slot by slot in f32; compare with an explicit per-element loop."""
    rng = np.random.default_rng(0)
    T, K, H = 5, 8, 16
    y = codecs.bf16_round_bits(rng.standard_normal((T * K, H)).astype(np.float32))
    wts = rng.uniform(0.1, 0.5, (T, K)).astype(np.float32)
    p2r = rng.permutation(T * K).astype(np.int32)
    out = oracle.combine(y, wts, p2r, T, K)
    yf = codecs.bf16_to_f64(y)
    for t in range(T):
        for n in range(H):
            acc = np.float32(0.0)
            for k in range(K):
                acc = np.float32(acc + np.float32(wts[t, k] * np.float32(yf[p2r[t * K + k], n])))
            assert out[t, n] == codecs.bf16_round_bits(np.array([acc], np.float32))[0]


def test_dense_mlp_naive_loops_and_moe_reduction():
    """The dense MLP oracle against exactly rounded loops, and against the MoE
    layer with 32 identical experts (out = bf16(2.5 * dense), exact: y has 8
    significant bits)."""
    w, spec, src = _tiny_src(0)
    x, wr, b = gen.router_inputs(w, 0)
    e = 7
    mats = [src.get(k, e) for k in ("gate", "up", "down")]
    y = oracle.dense_mlp(x[:4], *mats)
    X = codecs.bf16_to_f64(x[:4])
    wg, wu, wd = (codecs.bf16_to_f64(m) for m in mats)
    ref = np.zeros_like(y)
    for r in range(X.shape[0]):
        h = []
        for i in range(spec.inter):
            g = float(np.float32(math.fsum(X[r, hh] * wg[i, hh] for hh in range(spec.hidden))))
            u = float(np.float32(math.fsum(X[r, hh] * wu[i, hh] for hh in range(spec.hidden))))
            a = float(np.float32(g / (1.0 + math.exp(-g))))
            h.append(float(codecs.bf16_to_f64(codecs.bf16_round_bits(np.float32(a * u)))))
        for n in range(spec.hidden):
            ref[r, n] = codecs.bf16_round_bits(np.array([math.fsum(h[i] * wd[n, i] for i in range(spec.inter))],
                                                        np.float32))[0]
    d = _ulps_bf16(y, ref)
    assert d.max() <= 1 and (d == 0).mean() > 0.99
    full = oracle.dense_mlp(x, *mats)
    moe = oracle.forward(spec, x, wr, b, _identical_expert_weights(w, src, e))
    _assert_rounds_to(moe["out"], 2.5 * codecs.bf16_to_f64(full))
