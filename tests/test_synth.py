"""Input generators: determinism, the gap guard, load balance and skew, fp8 scales."""
import numpy as np
import pytest

import oracle
from synth import gen


def test_router_inputs_deterministic():
    w = gen.workload("tiny")
    a = gen.router_inputs(w, 3)
    b = gen.router_inputs(w, 3)
    c = gen.router_inputs(w, 4)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)
    assert not np.array_equal(a[0], c[0])


def test_expert_matrix_per_expert_stream():
    w = gen.workload("tiny")
    g5 = gen.expert_matrix(w, 0, "gate", 5)
    assert g5.shape == (w.inter, w.hidden) and g5.dtype == np.uint16
    assert np.array_equal(g5, gen.expert_matrix(w, 0, "gate", 5))
    assert not np.array_equal(g5, gen.expert_matrix(w, 0, "up", 5))
    d = gen.bf16_bits_to_f32(gen.expert_matrix(w, 0, "down", 5))
    assert d.shape == (w.hidden, w.inter)
    assert abs(d.std() - 0.02) < 0.002


def test_fp8_scales_rowmax():
    w = gen.workload("fp8_decode")
    q, s = gen.expert_matrix(w, 0, "gate", 0)
    assert q.dtype == np.uint8 and q.shape == (w.inter, w.hidden) and s.shape == (w.inter,)
    a = np.random.default_rng([0, w.weights_id, gen.WG_ID, 0]).standard_normal((w.inter, w.hidden), dtype=np.float32)
    a *= np.float32(w.sigma_expert)
    assert np.array_equal(s, (np.abs(a).max(axis=1) / np.float32(448.0)).astype(np.float32))
    assert not np.any((q & 0x7F) == 0x7F)          # no NaN codes


def test_balanced_prefill_loads():
    """Fitted bias: max expert load within 1.1x of the mean 256 on the guarded inputs."""
    w = gen.workload("prefill")
    spec = oracle.LayerSpec.of(w)
    x, wr, b, n = gen.guarded_router_inputs(w, 0, lambda x, wr, b: oracle.gap_violations(spec, x, wr, b))
    ids, _ = oracle.route(spec, x, wr, b)
    ld = np.bincount(ids.ravel(), minlength=spec.n_experts)
    mean = w.T * w.top_k / spec.n_experts
    assert mean == 256 and ld.max() <= 1.1 * mean and ld.min() > 0


def test_skew_loads():
    w = gen.workload("skew")
    spec = oracle.LayerSpec.of(w)
    x, wr, b = gen.router_inputs(w, 0)
    ids, _ = oracle.route(spec, x, wr, b)
    ld = np.bincount(ids.ravel(), minlength=spec.n_experts)
    mean = w.T * w.top_k / spec.n_experts
    assert ld.max() > 3 * mean          # heavy experts
    assert (ld == 0).sum() >= 1          # some experts receive no token


def test_stored_bias_is_reproducible():
    """Re-running the fit gives the stored bit patterns."""
    from oracle import fit_prefill_bias
    b, it, ratio = fit_prefill_bias.fit(0)
    assert np.array_equal(b, gen.load_balanced_bias(0, 256))
