"""CPU checks of the GPU tests' own helpers (tests/gpu_cases.py): the validity check for
near-tie routings accepts the oracle's selection and rejects planted wrong ones, the bf16
step distance counts steps across zero, and the coverage sample takes every permuted row of
the most loaded expert."""
import numpy as np
import pytest

import oracle
from synth import gen
from tests import gpu_cases as C


def _tiny_routing(T=200, seed=3):
    w = gen.workload("tiny", T)
    spec = oracle.LayerSpec.of(w)
    x, wr, b = gen.router_inputs(w, seed)
    s = oracle.router_scores(x, wr, b)
    ids, wts = oracle.route(spec, x, wr, b)
    return spec, s, ids, wts


def test_valid_selection_accepts_the_oracle():
    spec, s, ids, wts = _tiny_routing()
    C.check_valid_selection(spec, s, ids, wts, tol=1e-6)


def test_valid_selection_rejects_a_swapped_expert():
    spec, s, ids, wts = _tiny_routing()
    bad = ids.copy()
    t = 0
    chosen = set(bad[t].tolist())
    # the lowest-scoring expert outside the selection, kept in order
    worst = int(np.argmin(np.where(np.isin(np.arange(spec.n_experts), list(chosen)), np.inf, s[t])))
    bad[t, 0] = worst
    bad[t] = np.sort(bad[t])
    with pytest.raises(AssertionError):
        C.check_valid_selection(spec, s[:1], bad[:1], oracle.combine_weights(s[:1], bad[:1], spec.alpha))


def test_valid_selection_rejects_a_dropped_group_rule():
    """Plain top-8 over all experts (no group limit) is caught where it differs."""
    spec, s, ids, wts = _tiny_routing()
    plain = np.sort(np.argsort(-s.astype(np.float64), axis=1, kind="stable")[:, :spec.top_k], axis=1)
    diff = np.nonzero((plain != ids).any(axis=1))[0]
    assert len(diff) > 0
    t = diff[:1]
    with pytest.raises(AssertionError):
        C.check_valid_selection(spec, s[t], plain[t], oracle.combine_weights(s[t], plain[t], spec.alpha))


def test_valid_selection_rejects_wrong_weights():
    spec, s, ids, wts = _tiny_routing()
    with pytest.raises(AssertionError):
        C.check_valid_selection(spec, s[:4], ids[:4], wts[:4] * np.float32(1.001))


def test_bf16_steps_across_zero():
    a = np.array([0x0001, 0x8001, 0x0000, 0x8000, 0x3F80, 0x3F81], np.uint16)
    b = np.array([0x8001, 0x0000, 0x8000, 0x0000, 0x3F81, 0x3F80], np.uint16)
    assert list(np.abs(C.bf16_order(a) - C.bf16_order(b))) == [2, 1, 0, 0, 1, 1]


def test_coverage_sample_takes_every_row_of_the_busiest_expert():
    spec, s, ids, wts = _tiny_routing(T=1000)
    sample, e, ne = C.coverage_sample(ids, spec.n_experts, n_min=300, span=64, seed=0)
    rows_of_e = np.nonzero((ids == e).any(axis=1))[0]
    assert ne == len(rows_of_e) and ne > 64
    assert set(rows_of_e[:64]) <= set(sample) and set(rows_of_e[-32:]) <= set(sample)
    assert len(sample) >= 300 and 0 in sample and 999 in sample
