"""Planted mistakes in the oracle (on the CPU) must each fail one of its pins.

Each mutant swaps one oracle function for a plausible wrong version, runs the
pin tests that should catch it, and expects an AssertionError.
"""
import numpy as np
import pytest

import oracle
from oracle import codecs, moe
import tests.test_oracle_route as R
import tests.test_oracle_permute as P
import tests.test_oracle_expert as X


def _top1_group_scores(s, spec):
    T = s.shape[0]
    sg = np.sort(s.reshape(T, spec.n_groups, spec.group_size).astype(np.float64), axis=2)
    return codecs.f32(2 * sg[:, :, -1])


def _unnormalised_weights(s, ids, alpha):
    return (np.take_along_axis(s, ids, axis=1) * np.float32(alpha)).astype(np.float32)


def _no_alpha(s, ids, alpha):
    return moe.__dict__["_orig_combine_weights"](s, ids, 1.0)


def _wrong_sign_sigmoid(x_bits, w_router, b_router):
    z = moe.router_logits(x_bits, w_router, b_router).astype(np.float64)
    return codecs.f32(1.0 / (1.0 + np.exp(z)))


def _unstable_permute(ids, E):
    off, sp, p2r = moe.__dict__["_orig_permute"](ids, E)
    sp = sp.copy()
    for e in range(E):
        sp[off[e]:off[e + 1]] = sp[off[e]:off[e + 1]][::-1]
    p2r = np.empty_like(sp)
    p2r[sp] = np.arange(len(sp), dtype=np.int32)
    return off, sp, p2r


def _swapped_swiglu(spec, X_, wg, wu, wd):
    return moe.__dict__["_orig_expert_rows"](spec, X_, wu, wg, wd)


def _combine_wrong_index(y_bits, w, pair_to_row, T, K):
    return moe.__dict__["_orig_combine"](y_bits, w, np.argsort(pair_to_row), T, K)


def _dropped_bias(x_bits, w_router, b_router):
    return moe.__dict__["_orig_router_logits"](x_bits, w_router, None)


def _gap_variant(dg=0, dk=0, all_groups=False):
    """gap_violations with the group boundary at Gk + dg, the expert boundary at K + dk, or the
    expert candidates taken from every group."""
    def f(spec, x_bits, w_router, b_router, guard=moe.GAP_GUARD):
        s = moe.router_scores(x_bits, w_router, b_router)
        gs = np.sort(moe._group_scores(s, spec).astype(np.float64), axis=1)[:, ::-1]
        gk, k = spec.topk_groups + dg, spec.top_k + dk
        bad = (gs[:, gk - 1] - gs[:, gk]) < guard
        _, kept = moe.select_experts(s, spec)
        in_kept = np.zeros((s.shape[0], spec.n_groups), bool)
        np.put_along_axis(in_kept, kept, True, axis=1)
        cand = np.ones_like(s, bool) if all_groups else np.repeat(in_kept, spec.group_size, axis=1)
        key = np.sort(np.where(cand, s.astype(np.float64), -np.inf), axis=1)[:, ::-1]
        bad |= (key[:, k - 1] - key[:, k]) < guard
        return np.nonzero(bad)[0]
    f.__name__ = f"gap_dg{dg}_dk{dk}" + ("_all_groups" if all_groups else "")
    return f


MUTANTS = [
    ("_group_scores", _top1_group_scores, [lambda: R.test_selection_brute_force(0)]),
    ("combine_weights", _unnormalised_weights, [R.test_weights_exact_normalisation]),
    ("combine_weights", _no_alpha, [R.test_weights_exact_normalisation]),
    ("router_scores", _wrong_sign_sigmoid, [R.test_scores_are_sigmoid]),
    ("router_logits", _dropped_bias, [lambda: R.test_logits_exact_dot(0)]),
    ("permute", _unstable_permute, [lambda: P.test_permute_vs_counting_sort("tiny", None)]),
    ("expert_rows", _swapped_swiglu, [X.test_expert_naive_loops]),
    ("combine", _combine_wrong_index, [X.test_combine_fixed_order, lambda: X.test_identical_experts_equal_dense_mlp(0)]),
    ("gap_violations", _gap_variant(dg=-1), [R.test_gap_violations_boundary_positions]),
    ("gap_violations", _gap_variant(dg=+1), [R.test_gap_violations_boundary_positions]),
    ("gap_violations", _gap_variant(dk=-1), [R.test_gap_violations_boundary_positions]),
    ("gap_violations", _gap_variant(dk=+1), [R.test_gap_violations_boundary_positions]),
    ("gap_violations", _gap_variant(all_groups=True), [R.test_gap_violations_boundary_positions]),
]


@pytest.mark.parametrize("name,mutant,pins", MUTANTS, ids=[f"{m[0]}:{m[1].__name__}" for m in MUTANTS])
def test_mutant_is_caught(monkeypatch, name, mutant, pins):
    orig = getattr(moe, name)
    monkeypatch.setitem(moe.__dict__, "_orig_" + name, orig)
    monkeypatch.setattr(moe, name, mutant)
    # the pins call the package-level names too
    if hasattr(oracle, name):
        monkeypatch.setattr(oracle, name, mutant)
    for pin in pins:
        with pytest.raises(AssertionError):
            pin()
