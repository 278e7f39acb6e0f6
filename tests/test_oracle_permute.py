"""Pins for the oracle's token -> expert permutation: a pure-Python counting sort
(a different algorithm from the oracle's stable argsort) and the invariants."""
import numpy as np
import pytest

import oracle
from synth import gen


def _counting_sort(flat, E):
    buckets = [[] for _ in range(E)]
    for p, e in enumerate(flat):
        buckets[e].append(p)
    offsets = [0]
    for b in buckets:
        offsets.append(offsets[-1] + len(b))
    order = [p for b in buckets for p in b]
    return offsets, order


def check_permutation(ids, E, offsets, sorted_pairs, pair_to_row):
    T, K = ids.shape
    flat = ids.ravel()
    n = T * K
    assert offsets[0] == 0 and offsets[E] == n and (np.diff(offsets) >= 0).all()
    assert np.array_equal(np.diff(offsets), np.bincount(flat, minlength=E))
    assert np.array_equal(np.sort(sorted_pairs), np.arange(n))
    assert np.array_equal(pair_to_row[sorted_pairs], np.arange(n))
    for e in range(E):
        seg = sorted_pairs[offsets[e]:offsets[e + 1]]
        assert (flat[seg] == e).all()
        assert (np.diff(seg) > 0).all()          # ascending pair index (so ascending token)


@pytest.mark.parametrize("name,T", [("tiny", None), ("decode", None), ("skew", 1024), ("tiny", 1), ("tiny", 0)])
def test_permute_vs_counting_sort(name, T):
    w = gen.workload(name, T)
    spec = oracle.LayerSpec.of(w)
    x, wr, b = gen.router_inputs(w, 0)
    ids, _ = oracle.route(spec, x, wr, b)
    offsets, sp, p2r = oracle.permute(ids, spec.n_experts)
    ref_off, ref_order = _counting_sort(list(ids.ravel()), spec.n_experts)
    assert list(offsets) == ref_off
    assert list(sp) == ref_order
    check_permutation(ids, spec.n_experts, offsets, sp, p2r)


def test_permute_all_one_expert_block():
    """Every token routed to the same 8 experts: each expert holds all T tokens in order."""
    T, K, E = 37, 8, 64
    ids = np.tile(np.arange(8, 16, dtype=np.int32), (T, 1))
    offsets, sp, p2r = oracle.permute(ids, E)
    for k, e in enumerate(range(8, 16)):
        assert list(sp[offsets[e]:offsets[e + 1]]) == [t * K + k for t in range(T)]
    check_permutation(ids, E, offsets, sp, p2r)
