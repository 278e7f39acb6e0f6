"""Pins for the oracle's router and group-limited selection.

The pages print no worked routing example, so the selection is pinned by brute
force over every subset on the tiny layer, by the plain top-k special case, and
by the invariants the layer's statement fixes (section "Mixture of Experts" of
the Reflection Beam 1.0 overview page): chosen experts lie in the 4 kept
groups, 8 distinct experts per token, weights sum to 2.5.
"""
import heapq
import itertools
import math

import numpy as np
import pytest
from scipy.special import expit

import oracle
from oracle import codecs
from synth import gen

SEEDS = [0, 1, 2, 3]


def _tiny(seed):
    w = gen.workload("tiny")
    spec = oracle.LayerSpec.of(w)
    x, wr, b, _ = gen.guarded_router_inputs(w, seed, lambda x, wr, b: oracle.gap_violations(spec, x, wr, b))
    return w, spec, x, wr, b


@pytest.mark.parametrize("seed", SEEDS)
def test_logits_exact_dot(seed):
    """z = f32(sum x*W + b): compare with exactly rounded sums (math.fsum) on a sample of entries."""
    w, spec, x, wr, b = _tiny(seed)
    b = np.random.default_rng(seed).standard_normal(spec.n_experts).astype(np.float32)
    z = oracle.router_logits(x, wr, b)
    xf = codecs.bf16_to_f64(x)
    rng = np.random.default_rng(100 + seed)
    for t, e in zip(rng.integers(0, w.T, 200), rng.integers(0, spec.n_experts, 200)):
        exact = math.fsum([xf[t, h] * float(wr[h, e]) for h in range(spec.hidden)] + [float(b[e])])
        ref = np.float32(exact)
        assert abs(float(z[t, e]) - float(ref)) <= abs(float(np.spacing(ref))), (t, e)


def test_scores_are_sigmoid():
    w, spec, x, wr, b = _tiny(0)
    s = oracle.router_scores(x, wr, b)
    z = oracle.router_logits(x, wr, b).astype(np.float64)
    ref = expit(z).astype(np.float32)
    assert np.max(np.abs(s.view(np.int32) - ref.view(np.int32))) <= 1
    assert (s > 0).all() and (s < 1).all()


def _brute_force_select(s_row, spec):
    g = spec.group_size
    gs = []
    for gi in range(spec.n_groups):
        vals = sorted((float(v) for v in s_row[gi * g:(gi + 1) * g]), reverse=True)
        gs.append(float(np.float32(vals[0] + vals[1])))
    # the kept set: every kept group score beats every dropped one
    winners = [c for c in itertools.combinations(range(spec.n_groups), spec.topk_groups)
               if min(gs[i] for i in c) > max(gs[i] for i in range(spec.n_groups) if i not in c)]
    assert len(winners) == 1
    kept = winners[0]
    cand = [e for gi in kept for e in range(gi * g, (gi + 1) * g)]
    best, best_sum = None, -1.0
    for c in itertools.combinations(cand, spec.top_k):
        sm = math.fsum(float(s_row[e]) for e in c)
        if sm > best_sum:
            best, best_sum = c, sm
    return sorted(best), sorted(kept)


@pytest.mark.parametrize("seed", SEEDS)
def test_selection_brute_force(seed):
    """All C(8,4)=70 group subsets and all C(16,8)=12870 expert subsets, per token."""
    w, spec, x, wr, b = _tiny(seed)
    s = oracle.router_scores(x, wr, b)
    ids, kept = oracle.select_experts(s, spec)
    for t in range(0, w.T, 4):   # 16 tokens per seed keeps this under a few seconds
        ref_ids, ref_kept = _brute_force_select(s[t], spec)
        assert list(ids[t]) == ref_ids
        assert sorted(kept[t]) == ref_kept


def test_single_group_is_plain_topk():
    """G = 1, Gk = 1 reduces group-limited selection to a plain top-K."""
    rng = np.random.default_rng(7)
    spec = oracle.LayerSpec(64, 32, 48, 1, 1, 6, 2.5)
    s = rng.uniform(0.01, 0.99, (100, 48)).astype(np.float32)
    ids, _ = oracle.select_experts(s, spec)
    for t in range(100):
        ref = sorted(e for _, e in heapq.nlargest(6, ((float(v), e) for e in range(48) for v in [s[t, e]])))
        assert list(ids[t]) == ref


def test_all_groups_kept_is_plain_topk():
    """Gk = G keeps every group: again a plain top-K over all experts."""
    rng = np.random.default_rng(8)
    spec = oracle.LayerSpec(64, 32, 32, 8, 8, 8, 2.5)
    s = rng.uniform(0.01, 0.99, (50, 32)).astype(np.float32)
    ids, _ = oracle.select_experts(s, spec)
    for t in range(50):
        ref = sorted(int(e) for e in sorted(range(32), key=lambda e: -float(s[t, e]))[:8])
        assert list(ids[t]) == ref


def test_group_score_uses_top2_not_top1():
    """A group with one huge score but a weak second must lose to a group with two good scores."""
    spec = oracle.LayerSpec(8, 8, 8, 4, 1, 2, 2.5)   # 4 groups of 2, keep 1 group, top-2
    s = np.array([[0.95, 0.01, 0.60, 0.55, 0.1, 0.1, 0.2, 0.2]], np.float32)
    ids, kept = oracle.select_experts(s, spec)
    assert list(kept[0]) == [1] and list(ids[0]) == [2, 3]


def test_kept_groups_mask_outside_experts():
    """The best experts overall can be excluded when their group is dropped."""
    spec = oracle.LayerSpec(8, 8, 8, 4, 2, 2, 2.5)   # 4 groups of 2, keep 2, top-2
    s = np.array([[0.5, 0.5, 0.9, 0.05, 0.45, 0.45, 0.1, 0.1]], np.float32)
    ids, kept = oracle.select_experts(s, spec)
    # group sums: 1.0, 0.95, 0.9, 0.2 -> keep groups 0,1; expert 2 (0.9) and expert 0/1 (0.5)
    assert sorted(kept[0]) == [0, 1]
    assert list(ids[0]) == [0, 2]


def _check_invariants(spec, ids, w, kept):
    T, K = ids.shape
    assert K == spec.top_k
    assert (np.diff(ids, axis=1) > 0).all()                    # distinct, ascending
    assert ((ids >= 0) & (ids < spec.n_experts)).all()
    grp = ids // spec.group_size
    for t in range(T):
        assert set(grp[t]) <= set(kept[t])                     # inside the kept groups
    assert (w > 0).all()
    tot = w.astype(np.float64).sum(axis=1)
    assert np.all(np.abs(tot - spec.alpha) <= 4 * np.spacing(np.float32(spec.alpha)))


@pytest.mark.parametrize("name,T", [("tiny", None), ("decode", None), ("skew", 512),
                                    ("prefill", 512), ("fp8_decode", None)])
def test_routing_invariants(name, T):
    w = gen.workload(name, T)
    spec = oracle.LayerSpec.of(w)
    x, wr, b = gen.router_inputs(w, 0)
    s = oracle.router_scores(x, wr, b)
    ids, kept = oracle.select_experts(s, spec)
    wts = oracle.combine_weights(s, ids, spec.alpha)
    _check_invariants(spec, ids, wts, kept)


def test_weights_exact_normalisation():
    """w_k = 2.5 s_k / sum(s) up to two fp32 roundings (checked with exact sums)."""
    w, spec, x, wr, b = _tiny(1)
    s = oracle.router_scores(x, wr, b)
    ids, wts = oracle.route(spec, x, wr, b)
    for t in range(w.T):
        sel = [float(s[t, e]) for e in ids[t]]
        den = math.fsum(sel)
        for k in range(spec.top_k):
            exact = 2.5 * sel[k] / den
            assert abs(float(wts[t, k]) - exact) <= 3 * float(np.spacing(np.float32(exact)))


def test_gap_guard_redraws():
    w = gen.workload("tiny")
    spec = oracle.LayerSpec.of(w)
    x, wr, b = gen.router_inputs(w, 0)
    # a huge guard flags most rows; a 1e-6 guard after re-draws flags none
    assert len(oracle.gap_violations(spec, x, wr, b, guard=1.0)) == w.T
    x2, wr2, b2, n = gen.guarded_router_inputs(w, 0, lambda x, wr, b: oracle.gap_violations(spec, x, wr, b))
    assert len(oracle.gap_violations(spec, x2, wr2, b2)) == 0


def _hand_routing(logit_rows):
    """x row t = the unit vector e_t (bf16 1.0) and W_router row t = token t's logits, so each
    token's fp32 logits are exactly the given values (rounded once to fp32)."""
    T, E = len(logit_rows), len(logit_rows[0])
    H = 256
    x = np.zeros((T, H), np.uint16)
    x[np.arange(T), np.arange(T)] = 0x3F80            # bf16 1.0
    wr = np.zeros((H, E), np.float32)
    wr[:T] = np.asarray(logit_rows, np.float32)
    return x, wr


def test_gap_violations_boundary_positions():
    """Hand-built tiny routings (8 groups of 4, Gk = 4, K = 8), one boundary gap of about 4e-7 per
    token and every other gap wide.  Only a close pair AT a selection boundary (the 4th vs 5th group
    score; the 8th vs 9th candidate inside the kept groups) flags a token: the same close pair one
    position earlier or later, or among the experts of a dropped group, does not.  Each boundary
    index off by one, or candidates taken from every group, changes the flagged set."""
    spec = oracle.LayerSpec(256, 128, 32, 8, 4, 8, 2.5)
    eps = 2.5e-6                         # logit step near 1.4-2: a score step of about 4e-7
    low = -3.0
    rank_to_group = [5, 2, 7, 0, 3, 6, 1, 4]            # group of the r-th best group
    slot = [2, 0, 3, 1]                                 # expert position in the group of its r-th value

    def row(groups):
        """groups[r] = the 4 logits of the r-th ranked group, best first."""
        z = np.full(32, low, np.float64)
        for r, vals in enumerate(groups):
            g = rank_to_group[r]
            for j, v in enumerate(vals):
                z[4 * g + slot[j]] = v
        return z

    base = [[3.0, 2.9, low, low], [2.5, 2.4, low, low], [2.0, 1.9, low, low], [1.5, 1.4, low, low],
            [1.0, 0.9, low, low], [0.5, 0.4, low, low], [0.0, -0.1, low, low], [-0.5, -0.6, low, low]]

    def variant(changes):
        g = [list(v) for v in base]
        for (r, j), v in changes.items():
            g[r][j] = v
        return row(g)

    rows = [
        variant({(4, 0): 1.5, (4, 1): 1.4 - eps}),           # 0: 4th vs 5th group score: flagged
        variant({(3, 0): 2.0, (3, 1): 1.9 - eps}),           # 1: 3rd vs 4th group (and 7th vs 8th expert)
        variant({(5, 0): 1.0, (5, 1): 0.9 - eps}),           # 2: 5th vs 6th group
        variant({(0, 2): 1.4 - eps}),                        # 3: 8th vs 9th candidate: flagged
        variant({(3, 1): 1.5 - eps}),                        # 4: 7th vs 8th candidate
        variant({(0, 2): 0.5, (0, 3): 0.5 - eps}),           # 5: 9th vs 10th candidate
        variant({}),                                         # 6: every gap wide
        variant({(4, 0): 1.4 - eps}),                        # 7: a dropped group's expert next to the 8th
    ]
    x, wr = _hand_routing(rows)
    b = np.zeros(32, np.float32)
    # the fixture does what it says: the designed gaps are in (0, 1e-6), the rest far wider
    s = oracle.router_scores(x, wr, b).astype(np.float64)
    gs = np.sort(oracle.moe._group_scores(s.astype(np.float32), spec).astype(np.float64), axis=1)[:, ::-1]
    assert 0 < gs[0, 3] - gs[0, 4] < 1e-6 and 0 < gs[1, 2] - gs[1, 3] < 1e-6 and 0 < gs[2, 4] - gs[2, 5] < 1e-6
    assert np.all(np.diff(-gs[6]) > 1e-3)
    ids, kept = oracle.select_experts(s.astype(np.float32), spec)
    assert [sorted(int(rank_to_group.index(g)) for g in kept[t]) for t in (3, 4, 5, 6, 7)] == [[0, 1, 2, 3]] * 5
    assert list(oracle.gap_violations(spec, x, wr, b)) == [0, 3]
    # a guard below the designed gaps flags nothing
    assert list(oracle.gap_violations(spec, x, wr, b, guard=1e-9)) == []


def test_group_size_one_is_rejected():
    spec = oracle.LayerSpec(256, 128, 8, 8, 4, 4, 2.5)
    s = np.full((2, 8), 0.5, np.float32)
    with pytest.raises(ValueError):
        oracle.select_experts(s, spec)
