"""Pins for the oracle's norms and residual mix (oracle/block.py), against what
the pages and the mathematics fix, not against the oracle's own formula:

  * the sum of squares: the exact sum rounded once (cases where a float32 chain or a
    second rounding of the float64 sum give other values), independent of channel order;
  * RMSNorm against an exactly summed (math.fsum) float64 reference, within one
    bf16 ulp, at magnitudes where eps matters and at a width where H vs H-1 shows;
  * closed forms for constant rows; exact invariance under power-of-two scaling;
  * the mix weights' squares sum to one (Reflection Beam 1.0 overview, section
    "Residual stream"); the mixed stream keeps unit scale for unit-scale inputs;
    late steps keep the old stream almost unchanged;
  * planted mistakes in the oracle fail these pins.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import block, codecs


def _bf16(a):
    return codecs.bf16_round_bits(np.asarray(a, np.float32))


def _ulp_bf16(x):
    """Spacing of bf16 values at |x| (for x != 0)."""
    e = np.floor(np.log2(np.abs(x)))
    return np.exp2(e - 7)


def _exact_rms_norm(v_bits, gamma, eps):
    v = codecs.bf16_to_f64(v_bits)
    H = v.shape[-1]
    ss = np.array([math.fsum(row * row) for row in v.reshape(-1, H)]).reshape(v.shape[:-1])
    return v / np.sqrt(ss / H + eps)[..., None] * np.asarray(gamma, np.float64)


@pytest.mark.parametrize("sigma,eps,H", [(1.0, 1e-6, 64), (1e-3, 1e-6, 64), (1e-3, 1e-5, 256), (3.0, 1e-6, 5120)])
def test_rms_norm_within_one_ulp_of_exact(sigma, eps, H):
    rng = np.random.default_rng([7, H])
    v = _bf16(rng.standard_normal((8, H)) * sigma)
    g = codecs.bf16_to_f64(_bf16(1.0 + 0.25 * rng.standard_normal(H))).astype(np.float32)
    got = codecs.bf16_to_f64(oracle.rms_norm_bits(v, g, eps))
    ref = _exact_rms_norm(v, g, eps)
    nz = ref != 0
    assert np.all(np.abs(got[nz] - ref[nz]) <= _ulp_bf16(ref[nz]))
    assert np.all(got[~nz] == 0)


def _squares_row(vals, H=128):
    v = np.zeros((1, H), np.float32)
    v[0, :len(vals)] = vals
    assert np.array_equal(codecs.bf16_to_f64(_bf16(v)), v.astype(np.float64))   # bf16 values
    return v


def test_sum_squares_is_the_exact_sum_rounded_once():
    """The definition fixes no order of additions: the float32 sum of squares is the exact sum,
    rounded once.  Cases built so that the plausible shortcuts give other answers:
      * a square of 2^24 then 5040 unit squares: exact 2^24 + 5040 (a float32 value); a float32
        chain in channel order absorbs every +1 (ties to even) and gives 2^24;
      * exact 1 + 2^-24 + 2^-80, just above the float32 midpoint between 1 and 1 + 2^-23:
        rounds up; the float64 sum lands on the midpoint and a second rounding (ties to even)
        gives 1;
      * exact 1 + 3*2^-24 - 2^-80 (the 2^-80 deficit from three copies of each 4^-j,
        j = 13..40), just below the midpoint between 1 + 2^-23 and 1 + 2^-22: rounds down; a
        second rounding of the float64 sum gives 1 + 2^-22."""
    v = np.zeros((1, 5120), np.float32)
    v[0, 79] = 4096.0
    v[0, 80:] = 1.0
    assert block.sum_squares_f32(v)[0] == np.float32(2.0 ** 24 + 5040)
    seq = np.float32(0)
    for h in range(5120):
        seq = np.float32(seq + v[0, h] * v[0, h])
    assert seq == np.float32(2.0 ** 24)               # what a channel-order float32 chain gives

    up = _squares_row([1.0, 2.0 ** -12, 2.0 ** -40])
    assert block.sum_squares_f32(up)[0] == np.float32(1 + 2.0 ** -23)
    assert np.float32(math.fsum(np.float64(up[0]) ** 2)) == np.float32(1.0)      # double rounding

    down_vals = [1.0, 2.0 ** -12, 2.0 ** -12] + [2.0 ** -j for j in range(13, 41) for _ in range(3)]
    down = _squares_row(down_vals)
    assert block.sum_squares_f32(down)[0] == np.float32(1 + 2.0 ** -23)
    assert np.float32(math.fsum(np.float64(down[0]) ** 2)) == np.float32(1 + 2.0 ** -22)

    # an exact tie stays a tie: 1 + 2^-24 goes to the even neighbour, 1
    assert block.sum_squares_f32(_squares_row([1.0, 2.0 ** -12]))[0] == np.float32(1.0)


def test_sum_squares_does_not_depend_on_channel_order():
    rng = np.random.default_rng(17)
    v = codecs.bf16_to_f64(_bf16(rng.standard_normal((6, 5120)) * np.exp2(rng.integers(-20, 20, (6, 5120)))))
    v = v.astype(np.float32)
    ref = block.sum_squares_f32(v)
    for seed in range(3):
        perm = np.random.default_rng(seed).permutation(5120)
        assert np.array_equal(block.sum_squares_f32(v[:, perm]), ref)
    g = np.ones(5120, np.float32)
    perm = np.random.default_rng(5).permutation(5120)
    assert np.array_equal(oracle.rms_norm_bits(_bf16(v)[:, perm], g, 1e-6), oracle.rms_norm_bits(_bf16(v), g, 1e-6)[:, perm])


def test_rms_norm_constant_rows_closed_form():
    H = 256
    v = _bf16(np.full((2, H), 0.5))
    g = codecs.bf16_to_f64(_bf16(np.linspace(-2, 2, H))).astype(np.float32)
    # mean(v^2) = 1/4: eps = 0 gives r = 2 exactly, so out = gamma
    assert np.array_equal(oracle.rms_norm_bits(v, g, 0.0), np.broadcast_to(_bf16(g), (2, H)))
    # eps = 3/4 gives r = 1, so out = v * gamma = gamma / 2
    assert np.array_equal(oracle.rms_norm_bits(v, g, 0.75), np.broadcast_to(_bf16(g / 2), (2, H)))


def test_rms_norm_power_of_two_scale_invariance():
    rng = np.random.default_rng(3)
    v = _bf16(rng.standard_normal((4, 512)))
    w = _bf16(codecs.bf16_to_f64(v) * 32.0)        # exact: power-of-two scaling of bf16 values
    g = np.ones(512, np.float32)
    assert np.array_equal(oracle.rms_norm_bits(v, g, 0.0), oracle.rms_norm_bits(w, g, 0.0))
    # and the gain scales the output exactly
    g4 = np.full(512, 4.0, np.float32)
    assert np.array_equal(codecs.bf16_to_f64(oracle.rms_norm_bits(v, g4, 1e-6)),
                          4.0 * codecs.bf16_to_f64(oracle.rms_norm_bits(v, g, 1e-6)))


def test_rms_norm_output_has_unit_rms():
    rng = np.random.default_rng(11)
    v = _bf16(rng.standard_normal((16, 5120)) * 0.37)
    out = codecs.bf16_to_f64(oracle.rms_norm_bits(v, np.ones(5120, np.float32), 1e-6))
    assert np.allclose(np.sqrt((out ** 2).mean(axis=1)), 1.0, atol=2e-3)


def test_mix_weights_squares_sum_to_one():
    for k in range(2, 106):
        a, b = oracle.mix_weights(k)
        assert abs(float(a) ** 2 + float(b) ** 2 - 1.0) <= 3 * 2.0 ** -24
        assert 0 < b <= a or k == 2
    a2, b2 = oracle.mix_weights(2)
    assert a2 == b2
    with pytest.raises(ValueError):
        oracle.mix_weights(1)


def test_mix_keeps_unit_scale_and_weights_the_new_output_less_with_depth():
    rng = np.random.default_rng(5)
    H = 5120
    s = _bf16(rng.standard_normal((8, H)))
    p = _bf16(rng.standard_normal((8, H)))
    sv, pv = codecs.bf16_to_f64(s), codecs.bf16_to_f64(p)
    for k in (2, 3, 10, 105):
        new = codecs.bf16_to_f64(oracle.residual_mix_bits(s, p, k))
        rms = np.sqrt((new ** 2).mean(axis=1)) / np.sqrt((sv ** 2).mean(axis=1))
        assert np.allclose(rms, 1.0, atol=0.03)
        # least squares: new = a_hat * s + b_hat * p, with a_hat^2 + b_hat^2 = 1 and b_hat = 1/sqrt(k)
        A = np.stack([sv.ravel(), pv.ravel()], axis=1)
        coef = np.linalg.lstsq(A, new.ravel(), rcond=None)[0]
        assert abs(coef[1] - 1 / math.sqrt(k)) < 2e-3 and abs(coef[0] - math.sqrt((k - 1) / k)) < 2e-3


def test_mix_of_equal_inputs_is_sum_of_weights():
    rng = np.random.default_rng(9)
    s = _bf16(rng.standard_normal((4, 256)))
    new = codecs.bf16_to_f64(oracle.residual_mix_bits(s, s, 2))
    ref = math.sqrt(2.0) * codecs.bf16_to_f64(s)
    nz = ref != 0
    assert np.all(np.abs(new[nz] - ref[nz]) <= _ulp_bf16(ref[nz]))


def test_block_special_cases():
    spec = oracle.LayerSpec(256, 128, 32, 8, 4, 8, 2.5)
    from synth import gen
    w = gen.workload("tiny")
    x_bits, wr, b = gen.router_inputs(w, 0)
    weights = lambda which, e: gen.expert_matrix(w, 0, which, e)
    rng = np.random.default_rng(1)
    g = (1.0 + 0.1 * rng.standard_normal(256)).astype(np.float32)
    # zero post-norm gain: the block adds nothing, the stream is only rescaled by a
    res = oracle.block_forward(spec, x_bits, g, np.zeros(256, np.float32), 1e-6, 7, wr, b, weights)
    a, _ = oracle.mix_weights(7)
    assert np.array_equal(res["stream_out"], _bf16(a * codecs.bf16_to_f64(x_bits).astype(np.float32)))
    # the MoE part sees the pre-norm output
    assert np.array_equal(res["x"], oracle.rms_norm_bits(x_bits, g, 1e-6))
    assert np.array_equal(res["out"], oracle.forward(spec, res["x"], wr, b, weights)["out"])


# ------------------------------------------------------------ planted mistakes

def _eps_outside_sqrt(v_bits, gamma, eps):
    v = codecs.bf16_to_f64(v_bits).astype(np.float32)
    r = np.float32(1.0) / (np.sqrt((v * v).mean(axis=-1, dtype=np.float32)) + np.float32(eps))
    return codecs.bf16_round_bits(v * r[..., None] * np.asarray(gamma, np.float32))


def _mean_over_h_minus_1(v_bits, gamma, eps):
    v = codecs.bf16_to_f64(v_bits).astype(np.float32)
    H = v.shape[-1]
    r = np.float32(1.0) / np.sqrt((v * v).sum(axis=-1, dtype=np.float32) / np.float32(H - 1) + np.float32(eps))
    return codecs.bf16_round_bits(v * r[..., None] * np.asarray(gamma, np.float32))


def _no_gain(v_bits, gamma, eps):
    return block.__dict__["_orig_rms_norm_bits"](v_bits, np.ones_like(np.asarray(gamma, np.float32)), eps)


def _swapped_mix_weights(step):
    a, b = block.__dict__["_orig_mix_weights"](step)
    return b, a


def _sum_squares_channel_chain(v):
    v = np.asarray(v, np.float32)
    acc = np.zeros(v.shape[0], np.float32)
    for h in range(v.shape[1]):
        acc = acc + v[:, h] * v[:, h]
    return acc


def _sum_squares_rounded_twice(v):
    v = np.asarray(v, np.float32)
    return np.array([np.float32(math.fsum(np.float64(r) ** 2)) for r in v], np.float32)


BLOCK_MUTANTS = [
    ("rms_norm_bits", _eps_outside_sqrt, [lambda: test_rms_norm_within_one_ulp_of_exact(1e-3, 1e-6, 64)]),
    ("rms_norm_bits", _mean_over_h_minus_1, [lambda: test_rms_norm_within_one_ulp_of_exact(1.0, 1e-6, 64)]),
    ("rms_norm_bits", _no_gain, [test_rms_norm_constant_rows_closed_form]),
    ("mix_weights", _swapped_mix_weights, [test_mix_keeps_unit_scale_and_weights_the_new_output_less_with_depth]),
    ("sum_squares_f32", _sum_squares_channel_chain, [test_sum_squares_is_the_exact_sum_rounded_once]),
    ("sum_squares_f32", _sum_squares_rounded_twice, [test_sum_squares_is_the_exact_sum_rounded_once]),
]


@pytest.mark.parametrize("name,mutant,pins", BLOCK_MUTANTS, ids=[f"{m[0]}:{m[1].__name__}" for m in BLOCK_MUTANTS])
def test_block_mutant_is_caught(monkeypatch, name, mutant, pins):
    monkeypatch.setitem(block.__dict__, "_orig_" + name, getattr(block, name))
    monkeypatch.setattr(block, name, mutant)
    if hasattr(oracle, name):
        monkeypatch.setattr(oracle, name, mutant)
    for pin in pins:
        with pytest.raises(AssertionError):
            pin()
