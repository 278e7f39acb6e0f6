"""Pins for the oracle's MXFP4 codecs (oracle/codecs.py):

  * E2M1 decoding and the element rounding (nearest, ties to even mantissa,
    saturating at 6) against PyTorch's own E2M1 helpers
    (torch/testing/_internal/common_quantized.py; that module imports test-only
    packages that are not installed, so the three helpers are compiled from its
    source on their own);
  * the packing convention (lower-indexed value in the low nibble) against the
    same module's pack_uint4;
  * the shared-exponent rule floor(log2(max|v|)) - 2 against math.frexp;
    round trips of on-grid blocks, the error bound, saturation, zero blocks;
  * planted mistakes fail these pins.
"""
import ast
import math
import os

import numpy as np
import pytest
import torch

from oracle import codecs

_QPATH = os.path.join(os.path.dirname(torch.__file__), "testing", "_internal", "common_quantized.py")


def _torch_helpers():
    tree = ast.parse(open(_QPATH).read())

    def const_assign(n):
        return isinstance(n, ast.Assign) and all(
            (isinstance(t, ast.Name) and t.id.isupper())
            or (isinstance(t, ast.Tuple) and all(isinstance(e, ast.Name) and e.id.isupper() for e in t.elts))
            for t in n.targets)

    names = ("_n_ones", "_f32_to_floatx_unpacked", "_floatx_unpacked_to_f32", "pack_uint4", "down_size")
    body = [n for n in tree.body if (isinstance(n, ast.FunctionDef) and n.name in names) or const_assign(n)]
    ns = {"torch": torch, "Tensor": torch.Tensor}
    for n in body:                      # constants may need earlier functions: define in file order, skip failures
        try:
            exec(compile(ast.Module(body=[n], type_ignores=[]), _QPATH, "exec"), ns)
        except NameError:
            pass
    return ns


@pytest.fixture(scope="module")
def th():
    if not os.path.exists(_QPATH):
        pytest.skip("torch's quantisation test helpers are not available")
    return _torch_helpers()


def _bf16(a):
    return codecs.bf16_round_bits(np.asarray(a, np.float32))


def test_e2m1_decode_matches_torch(th):
    ref = th["_floatx_unpacked_to_f32"](torch.arange(16, dtype=torch.uint8), 2, 1).double().numpy()
    got = codecs.e2m1_decode(np.arange(16))
    assert np.array_equal(got, ref)
    assert np.array_equal(np.signbit(got), np.signbit(ref))


def test_element_rounding_matches_torch(th):
    rng = np.random.default_rng(0)
    grid = codecs.e2m1_decode(np.arange(8))
    mids = 0.5 * (grid[1:] + grid[:-1])
    u = np.concatenate([rng.uniform(0, 8, 20000), grid, mids, np.nextafter(mids, 0), np.nextafter(mids, 9), [7.99, 6.0001]])
    ref = th["_f32_to_floatx_unpacked"](torch.from_numpy(u.astype(np.float32)), 2, 1).numpy()
    got = codecs._e2m1_round(u.astype(np.float32).astype(np.float64))
    assert np.array_equal(got, ref)


def test_packing_matches_torch(th):
    rng = np.random.default_rng(1)
    v = _bf16(rng.standard_normal((3, 64)) * 0.1)
    packed, _ = codecs.mxfp4_quantize(v)
    codes = codecs.mxfp4_unpack(packed)
    ref = th["pack_uint4"](torch.from_numpy(codes)).numpy()
    assert np.array_equal(packed, ref)


def test_shared_exponent_rule():
    rng = np.random.default_rng(2)
    v = _bf16(rng.standard_normal((16, 32 * 8)) * np.exp2(rng.integers(-20, 10, (16, 1))))
    _, e = codecs.mxfp4_quantize(v)
    blocks = np.abs(codecs.bf16_to_f64(v)).reshape(16, 8, 32).max(axis=-1)
    for (r, b), amax in np.ndenumerate(blocks):
        ex = math.frexp(float(amax))[1] - 1          # floor(log2(amax)) for amax > 0
        assert e[r, b] == ex - 2 + 127


def test_on_grid_blocks_round_trip():
    rng = np.random.default_rng(3)
    rows, nb = 8, 6
    mags = rng.integers(0, 8, (rows, nb, 32))
    mags[:, :, 0] = rng.choice([6, 7], (rows, nb))            # the block maximum is 4 or 6: scale is exact
    signs = rng.integers(0, 2, (rows, nb, 32)) * 8
    codes = np.where(mags == 0, 0, mags | signs).astype(np.uint8).reshape(rows, nb * 32)   # no negative zero
    e = rng.integers(100, 140, (rows, nb)).astype(np.uint8)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    vals = codecs.mxfp4_dequant(packed, e)
    p2, e2 = codecs.mxfp4_quantize(_bf16(vals))
    assert np.array_equal(e2, e) and np.array_equal(p2, packed)


def test_error_bound_saturation_and_zero_blocks():
    rng = np.random.default_rng(4)
    v = rng.standard_normal((4, 32 * 16)) * 0.02
    v[0, :32] = 0.0                                            # an all-zero block
    v[1, :32] = 0.0
    v[1, 0] = 7.5                                              # amax 7.5: scale 1, saturates to 6
    bits = _bf16(v)
    packed, e = codecs.mxfp4_quantize(bits)
    assert e[0, 0] == 0 and np.all(codecs.mxfp4_unpack(packed)[0, :32] == 0)
    assert e[1, 0] == 127 and codecs.mxfp4_dequant(packed, e)[1, 0] == 6.0
    x = codecs.bf16_to_f64(bits)
    d = codecs.mxfp4_dequant(packed, e)
    X = np.repeat(codecs.e8m0_scale(e), 32, axis=-1)
    u = np.abs(x) / X
    spacing = np.where(u < 2, 0.5, np.where(u < 4, 1.0, 2.0))
    ok = np.abs(d - x) <= 0.5 * spacing * X * (1 + 1e-12)
    sat = u > 6
    assert np.all(ok | sat) and np.all(np.abs(d[sat]) == 6 * X[sat])


# ------------------------------------------------------------ planted mistakes

def _ties_away(u):
    grid = codecs.e2m1_decode(np.arange(8))
    code = np.zeros(u.shape, np.uint8)
    for c in range(1, 8):
        code = np.where(u >= 0.5 * (grid[c - 1] + grid[c]), c, code).astype(np.uint8)
    return code


def _wrong_max(u):
    """Saturates at 4 (code 6) instead of 6."""
    return np.minimum(codecs.__dict__["_orig__e2m1_round"](u), 6).astype(np.uint8)


def _swapped_nibbles(packed):
    p = np.asarray(packed, np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), np.uint8)
    out[..., 0::2] = p >> 4
    out[..., 1::2] = p & 15
    return out


MUTANTS = [
    ("_e2m1_round", _ties_away, [lambda th: test_element_rounding_matches_torch(th)]),
    ("_e2m1_round", _wrong_max, [lambda th: test_element_rounding_matches_torch(th),
                                     lambda th: test_error_bound_saturation_and_zero_blocks()]),
    ("mxfp4_unpack", _swapped_nibbles, [lambda th: test_packing_matches_torch(th),
                                        lambda th: test_on_grid_blocks_round_trip()]),
]


@pytest.mark.parametrize("name,mutant,pins", MUTANTS, ids=[f"{m[0]}:{m[1].__name__}" for m in MUTANTS])
def test_mxfp4_mutant_is_caught(monkeypatch, th, name, mutant, pins):
    monkeypatch.setitem(codecs.__dict__, "_orig_" + name, getattr(codecs, name))
    monkeypatch.setattr(codecs, name, mutant)
    for pin in pins:
        with pytest.raises(AssertionError):
            pin(th)


def test_shared_exponent_mutant_is_caught(monkeypatch):
    orig = codecs.mxfp4_quantize

    def off_by_one(v_bits):
        packed, e = orig(v_bits)
        return packed, np.where(e > 0, e + 1, e).astype(np.uint8)

    monkeypatch.setattr(codecs, "mxfp4_quantize", off_by_one)
    with pytest.raises(AssertionError):
        test_shared_exponent_rule()
