"""Pins for the oracle's number formats against torch's CPU casts (a library routine)."""
import numpy as np
import pytest
import torch

from oracle import codecs


def _torch_bf16_bits(a):
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_bf16_edge_cases():
    f = np.float32
    edge = np.array([0.0, -0.0, 1.0, -1.0, np.inf, -np.inf,
                     np.finfo(f).max, -np.finfo(f).max, np.finfo(f).tiny, np.finfo(f).tiny / 4,
                     1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20,   # ties and near-ties
                     3.3895314e38, 1e-40, -1e-45], f)
    assert np.array_equal(codecs.bf16_round_bits(edge), _torch_bf16_bits(edge))
    nan = codecs.bf16_round_bits(np.array([np.nan], f))
    assert (nan[0] & 0x7F80) == 0x7F80 and (nan[0] & 0x7F) != 0


def test_bf16_random_vs_torch():
    rng = np.random.default_rng(123)
    a = (rng.standard_normal(2_000_000) * np.exp(rng.uniform(-60, 60, 2_000_000))).astype(np.float32)
    # every tie pattern: low 16 bits exactly 0x8000
    t = (rng.integers(0, 2 ** 32, 100_000, dtype=np.uint64).astype(np.uint32) & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    t = t.view(np.float32)
    t = t[np.isfinite(t)]
    for arr in (a, t):
        assert np.array_equal(codecs.bf16_round_bits(arr), _torch_bf16_bits(arr))


def test_bf16_decode_exact():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = codecs.bf16_to_f64(bits)
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.isnan(got), np.isnan(ref))


def test_e4m3_all_codes_vs_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = codecs.e4m3_decode(codes)
    fin = ~np.isnan(ref)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(got[fin], ref[fin])
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9
    assert np.isnan(got[0x7F]) and np.isnan(got[0xFF])
