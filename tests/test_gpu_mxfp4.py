"""GPU parity of the MXFP4 weight path (E2M1 codes, one E8M0 scale per 32 inputs)
through the C ABI against the oracle:

  * beam_mxfp4_quantize bit-exact against oracle.codecs.mxfp4_quantize on random
    rows spanning many exponents, and on constructed blocks: values exactly on
    the rounding midpoints (ties to even), saturation, zero blocks, small
    negatives that become -0, bf16 subnormals and the clamped shared exponent;
  * the MoE forward and the dense MLP with MXFP4 weights, to the output bar of
    tests/gpu_cases.py, at ragged token counts and through the split reduction;
  * weights quantised on the GPU then used by the forward, against the oracle
    on the oracle's own quantisation of the same bf16 weights.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import codecs
from synth import gen
from tests import gpu_cases as C

pytestmark = pytest.mark.gpu


def _quantize_gpu(bits):
    import sparse_moe_layer_top_amd as bm
    codes, scales = bm.beam_mxfp4_quantize(C.to_bf16(bits))
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scales.cpu().numpy()


def _check_quantize(bits):
    bits = np.ascontiguousarray(bits, np.uint16)
    got_p, got_e = _quantize_gpu(bits)
    ref_p, ref_e = codecs.mxfp4_quantize(bits.reshape(-1, bits.shape[-1]))
    assert np.array_equal(got_e.reshape(ref_e.shape), ref_e), "E8M0 scales differ"
    bad = np.nonzero(got_p.reshape(ref_p.shape) != ref_p)
    assert len(bad[0]) == 0, f"{len(bad[0])} code bytes differ, first at {bad[0][:3]}, {bad[1][:3]}"


@pytest.mark.parametrize("shape", [(1, 32), (7, 64), (37, 1024), (3, 5, 256)])
def test_quantize_random_rows(shape):
    C.say(f"[mxfp4 quantize] random {shape}")
    rng = np.random.default_rng(sum(shape))
    v = rng.standard_normal(shape)
    # every 32-block gets its own magnitude, 2^-40 .. 2^40
    nb = shape[-1] // 32
    mag = np.exp2(rng.integers(-40, 41, shape[:-1] + (nb, 1)).astype(np.float64))
    v = (v.reshape(shape[:-1] + (nb, 32)) * mag).reshape(shape)
    _check_quantize(codecs.bf16_round_bits(v.astype(np.float32)))


def _special_blocks():
    grid = codecs.e2m1_decode(np.arange(8))
    mids = 0.5 * (grid[1:] + grid[:-1])                    # 0.25 .. 5: every one a bf16 value
    blocks = []
    for k in (-20, -1, 0, 3, 60):
        b = np.zeros(32)
        b[0] = 4.0                                          # amax 4 * 2^k: shared exponent k
        b[1:8] = mids
        b[8:15] = -mids
        b[15:23] = grid
        b[23] = 7.5                                         # past 6: saturates (amax still in [4, 8))
        b[24] = -7.0
        b[25:29] = [0.125, -0.125, 0.1875, -0.1875]         # below a quarter: 0 and -0
        b[29:32] = [0.251953125, 1.2421875, 4.96875]        # one bf16 step off a midpoint
        blocks.append(b * 2.0 ** k)
    blocks.append(np.zeros(32))                             # all-zero block: scale byte 0
    z = np.zeros(32)
    z[5] = -3e-39                                           # a bf16 subnormal block: shared exponent clamped
    z[6] = 2e-39
    blocks.append(z)
    rng = np.random.default_rng(7)
    blocks.append(rng.standard_normal(32) * 2.0 ** 125)     # near the top of the bf16 range
    return np.concatenate(blocks)[None, :]


def test_quantize_constructed_blocks():
    v = _special_blocks()
    bits = codecs.bf16_round_bits(v.astype(np.float32))
    # the construction is exact in bf16 (bar the random and subnormal blocks)
    assert np.array_equal(codecs.bf16_to_f64(bits)[0, :32 * 6], v[0, :32 * 6])
    # subnormal bf16 inputs
    raw = np.arange(1, 129, dtype=np.uint16)
    raw[64:] |= 0x8000
    _check_quantize(bits)
    _check_quantize(raw[None, :])


def test_quantize_zero_rows_is_a_noop():
    import sparse_moe_layer_top_amd as bm
    x = torch.empty(0, 64, dtype=torch.bfloat16, device=C.dev())
    codes, scales = bm.beam_mxfp4_quantize(x)
    assert codes.shape == (0, 32) and scales.shape == (0, 2)


# ---------------------------------------------------------------- forward ---

@pytest.mark.parametrize("T,seed", [(1, 0), (64, 1), (100, 2), (1100, 3)])
def test_tiny_mx_forward(T, seed):
    w = gen.workload("tiny_mx", T)
    C.say(f"[tiny_mx] T={T} seed={seed}")
    spec, x, wr, b = C.guarded(w, seed)
    W, src = C.host_expert_weights(w, seed)
    out, ids, wts = C.run_forward(w, *C.router_tensors(x, wr, b), W)
    ref = oracle.forward(spec, x, wr, b, src.get)
    C.check_ids_w(ids.cpu().numpy(), wts.cpu().numpy(), ref["ids"], ref["w"])
    C.check_out(C.bits_of(out), ref["out"])
    again, _, _ = C.run_forward(w, *C.router_tensors(x, wr, b), W)
    assert np.array_equal(C.bits_of(out), C.bits_of(again))


def test_quantized_on_gpu_then_forward():
    """bf16 experts quantised by beam_mxfp4_quantize (bit-exact to the oracle's
    quantisation), then the MXFP4 forward against the oracle on those codes."""
    import sparse_moe_layer_top_amd as bm
    wmx = gen.workload("tiny_mx", 200)
    wbf = gen.Workload("tiny_mx_src", 11, 200, 256, 256, 32, 8, 4, 8, 2.5, 0.05, 0.02, "zero", "bf16", 13)
    spec, x, wr, b = C.guarded(wmx, 5)
    src = gen.ExpertSource(wbf, 5)
    W, mats = {}, {}
    for k in ("gate", "up", "down"):
        stack = np.stack([src.get(k, e) for e in range(wmx.n_experts)])
        codes, scales = bm.beam_mxfp4_quantize(C.to_bf16(stack))
        W[k], W["s_" + k] = codes, scales
        ref_p, ref_e = codecs.mxfp4_quantize(stack.reshape(-1, stack.shape[-1]))
        torch.cuda.synchronize()
        assert np.array_equal(codes.cpu().numpy().reshape(ref_p.shape), ref_p)
        assert np.array_equal(scales.cpu().numpy().reshape(ref_e.shape), ref_e)
        mats[k] = (ref_p.reshape(codes.shape), ref_e.reshape(scales.shape))
    out, ids, wts = C.run_forward(wmx, *C.router_tensors(x, wr, b), W)
    ref = oracle.forward(spec, x, wr, b, lambda which, e: (mats[which][0][e], mats[which][1][e]))
    C.check_ids_w(ids.cpu().numpy(), wts.cpu().numpy(), ref["ids"], ref["w"])
    C.check_out(C.bits_of(out), ref["out"])


@pytest.mark.parametrize("T", [1, 64, 300, 1100])
def test_tiny_dense_mx(T):
    """Dense MLP with MXFP4 weights; at small T the down GEMM is split over the reduction."""
    import sparse_moe_layer_top_amd as bm
    w = gen.workload("dense_tiny_mx", T)
    C.say(f"[dense_tiny_mx] T={T}")
    x, _, _ = gen.router_inputs(w, 0)
    m = {k: gen.expert_matrix(w, 0, k, 0) for k in ("gate", "up", "down")}
    d = C.dev()
    W = {k: torch.from_numpy(v[0]).to(d) for k, v in m.items()}
    W.update({"s_" + k: torch.from_numpy(v[1]).to(d) for k, v in m.items()})
    cfg = bm.DenseConfig(w.hidden, w.inter, bm.W_MXFP4)
    out = bm.beam_dense_mlp_forward(cfg, C.to_bf16(x), W["gate"], W["up"], W["down"], W["s_gate"], W["s_up"],
                                    W["s_down"])
    torch.cuda.synchronize()
    C.check_out(C.bits_of(out), oracle.dense_mlp(x, m["gate"], m["up"], m["down"], weight="mxfp4"))
