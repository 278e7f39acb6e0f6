"""GPU parity of the norms and the residual mix around the MoE block (HIP path
through the C ABI vs oracle/block.py).

  * beam_moe_rms_norm is bit-exact: both sides do the same correctly rounded
    FP32 steps in the order the definition states;
  * beam_moe_block_forward: routing ids bit-exact (so the pre-norm the router
    saw is the oracle's), weights to 1e-5, the MoE output and the new stream to
    the output bar of tests/gpu_cases.py; and the fused post-norm + mix is
    bit-exact when the oracle is fed the GPU's own MoE output (a call output).
Inputs are drawn so that the oracle's routing has no near-ties after the pre-norm.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import codecs
from synth import gen
import tests.gpu_cases as C

pytestmark = pytest.mark.gpu

EPS = 1e-6


def guarded_block(w, seed=0):
    spec = oracle.LayerSpec.of(w)
    gpre, gpost = gen.norm_gains(w, seed)
    s, wr, b, _ = gen.guarded_router_inputs(
        w, seed, lambda xs, wr_, b_: oracle.gap_violations(spec, oracle.rms_norm_bits(xs, gpre, EPS), wr_, b_))
    return spec, s, wr, b, gpre, gpost


def run_block(w, s, wr, b, gpre, gpost, W, step, in_place=False):
    import sparse_moe_layer_top_amd as bm
    d = C.dev()
    T = s.shape[0]
    st, wrt, bt = C.router_tensors(s, wr, b)
    ids = torch.empty(T, w.top_k, dtype=torch.int32, device=d)
    wts = torch.empty(T, w.top_k, dtype=torch.float32, device=d)
    moe = torch.empty(T, w.hidden, dtype=torch.bfloat16, device=d)
    out = bm.beam_moe_block_forward(C.cfg_of(w), step, EPS, st, torch.from_numpy(gpre).to(d),
                                    torch.from_numpy(gpost).to(d), wrt, bt, W["gate"], W["up"], W["down"],
                                    W.get("s_gate"), W.get("s_up"), W.get("s_down"),
                                    stream_out=st if in_place else None, moe_out=moe, topk_ids_out=ids,
                                    topk_w_out=wts)
    torch.cuda.synchronize()
    return C.bits_of(out), C.bits_of(moe), ids.cpu().numpy(), wts.cpu().numpy()


@pytest.mark.parametrize("T,H,sigma", [(1, 256, 1.0), (7, 256, 1e-3), (64, 5120, 1.0), (1000, 5120, 0.02),
                                       (3, 8, 5.0), (5, 8192, 1.0)])
def test_rms_norm_bit_exact(T, H, sigma):
    import sparse_moe_layer_top_amd as bm
    C.say(f"[rms_norm] T={T} H={H} sigma={sigma}")
    rng = np.random.default_rng([T, H])
    x = codecs.bf16_round_bits((rng.standard_normal((T, H)) * sigma).astype(np.float32))
    g = (1.0 + 0.1 * rng.standard_normal(H)).astype(np.float32)
    got = bm.beam_moe_rms_norm(C.to_bf16(x), torch.from_numpy(g).to(C.dev()), EPS)
    torch.cuda.synchronize()
    assert np.array_equal(C.bits_of(got), oracle.rms_norm_bits(x, g, EPS))


def test_rms_norm_in_place_and_eps_dominated_rows():
    import sparse_moe_layer_top_amd as bm
    rng = np.random.default_rng(2)
    x = codecs.bf16_round_bits((rng.standard_normal((16, 512)) * 1e-4).astype(np.float32))
    x[3] = 0                                            # an all-zero row: r = 1/sqrt(eps)
    g = np.ones(512, np.float32)
    t = C.to_bf16(x)
    bm.beam_moe_rms_norm(t, torch.from_numpy(g).to(C.dev()), 1e-5, out=t)
    torch.cuda.synchronize()
    assert np.array_equal(C.bits_of(t), oracle.rms_norm_bits(x, g, 1e-5))


@pytest.mark.parametrize("seed,step", [(0, 3), (1, 2), (2, 105)])
def test_tiny_block(seed, step):
    w = gen.workload("tiny")
    C.say(f"[tiny block] seed={seed} step={step}")
    spec, s, wr, b, gpre, gpost = guarded_block(w, seed)
    W, src = C.host_expert_weights(w, seed)
    out, moe, ids, wts = run_block(w, s, wr, b, gpre, gpost, W, step)
    ref = oracle.block_forward(spec, s, gpre, gpost, EPS, step, wr, b, src.get)
    C.check_ids_w(ids, wts, ref["ids"], ref["w"])
    C.check_out(moe, ref["out"])
    C.check_out(out, ref["stream_out"])
    # the fused post-norm + mix, exactly, from the GPU's own MoE output
    exact = oracle.residual_mix_bits(s, oracle.rms_norm_bits(moe, gpost, EPS), step)
    assert np.array_equal(out, exact)


def test_tiny_block_in_place_and_ragged():
    w = gen.workload("tiny", T=130)
    spec, s, wr, b, gpre, gpost = guarded_block(w, 4)
    W, src = C.host_expert_weights(w, 4)
    out, moe, ids, wts = run_block(w, s, wr, b, gpre, gpost, W, 9, in_place=True)
    ref = oracle.block_forward(spec, s, gpre, gpost, EPS, 9, wr, b, src.get)
    C.check_ids_w(ids, wts, ref["ids"], ref["w"])
    assert np.array_equal(out, oracle.residual_mix_bits(s, oracle.rms_norm_bits(moe, gpost, EPS), 9))


def test_tiny_block_fp8():
    w = gen.Workload("tiny_fp8", 1, 96, 256, 128, 32, 8, 4, 8, 2.5, 0.05, 0.02, "zero", "fp8", 1)
    spec, s, wr, b, gpre, gpost = guarded_block(w, 0)
    W, src = C.host_expert_weights(w, 0)
    out, moe, ids, wts = run_block(w, s, wr, b, gpre, gpost, W, 4)
    ref = oracle.block_forward(spec, s, gpre, gpost, EPS, 4, wr, b, src.get)
    C.check_ids_w(ids, wts, ref["ids"], ref["w"])
    C.check_out(out, ref["stream_out"])


@pytest.mark.parametrize("name,n_sample", [("decode", 8), ("prefill", 4)])
def test_real_shape_block(name, n_sample):
    from tests.test_gpu_parity import real_weights
    w = gen.workload(name)
    C.say(f"[{name} block] T={w.T} inputs")
    spec, s, wr, b, gpre, gpost = guarded_block(w, 0)
    W = real_weights(w.weight)
    C.say(f"[{name} block] block forward on the GPU")
    out, moe, ids, wts = run_block(w, s, wr, b, gpre, gpost, W, 2 * 10 + 3)
    C.say(f"[{name} block] oracle pre-norm and routing over all {w.T} tokens")
    x = oracle.rms_norm_bits(s, gpre, EPS)
    rid, rw = oracle.route(spec, x, wr, b)
    C.check_ids_w(ids, wts, rid, rw)
    C.say(f"[{name} block] fused post-norm + mix, exact, over all tokens")
    assert np.array_equal(out, oracle.residual_mix_bits(s, oracle.rms_norm_bits(moe, gpost, EPS), 23))
    rng = np.random.default_rng(4321)
    sample = np.unique(np.concatenate([[0, w.T - 1], rng.choice(w.T, min(n_sample, w.T), replace=False)]))
    src = gen.ExpertSource(w, 0)
    src.prefetch(np.unique(rid[sample]))
    C.say(f"[{name} block] oracle block on {len(sample)} sampled tokens")
    ref = oracle.block_forward(spec, s[sample], gpre, gpost, EPS, 23, wr, b, src.get)
    C.check_out(moe[sample], ref["out"])
    mx, mn = C.check_out(out[sample], ref["stream_out"])
    C.say(f"[{name} block] stream max rel {mx:.2e} mean|d|/rms {mn:.2e}")
