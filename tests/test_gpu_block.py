"""GPU parity of the norms and the residual mix around the MoE block (HIP path
through the C ABI vs oracle/block.py).

  * beam_moe_rms_norm within one bf16 step of the oracle on every element, with
    the fraction of exact matches reported.  The oracle's sum of squares is the
    exact sum rounded once to FP32; the kernel adds the squares in FP32 in its
    own fixed order (64 blocks), so the two FP32 sums may differ in their last
    bits, which can move a bf16 result that lies next to a rounding midpoint by
    one step; every later step is the same correctly rounded FP32 operation;
  * beam_moe_block_forward: the block's routing ids bit-exact against the
    oracle's routing of the GPU's own pre-norm output (itself within one step
    of the oracle's pre-norm), weights to 1e-5; the MoE output and the new
    stream to the output bar of tests/gpu_cases.py against the oracle's block;
    and the fused post-norm + mix against the oracle's mix of the oracle's
    post-norm of the GPU's own MoE output (a call output), within the bound a
    one-step post-norm difference allows.
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


def gpu_prenorm(s, gpre):
    import sparse_moe_layer_top_amd as bm
    out = bm.beam_moe_rms_norm(C.to_bf16(s), torch.from_numpy(gpre).to(C.dev()), EPS)
    torch.cuda.synchronize()
    return C.bits_of(out)


def check_block_routing(spec, s, wr, b, gpre, ids, wts):
    """The block's ids and weights against the oracle's routing of the GPU's own pre-norm output,
    which must itself be within one bf16 step of the oracle's pre-norm.  Tokens whose gaps on the
    GPU's pre-norm fall below the guard (none expected) are checked for validity instead."""
    xg = gpu_prenorm(s, gpre)
    C.check_within_ulp(xg, oracle.rms_norm_bits(s, gpre, EPS), what="pre-norm")
    rid, rw = oracle.route(spec, xg, wr, b)
    near = oracle.gap_violations(spec, xg, wr, b)
    keep = np.setdiff1d(np.arange(len(rid)), near)
    C.check_ids_w(ids[keep], wts[keep], rid[keep], rw[keep])
    if len(near):
        C.say(f"  {len(near)} near-tie tokens after the GPU's pre-norm: validity only")
        C.check_valid_selection(spec, oracle.router_scores(xg[near], wr, b), ids[near], wts[near])
    return rid


def check_mix(out, s, moe, gpost, step):
    """The fused post-norm + mix against the oracle's mix of the oracle's post-norm of the GPU's own
    MoE output.  The GPU's post-norm is within one bf16 step of that post-norm (at most twice its
    spacing), so an element of new = bf16(a*stream + b*post) may move by b times that plus the
    output's own rounding step."""
    post = oracle.rms_norm_bits(moe, gpost, EPS)
    ref = oracle.residual_mix_bits(s, post, step)
    _, bw = oracle.mix_weights(step)
    g, r, p = (codecs.bf16_to_f64(v) for v in (out, ref, post))
    bound = float(bw) * 2 * C.bf16_spacing(p) + C.bf16_spacing(np.maximum(np.abs(g), np.abs(r)))
    d = np.abs(g - r)
    assert np.all(d <= bound), f"mix: {int((d > bound).sum())} elements past the one-step bound"
    frac = float((d == 0).mean())
    C.say(f"  post-norm + mix: within the bound everywhere, exact on {100 * frac:.4f}% of {d.size}")
    return frac


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
                                       (3, 8, 5.0), (5, 8192, 1.0), (4096, 5120, 1.0)])
def test_rms_norm_within_one_step(T, H, sigma):
    import sparse_moe_layer_top_amd as bm
    C.say(f"[rms_norm] T={T} H={H} sigma={sigma}")
    rng = np.random.default_rng([T, H])
    x = codecs.bf16_round_bits((rng.standard_normal((T, H)) * sigma).astype(np.float32))
    g = (1.0 + 0.1 * rng.standard_normal(H)).astype(np.float32)
    got = bm.beam_moe_rms_norm(C.to_bf16(x), torch.from_numpy(g).to(C.dev()), EPS)
    torch.cuda.synchronize()
    frac = C.check_within_ulp(C.bits_of(got), oracle.rms_norm_bits(x, g, EPS), what="rms_norm")
    # FP32 sums that differ in their last bits move a bf16 result only next to a rounding midpoint
    assert frac >= 0.99


def test_rms_norm_in_place_and_eps_dominated_rows():
    import sparse_moe_layer_top_amd as bm
    rng = np.random.default_rng(2)
    x = codecs.bf16_round_bits((rng.standard_normal((16, 512)) * 1e-4).astype(np.float32))
    x[3] = 0                                            # an all-zero row: r = 1/sqrt(eps)
    g = np.ones(512, np.float32)
    t = C.to_bf16(x)
    bm.beam_moe_rms_norm(t, torch.from_numpy(g).to(C.dev()), 1e-5, out=t)
    torch.cuda.synchronize()
    got = C.bits_of(t)
    C.check_within_ulp(got, oracle.rms_norm_bits(x, g, 1e-5), what="rms_norm in place")
    # the all-zero row is exactly zero
    assert np.all(got[3] & 0x7FFF == 0)


@pytest.mark.parametrize("seed,step", [(0, 3), (1, 2), (2, 105)])
def test_tiny_block(seed, step):
    w = gen.workload("tiny")
    C.say(f"[tiny block] seed={seed} step={step}")
    spec, s, wr, b, gpre, gpost = guarded_block(w, seed)
    W, src = C.host_expert_weights(w, seed)
    out, moe, ids, wts = run_block(w, s, wr, b, gpre, gpost, W, step)
    ref = oracle.block_forward(spec, s, gpre, gpost, EPS, step, wr, b, src.get)
    check_block_routing(spec, s, wr, b, gpre, ids, wts)
    C.check_out(moe, ref["out"], what="MoE output")
    C.check_out(out, ref["stream_out"], what="new stream")
    check_mix(out, s, moe, gpost, step)


def test_tiny_block_in_place_and_ragged():
    w = gen.workload("tiny", T=130)
    spec, s, wr, b, gpre, gpost = guarded_block(w, 4)
    W, src = C.host_expert_weights(w, 4)
    out, moe, ids, wts = run_block(w, s, wr, b, gpre, gpost, W, 9, in_place=True)
    ref = oracle.block_forward(spec, s, gpre, gpost, EPS, 9, wr, b, src.get)
    check_block_routing(spec, s, wr, b, gpre, ids, wts)
    C.check_out(out, ref["stream_out"], what="new stream")
    check_mix(out, s, moe, gpost, 9)


def test_tiny_block_fp8():
    w = gen.Workload("tiny_fp8", 1, 96, 256, 128, 32, 8, 4, 8, 2.5, 0.05, 0.02, "zero", "fp8", 1)
    spec, s, wr, b, gpre, gpost = guarded_block(w, 0)
    W, src = C.host_expert_weights(w, 0)
    out, moe, ids, wts = run_block(w, s, wr, b, gpre, gpost, W, 4)
    ref = oracle.block_forward(spec, s, gpre, gpost, EPS, 4, wr, b, src.get)
    check_block_routing(spec, s, wr, b, gpre, ids, wts)
    C.check_out(out, ref["stream_out"], what="new stream")
    check_mix(out, s, moe, gpost, 4)


@pytest.mark.parametrize("T", [64, 1100])
def test_tiny_block_mxfp4(T):
    """The whole sublayer with MXFP4 experts (streaming GEMMs at 64 tokens, the one-workgroup-per-CU
    GEMMs at 1100 tokens: about 34 rows per expert)."""
    w = gen.workload("tiny_mx", T)
    C.say(f"[tiny_mx block] T={T}")
    spec, s, wr, b, gpre, gpost = guarded_block(w, 6)
    W, src = C.host_expert_weights(w, 6)
    out, moe, ids, wts = run_block(w, s, wr, b, gpre, gpost, W, 7)
    ref = oracle.block_forward(spec, s, gpre, gpost, EPS, 7, wr, b, src.get)
    check_block_routing(spec, s, wr, b, gpre, ids, wts)
    C.check_out(moe, ref["out"], what="MoE output")
    C.check_out(out, ref["stream_out"], what="new stream")
    check_mix(out, s, moe, gpost, 7)


@pytest.mark.parametrize("name,n_sample", [("decode", 8), ("prefill", 16)])
def test_real_shape_block(name, n_sample):
    from tests.test_gpu_parity import real_source, real_weights
    w = gen.workload(name)
    C.say(f"[{name} block] T={w.T} inputs")
    spec, s, wr, b, gpre, gpost = guarded_block(w, 0)
    W = real_weights(w.weight)
    C.say(f"[{name} block] block forward on the GPU")
    out, moe, ids, wts = run_block(w, s, wr, b, gpre, gpost, W, 2 * 10 + 3)
    C.say(f"[{name} block] routing of the pre-norm over all {w.T} tokens")
    check_block_routing(spec, s, wr, b, gpre, ids, wts)
    C.say(f"[{name} block] fused post-norm + mix over all tokens")
    check_mix(out, s, moe, gpost, 23)
    rng = np.random.default_rng(4321)
    sample = np.unique(np.concatenate([[0, w.T - 1], rng.choice(w.T, min(n_sample, w.T), replace=False)]))
    C.say(f"[{name} block] oracle block on {len(sample)} sampled tokens")
    x = oracle.rms_norm_bits(s[sample], gpre, EPS)
    ref = C.oracle_forward_threads(spec, x, wr, b, real_source(w.weight).get)
    post = oracle.rms_norm_bits(ref["out"], gpost, EPS)
    new = oracle.residual_mix_bits(s[sample], post, 23)
    C.check_out(moe[sample], ref["out"], what=f"{name} block MoE output")
    C.check_out(out[sample], new, what=f"{name} block new stream")
