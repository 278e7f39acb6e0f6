"""GPU parity of the dense SwiGLU MLP (beam_dense_mlp_forward through the C ABI)
against oracle.moe.dense_mlp, to the output bar of tests/gpu_cases.py, on the
streaming path (small T, down GEMM split over the reduction), the LDS-tiled path
(T > 1024), fp8 weights and the real shape; plus the speculative-verify MoE
shape (8 sequences x 16 tokens) through the MoE forward."""
import numpy as np
import pytest
import torch

import oracle
from synth import gen
import tests.gpu_cases as C

pytestmark = pytest.mark.gpu


def dense_cfg(w):
    import sparse_moe_layer_top_amd as bm
    return bm.DenseConfig(w.hidden, w.inter, bm.W_FP8_E4M3 if w.weight == "fp8" else bm.W_BF16)


def dense_weights(w, seed=0):
    d = C.dev()
    m = {k: gen.expert_matrix(w, seed, k, 0) for k in ("gate", "up", "down")}
    if w.weight == "fp8":
        t = {k: torch.from_numpy(v[0]).to(d) for k, v in m.items()}
        t.update({"s_" + k: torch.from_numpy(v[1]).to(d) for k, v in m.items()})
    else:
        t = {k: C.to_bf16(v) for k, v in m.items()}
    return t, m


def run_dense(w, x_bits, W, deterministic_check=False):
    import sparse_moe_layer_top_amd as bm
    out = bm.beam_dense_mlp_forward(dense_cfg(w), C.to_bf16(x_bits), W["gate"], W["up"], W["down"],
                                    W.get("s_gate"), W.get("s_up"), W.get("s_down"))
    torch.cuda.synchronize()
    return C.bits_of(out)


@pytest.mark.parametrize("T", [1, 7, 64, 100, 1024, 1025, 1100, 2000])
def test_tiny_dense(T):
    w = gen.workload("dense_tiny", T)
    C.say(f"[dense tiny] T={T}")
    x, _, _ = gen.router_inputs(w, 0)
    W, m = dense_weights(w)
    got = run_dense(w, x, W)
    C.check_out(got, oracle.dense_mlp(x, m["gate"], m["up"], m["down"]))
    assert np.array_equal(got, run_dense(w, x, W))       # fixed reduction order


def test_tiny_dense_fp8():
    w = gen.Workload("dense_tiny_fp8", 7, 96, 256, 512, 1, 1, 1, 1, 1.0, 0.05, 0.02, "zero", "fp8", 7)
    x, _, _ = gen.router_inputs(w, 0)
    W, m = dense_weights(w)
    C.check_out(run_dense(w, x, W), oracle.dense_mlp(x, m["gate"], m["up"], m["down"], weight="fp8"))


@pytest.mark.parametrize("name,n_sample", [("dense_decode", 16), ("dense_prefill", 8)])
def test_real_shape_dense(name, n_sample):
    w = gen.workload(name)
    C.say(f"[{name}] T={w.T} H={w.hidden} I={w.inter}")
    x, _, _ = gen.router_inputs(w, 0)
    W, m = dense_weights(w)
    got = run_dense(w, x, W)
    rng = np.random.default_rng(77)
    sample = np.unique(np.concatenate([[0, w.T - 1], rng.choice(w.T, n_sample, replace=False)]))
    C.say(f"[{name}] oracle on {len(sample)} sampled rows")
    mx, mn = C.check_out(got[sample], oracle.dense_mlp(x[sample], m["gate"], m["up"], m["down"]))
    C.say(f"[{name}] max rel {mx:.2e} mean|d|/rms {mn:.2e}")


def test_spec_verify_shape():
    from tests.test_gpu_parity import real_source, real_weights
    w = gen.workload("spec_verify")
    C.say(f"[spec_verify] T={w.T}")
    spec, x, wr, b = C.guarded(w, 0)
    out, ids, wts = C.run_forward(w, *C.router_tensors(x, wr, b), real_weights("bf16"))
    rid, rw = oracle.route(spec, x, wr, b)
    C.check_ids_w(ids.cpu().numpy(), wts.cpu().numpy(), rid, rw)
    sample = np.arange(w.T)        # every token of the verify batch
    ref = C.oracle_forward_threads(spec, x[sample], wr, b, real_source("bf16").get)
    C.check_out(C.bits_of(out)[sample], ref["out"], what="spec_verify output")
