"""The allocation-free forward (beam_moe_forward_noalloc, workspace in the library's fixed device
array) against the forward with a caller workspace (beam_moe_forward): the same kernels on the same
inputs, so ids, weights and outputs must match bit for bit, on two calls in a row, the second with
a smaller input (the array keeps the first call's contents).  Both are also held to the oracle's
output bar on the small layer."""
import numpy as np
import pytest
import torch

import oracle
from synth import gen
from tests import gpu_cases as C

pytestmark = pytest.mark.gpu


def _both(w, cfg, xt, wrt, bt, W):
    import sparse_moe_layer_top_amd as bm
    T = xt.shape[0]
    res = []
    for fn in ("forward", "noalloc"):
        out = torch.empty(T, w.hidden, dtype=torch.bfloat16, device=C.dev())
        ids = torch.empty(T, w.top_k, dtype=torch.int32, device=C.dev())
        wts = torch.empty(T, w.top_k, dtype=torch.float32, device=C.dev())
        if fn == "forward":
            bm.beam_moe_forward(cfg, xt, wrt, bt, W["gate"], W["up"], W["down"], W.get("s_gate"), W.get("s_up"),
                                W.get("s_down"), out=out, topk_ids_out=ids, topk_w_out=wts)
        else:
            bm.beam_moe_forward_noalloc(cfg, xt, wrt, bt, W["gate"], W["up"], W["down"], out, W.get("s_gate"),
                                        W.get("s_up"), W.get("s_down"), topk_ids_out=ids, topk_w_out=wts)
        torch.cuda.synchronize()
        res.append((C.bits_of(out), ids.cpu().numpy(), wts.cpu().numpy()))
    return res


def test_noalloc_matches_forward_tiny_two_calls():
    w0 = gen.workload("tiny")
    W, src = C.host_expert_weights(w0, 3)
    for T in (1000, 100):                       # the second call smaller than the first
        w = gen.workload("tiny", T)
        C.say(f"[noalloc tiny] T={T}")
        spec, x, wr, b = C.guarded(w, 3)
        (o1, i1, w1), (o2, i2, w2) = _both(w, C.cfg_of(w), *C.router_tensors(x, wr, b), W)
        assert np.array_equal(o1, o2) and np.array_equal(i1, i2) and np.array_equal(w1.view(np.uint32), w2.view(np.uint32))
        ref = oracle.forward(spec, x, wr, b, src.get)
        C.check_ids_w(i2, w2, ref["ids"], ref["w"])
        C.check_out(o2, ref["out"], what=f"noalloc tiny T={T}")


def test_noalloc_matches_forward_real_decode_two_calls():
    from tests.test_gpu_parity import real_weights
    W = real_weights("bf16")
    for T in (256, 64):                         # the second call smaller than the first
        w = gen.workload("decode", T)
        C.say(f"[noalloc decode] T={T}")
        x, wr, b = gen.router_inputs(w, 0)
        (o1, i1, w1), (o2, i2, w2) = _both(w, C.cfg_of(w), *C.router_tensors(x, wr, b), W)
        assert np.array_equal(o1, o2) and np.array_equal(i1, i2) and np.array_equal(w1.view(np.uint32), w2.view(np.uint32))


def test_noalloc_rejects_a_layer_past_the_array():
    import sparse_moe_layer_top_amd as bm
    from sparse_moe_layer_top_amd import binding as B
    w = gen.workload("decode", 512)
    cfg = C.cfg_of(w)
    assert bm.beam_moe_workspace_bytes(cfg, 512) > bm.NOALLOC_SCRATCH_BYTES
    x = torch.zeros(512, w.hidden, dtype=torch.bfloat16, device=C.dev())
    wr = torch.zeros(w.hidden, w.n_experts, device=C.dev())
    wt = torch.zeros(w.n_experts, 1, 1, dtype=torch.bfloat16, device=C.dev())   # never read: rejected first
    out = torch.empty_like(x)
    st = B.LIB.beam_moe_forward_noalloc(__import__("ctypes").byref(cfg.c()), 512, B._ptr(x), B._ptr(wr), None,
                                        B._ptr(wt), B._ptr(wt), B._ptr(wt), None, None, None, B._ptr(out), None,
                                        None, None)
    assert st == B.ERR_WORKSPACE
