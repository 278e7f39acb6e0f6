"""beam_moe_forward (bf16 and MXFP4 weights), beam_moe_block_forward and beam_dense_mlp_forward
captured into a HIP graph (torch.cuda.graph on a side stream) and replayed:
the forward enqueues kernels only (no host sync, no allocation, no memset), so a captured call
must give the same bytes as a direct call on every replay, read its input buffers as they are at
replay time, and meet the oracle's bar.  Replays are separated by the program's own eager work
(a direct call on other inputs, a fill of the output) and synchronisations."""
import numpy as np
import pytest
import torch

import oracle
from synth import gen
from tests import gpu_cases as C

pytestmark = pytest.mark.gpu


def _capture_and_replay(w, W, seeds, src=None, layout=0):
    import sparse_moe_layer_top_amd as bm
    cfg = C.cfg_of(w, layout)
    d = C.dev()
    inputs = [C.guarded(w, s) for s in seeds]
    xt = C.to_bf16(inputs[0][1])
    wrt = torch.from_numpy(inputs[0][2]).to(d)
    bt = torch.from_numpy(inputs[0][3]).to(d)
    out = torch.empty(w.T, w.hidden, dtype=torch.bfloat16, device=d)
    ids = torch.empty(w.T, w.top_k, dtype=torch.int32, device=d)
    wts = torch.empty(w.T, w.top_k, dtype=torch.float32, device=d)
    ws = torch.empty(bm.beam_moe_workspace_bytes(cfg, w.T), dtype=torch.uint8, device=d)

    def call():
        bm.beam_moe_forward(cfg, xt, wrt, bt, W["gate"], W["up"], W["down"], W.get("s_gate"), W.get("s_up"),
                            W.get("s_down"), out=out, topk_ids_out=ids, topk_w_out=wts, workspace=ws)

    # direct results for every input set, with separate buffers
    direct = []
    for spec, x, wr, b in inputs:
        o, i, ww = C.run_forward(w, *C.router_tensors(x, wr, b), W, layout)
        direct.append((C.bits_of(o), i.cpu().numpy(), ww.cpu().numpy()))

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()                                   # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        call()
    torch.cuda.synchronize()

    for rep in range(4):
        k = rep % len(inputs)
        _, x, wr, b = inputs[k]
        xt.copy_(C.to_bf16(x))                   # new inputs into the captured buffers (eager)
        wrt.copy_(torch.from_numpy(wr))
        bt.copy_(torch.from_numpy(b))
        out.fill_(float("nan"))
        ids.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        C.say(f"[graph {w.name}] replay {rep}: input set {k}")
        o, i, ww = direct[k]
        assert np.array_equal(C.bits_of(out), o), f"replay {rep}: output bytes differ from the direct call"
        assert np.array_equal(ids.cpu().numpy(), i)
        assert np.array_equal(wts.cpu().numpy().view(np.uint32), ww.view(np.uint32))
        # eager work between replays: a direct call on the other input set
        C.run_forward(w, *C.router_tensors(*inputs[(k + 1) % len(inputs)][1:]), W, layout)
    return inputs, direct


def test_graph_tiny():
    w = gen.workload("tiny", 300)
    W, src = C.host_expert_weights(w, 2)
    inputs, direct = _capture_and_replay(w, W, seeds=[2, 3])
    for (spec, x, wr, b), (o, i, ww) in zip(inputs, direct):
        ref = oracle.forward(spec, x, wr, b, src.get)
        C.check_ids_w(i, ww, ref["ids"], ref["w"])
        C.check_out(o, ref["out"], what="graph tiny output")


def test_graph_decode():
    from tests.test_gpu_parity import real_weights
    w = gen.workload("decode")
    _capture_and_replay(w, real_weights("bf16"), seeds=[0, 1])


def test_graph_tiny_mxfp4():
    w = gen.workload("tiny_mx", 300)
    W, src = C.host_expert_weights(w, 4)
    inputs, direct = _capture_and_replay(w, W, seeds=[4, 5])
    for (spec, x, wr, b), (o, i, ww) in zip(inputs, direct):
        ref = oracle.forward(spec, x, wr, b, src.get)
        C.check_ids_w(i, ww, ref["ids"], ref["w"])
        C.check_out(o, ref["out"], what="graph tiny MXFP4 output")


def _replay_against_direct(run, set_inputs, outs, n_inputs, label):
    """Capture run() on a side stream, then replay it over the input sets set_inputs(k) installs into
    the captured buffers; every replay's output bytes equal a direct call's on the same inputs."""
    direct = []
    for k in range(n_inputs):
        set_inputs(k)
        run()
        torch.cuda.synchronize()
        direct.append([C.bits_of(t).copy() for t in outs])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        run()
    torch.cuda.synchronize()
    for rep in range(4):
        k = rep % n_inputs
        set_inputs(k)
        for t in outs:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        C.say(f"[graph {label}] replay {rep}: input set {k}")
        for t, ref in zip(outs, direct[k]):
            assert np.array_equal(C.bits_of(t), ref), f"replay {rep}: bytes differ from the direct call"
        set_inputs((k + 1) % n_inputs)
        run()                                         # eager work between replays
        torch.cuda.synchronize()


def test_graph_tiny_block():
    import sparse_moe_layer_top_amd as bm
    from tests.test_gpu_block import EPS, guarded_block
    w = gen.workload("tiny", 200)
    W, _ = C.host_expert_weights(w, 1)
    sets = [guarded_block(w, s) for s in (1, 2)]
    d = C.dev()
    cfg = C.cfg_of(w)
    st = C.to_bf16(sets[0][1])
    wrt = torch.from_numpy(sets[0][2]).to(d)
    bt = torch.from_numpy(sets[0][3]).to(d)
    gpre = torch.from_numpy(sets[0][4]).to(d)
    gpost = torch.from_numpy(sets[0][5]).to(d)
    out = torch.empty_like(st)
    moe = torch.empty_like(st)
    ws = torch.empty(bm.beam_moe_workspace_bytes(cfg, w.T, bm.OP_BLOCK), dtype=torch.uint8, device=d)

    def set_inputs(k):
        _, s, wr, b, gp, gq = sets[k]
        st.copy_(C.to_bf16(s)); wrt.copy_(torch.from_numpy(wr)); bt.copy_(torch.from_numpy(b))
        gpre.copy_(torch.from_numpy(gp)); gpost.copy_(torch.from_numpy(gq))

    def run():
        bm.beam_moe_block_forward(cfg, 9, EPS, st, gpre, gpost, wrt, bt, W["gate"], W["up"], W["down"],
                                  stream_out=out, moe_out=moe, workspace=ws)

    _replay_against_direct(run, set_inputs, [out, moe], 2, "tiny block")


@pytest.mark.parametrize("T", [64, 1100])
def test_graph_tiny_dense(T):
    """The dense MLP: at 64 tokens its GEMMs are split over the reduction (fp32 partial sums in the
    workspace, added in a fixed order), at 1100 tokens the one-workgroup-per-CU and LDS-tiled GEMMs."""
    import sparse_moe_layer_top_amd as bm
    from tests.test_gpu_dense import dense_cfg, dense_weights
    w = gen.workload("dense_tiny", T)
    W, _ = dense_weights(w)
    xs = [gen.router_inputs(w, s)[0] for s in (3, 4)]
    d = C.dev()
    cfg = dense_cfg(w)
    x = C.to_bf16(xs[0])
    out = torch.empty_like(x)
    ws = torch.empty(max(1, bm.beam_dense_workspace_bytes(cfg, T)), dtype=torch.uint8, device=d)

    def set_inputs(k):
        x.copy_(C.to_bf16(xs[k]))

    def run():
        bm.beam_dense_mlp_forward(cfg, x, W["gate"], W["up"], W["down"], out=out, workspace=ws)

    _replay_against_direct(run, set_inputs, [out], 2, f"tiny dense T={T}")


@pytest.mark.parametrize("name,T,H,I,weight", [("tiny", 64, 256, 128, "bf16"), ("wide272", 1500, 256, 256, "bf16"),
                                               ("moderate_mx", 230, 512, 512, "mxfp4")])
def test_graph_fragment_order(name, T, H, I, weight):
    """Weights (and MXFP4 scales) in fragment order, on the streaming, 272-row and 96-row MXFP4 schedules:
    every replay gives the direct call's bytes, and those are the row-order forward's bytes."""
    w = gen.Workload("graph_frag_" + name, 1, T, H, I, 32, 8, 4, 8, 2.5, 0.05, 0.02, "zero", weight, 1)
    W, _ = C.host_expert_weights(w, 4)
    P = C.packed(W)
    inputs, direct = _capture_and_replay(w, P, seeds=[4, 5], layout=1)
    for (spec, x, wr, b), (o, i, ww) in zip(inputs, direct):
        o_rows, _, _ = C.run_forward(w, *C.router_tensors(x, wr, b), W, 0)
        assert np.array_equal(C.bits_of(o_rows), o)
