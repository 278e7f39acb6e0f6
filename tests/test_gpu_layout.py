"""Expert weights in fragment order on the GPU: the pack entry point against the CPU reference of
the order (tests/fragment_order.py), and every schedule of the expert GEMMs giving byte-identical
results with the weights in row order and in fragment order.  Both orders feed each lane the same
16 bytes, so identical bytes out are the bar; the row-order path is held to the oracle by the
parity tests, on the same cases."""
import numpy as np
import pytest
import torch

from synth import gen
from tests import fragment_order as F
from tests import gpu_cases as C

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import sparse_moe_layer_top_amd  # noqa: F401  (fails loudly if the library is not built)
    assert torch.cuda.is_available()


@pytest.mark.parametrize("dtype,shape", [(np.uint16, (3, 48, 256)), (np.uint8, (2, 32, 192)),
                                         (np.uint8, (5, 16, 128)), (np.uint16, (16, 32))])
def test_pack_matches_reference(dtype, shape):
    import sparse_moe_layer_top_amd as bm
    rng = np.random.default_rng(3)
    w = rng.integers(0, np.iinfo(dtype).max, size=shape, dtype=dtype)
    t = C.to_bf16(w) if dtype == np.uint16 else torch.from_numpy(w).to(C.dev())
    got = bm.beam_moe_pack_weights(t)
    torch.cuda.synchronize()
    g = C.bits_of(got) if dtype == np.uint16 else got.cpu().numpy()
    assert np.array_equal(g, F.pack_by_reshape(w))


@pytest.mark.parametrize("shape", [(2, 32, 160), (3, 16, 16), (4, 48, 80)])
def test_pack_scales_matches_reference(shape):
    import sparse_moe_layer_top_amd as bm
    rng = np.random.default_rng(6)
    s = rng.integers(0, 256, size=shape, dtype=np.uint8)
    got = bm.beam_moe_pack_scales(torch.from_numpy(s).to(C.dev()))
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), F.pack_by_reshape(s, 16))


def test_pack_real_shape_stack():
    """Four experts of the real gate matrix shape [4, 2560, 5120] bf16: 100 MB."""
    import sparse_moe_layer_top_amd as bm
    rng = np.random.default_rng(4)
    w = rng.integers(0, 1 << 16, size=(4, 2560, 5120), dtype=np.uint16)
    got = bm.beam_moe_pack_weights(C.to_bf16(w))
    torch.cuda.synchronize()
    assert np.array_equal(C.bits_of(got), F.pack_by_reshape(w))


def _same_bytes(w, seed, W=None, what=""):
    spec, x, wr, b = C.guarded(w, seed)
    if W is None:
        W, _ = C.host_expert_weights(w, seed)
    t = C.router_tensors(x, wr, b)
    out_r, ids_r, w_r = C.run_forward(w, *t, W, layout=0)
    out_f, ids_f, w_f = C.run_forward(w, *t, C.packed(W), layout=1)
    assert torch.equal(ids_r, ids_f) and torch.equal(w_r, w_f)
    a, f = C.bits_of(out_r), C.bits_of(out_f)
    diff = int((a != f).sum())
    assert diff == 0, f"{what}: {diff} of {a.size} output values differ between the weight orders"


# every schedule: streaming (decode-sized, each weight type), the 96-row one-workgroup-per-CU GEMMs
# (bf16, fp8, MXFP4 over one and two rounds of the ring), the LDS-tiled GEMMs (bf16, fp8, the 320-column
# down), the 272-row gate/up, and the schedule boundaries
CASES = [
    ("tiny", 64, 256, 128, 32, 8, 4, 8, 2.5, "bf16"),
    ("tiny_ragged", 1000, 256, 128, 32, 8, 4, 8, 2.5, "bf16"),
    ("h128", 37, 128, 128, 16, 4, 2, 4, 1.0, "bf16"),
    ("stream_fp8", 40, 512, 256, 32, 8, 4, 8, 2.5, "fp8"),
    ("stream_mx", 40, 512, 512, 32, 8, 4, 8, 2.5, "mxfp4"),
    ("stream64_bf16", 240, 512, 256, 32, 8, 4, 4, 2.5, "bf16"),
    ("stream64_mx", 240, 512, 512, 32, 8, 4, 4, 2.5, "mxfp4"),
    ("stream64_fp8", 240, 512, 256, 32, 8, 4, 4, 2.5, "fp8"),
    ("g1_k6", 300, 384, 256, 64, 1, 1, 6, 2.5, "bf16"),
    ("all_groups", 700, 256, 256, 32, 8, 8, 8, 2.5, "bf16"),
    ("fp8_tiled", 600, 256, 128, 32, 8, 4, 8, 2.5, "fp8"),
    ("wide_gateup", 1500, 256, 256, 32, 8, 4, 8, 2.5, "bf16"),
    ("moderate_bf16", 250, 512, 256, 32, 8, 4, 8, 2.5, "bf16"),
    ("moderate_fp8", 240, 512, 256, 32, 8, 4, 8, 2.5, "fp8"),
    ("moderate_mx", 230, 512, 512, 32, 8, 4, 8, 2.5, "mxfp4"),
    ("moderate_mx_2rounds", 220, 1024, 1024, 32, 8, 4, 8, 2.5, "mxfp4"),
    ("edge_below_32", 127, 512, 256, 32, 8, 4, 8, 2.5, "bf16"),
    ("edge_above_64", 257, 512, 256, 32, 8, 4, 8, 2.5, "bf16"),
    ("edge_192_rows", 768, 512, 256, 32, 8, 4, 8, 2.5, "bf16"),
    ("down320_tiled", 600, 1280, 256, 32, 8, 4, 8, 2.5, "bf16"),
    ("down320_wide", 1500, 1280, 256, 32, 8, 4, 8, 2.5, "bf16"),
]


@pytest.mark.parametrize("name,T,H,I,E,G,Gk,K,alpha,weight", CASES, ids=[c[0] for c in CASES])
def test_forward_same_bytes_in_both_orders(name, T, H, I, E, G, Gk, K, alpha, weight):
    w = gen.Workload("layout_" + name, 1, T, H, I, E, G, Gk, K, alpha, 0.05, 0.02, "zero", weight, 1)
    C.say(f"[layout {name}] T={T} H={H} I={I} E={E} K={K} {weight}")
    _same_bytes(w, 9, what=name)


@pytest.mark.parametrize("name,T", [("dense_tiny", 7), ("dense_tiny", 64), ("dense_tiny", 1100),
                                    ("dense_tiny", 2000), ("dense_mx512", 64), ("dense_mx512", 1100),
                                    ("dense_fp8", 100), ("dense_fp8", 1500)])
def test_dense_same_bytes_in_both_orders(name, T):
    import sparse_moe_layer_top_amd as bm
    if name == "dense_fp8":
        w = gen.Workload("dense_tiny_fp8", 7, T, 256, 512, 1, 1, 1, 1, 1.0, 0.05, 0.02, "zero", "fp8", 7)
    elif name == "dense_mx512":     # MXFP4 in fragment order: H and I multiples of 512
        w = gen.Workload("dense_mx512", 12, T, 512, 512, 1, 1, 1, 1, 1.0, 0.05, 0.02, "zero", "mxfp4", 12)
    else:
        w = gen.workload(name, T)
    C.say(f"[layout dense {name}] T={T} {w.weight}")
    x, _, _ = gen.router_inputs(w, 0)
    m = {k: gen.expert_matrix(w, 0, k, 0) for k in ("gate", "up", "down")}
    d = C.dev()
    if w.weight == "bf16":
        W = {k: C.to_bf16(v) for k, v in m.items()}
    else:
        W = {k: torch.from_numpy(v[0]).to(d) for k, v in m.items()}
        W.update({"s_" + k: torch.from_numpy(v[1]).to(d) for k, v in m.items()})
    wt = {"bf16": bm.W_BF16, "fp8": bm.W_FP8_E4M3, "mxfp4": bm.W_MXFP4}[w.weight]
    outs = []
    for layout, WW in ((0, W), (1, C.packed(W))):
        cfg = bm.DenseConfig(w.hidden, w.inter, wt, layout)
        outs.append(C.bits_of(bm.beam_dense_mlp_forward(cfg, C.to_bf16(x), WW["gate"], WW["up"], WW["down"],
                                                        WW.get("s_gate"), WW.get("s_up"), WW.get("s_down"))))
    assert np.array_equal(outs[0], outs[1])


def test_block_and_noalloc_same_bytes_in_both_orders():
    import sparse_moe_layer_top_amd as bm
    w = gen.workload("tiny", 300)
    spec, x, wr, b = C.guarded(w, 3)
    W, _ = C.host_expert_weights(w, 3)
    P = C.packed(W)
    d = C.dev()
    xt, wrt, bt = C.router_tensors(x, wr, b)
    rng = np.random.default_rng(5)
    gpre = torch.from_numpy(rng.uniform(0.5, 1.5, w.hidden).astype(np.float32)).to(d)
    gpost = torch.from_numpy(rng.uniform(0.5, 1.5, w.hidden).astype(np.float32)).to(d)
    outs = []
    for layout, WW in ((0, W), (1, P)):
        cfg = C.cfg_of(w, layout)
        blk = bm.beam_moe_block_forward(cfg, 5, 1e-6, xt, gpre, gpost, wrt, bt, WW["gate"], WW["up"], WW["down"])
        na = torch.empty(w.T, w.hidden, dtype=torch.bfloat16, device=d)
        bm.beam_moe_forward_noalloc(cfg, xt, wrt, bt, WW["gate"], WW["up"], WW["down"], na)
        torch.cuda.synchronize()
        outs.append((C.bits_of(blk), C.bits_of(na)))
    assert np.array_equal(outs[0][0], outs[1][0])
    assert np.array_equal(outs[0][1], outs[1][1])


_PACKED = {}


def _real_packed(kind):
    from tests.test_gpu_parity import real_weights
    if kind not in _PACKED:
        _PACKED[kind] = C.packed(real_weights(kind))
        C.say(f"{kind} expert weights packed into fragment order")
    return _PACKED[kind]


@pytest.mark.parametrize("name", ["decode", "prefill", "skew", "fp8_decode", "fp8_prefill", "mxfp4_decode",
                                  "mxfp4_prefill", "spec_verify"])
def test_real_shape_same_bytes_in_both_orders(name):
    from tests.test_gpu_parity import real_weights
    w = gen.workload(name)
    C.say(f"[layout real {name}] T={w.T}")
    W = real_weights(w.weight)
    _real_packed(w.weight)
    spec, x, wr, b = C.guarded(w, 0)
    t = C.router_tensors(x, wr, b)
    out_r, ids_r, _ = C.run_forward(w, *t, W, layout=0)
    out_f, ids_f, _ = C.run_forward(w, *t, _PACKED[w.weight], layout=1)
    assert torch.equal(ids_r, ids_f)
    a, f = C.bits_of(out_r), C.bits_of(out_f)
    assert np.array_equal(a, f), f"{name}: {int((a != f).sum())} of {a.size} values differ"
