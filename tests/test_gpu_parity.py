"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Tiny layer: every step compared in full, several seeds, ragged token counts,
degenerate routings.  Real shape (hidden 5120, 256 experts, intermediate
2560): ids, weights and permutation compared in full at the real token counts,
in the launch configuration the benchmark times, outputs on sampled tokens
(the oracle computes a token's output from that token alone).
"""
import numpy as np
import pytest
import torch

import oracle
from synth import gen
from tests import gpu_cases as C

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import sparse_moe_layer_top_amd  # noqa: F401  (fails loudly if the library is not built)
    assert torch.cuda.is_available()


# ------------------------------------------------------------------ tiny ---

@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_tiny_forward_full(seed):
    w = gen.workload("tiny")
    spec, x, wr, b = C.guarded(w, seed)
    W, src = C.host_expert_weights(w, seed)
    out, ids, wts = C.run_forward(w, *C.router_tensors(x, wr, b), W)
    ref = oracle.forward(spec, x, wr, b, src.get)
    C.check_ids_w(ids.cpu().numpy(), wts.cpu().numpy(), ref["ids"], ref["w"])
    C.check_out(C.bits_of(out), ref["out"])


@pytest.mark.parametrize("T", [1, 2, 7, 63, 64, 65, 130, 257, 1000, 4095, 4097])
def test_tiny_ragged_tokens(T):
    w = gen.workload("tiny", T)
    spec, x, wr, b = C.guarded(w, 5)
    W, src = C.host_expert_weights(w, 5)
    out, ids, wts = C.run_forward(w, *C.router_tensors(x, wr, b), W)
    ref = oracle.forward(spec, x, wr, b, src.get)
    C.check_ids_w(ids.cpu().numpy(), wts.cpu().numpy(), ref["ids"], ref["w"])
    C.check_out(C.bits_of(out), ref["out"])


def test_tiny_route_and_permute_entry_points():
    import sparse_moe_layer_top_amd as bm
    w = gen.workload("tiny", 333)
    spec, x, wr, b = C.guarded(w, 2)
    cfg = C.cfg_of(w)
    xt, wrt, bt = C.router_tensors(x, wr, b)
    ids, wts = bm.beam_moe_route(cfg, xt, wrt, bt)
    off, sp, p2r = bm.beam_moe_permute(cfg, ids)
    torch.cuda.synchronize()
    rid, rw = oracle.route(spec, x, wr, b)
    C.check_ids_w(ids.cpu().numpy(), wts.cpu().numpy(), rid, rw)
    C.check_permutation(rid, off.cpu().numpy(), sp.cpu().numpy(), p2r.cpu().numpy(), w.n_experts)
    # a NULL bias column is no bias
    assert len(oracle.gap_violations(spec, x, wr, None)) == 0
    ids0, w0 = bm.beam_moe_route(cfg, xt, wrt, None)
    torch.cuda.synchronize()
    rid0, rw0 = oracle.route(spec, x, wr, None)
    C.check_ids_w(ids0.cpu().numpy(), w0.cpu().numpy(), rid0, rw0)


def test_tiny_all_tokens_same_experts():
    """A large bias on 8 experts of 2 groups: each of them gets every token (tiles span many rows)."""
    w = gen.workload("tiny", 300)
    spec = oracle.LayerSpec.of(w)
    x, wr, _ = gen.router_inputs(w, 0)
    b = np.full(w.n_experts, -20.0, np.float32)
    chosen = [4, 5, 6, 7, 20, 21, 22, 23]
    b[chosen] = 20.0
    W, src = C.host_expert_weights(w, 0)
    out, ids, wts = C.run_forward(w, *C.router_tensors(x, wr, b), W)
    ref = oracle.forward(spec, x, wr, b, src.get)
    assert (ref["ids"] == np.array(chosen)).all()
    C.check_ids_w(ids.cpu().numpy(), wts.cpu().numpy(), ref["ids"], ref["w"])
    C.check_out(C.bits_of(out), ref["out"])


def test_tiny_skewed_bias():
    w = gen.workload("tiny", 512)
    spec = oracle.LayerSpec.of(w)
    bias = (np.random.default_rng(9).standard_normal(w.n_experts) * 1.5).astype(np.float32)
    x, wr, b, _ = gen.guarded_router_inputs(w, 3, lambda x, wr, b: oracle.gap_violations(spec, x, wr, b), bias=bias)
    W, src = C.host_expert_weights(w, 3)
    out, ids, wts = C.run_forward(w, *C.router_tensors(x, wr, b), W)
    ref = oracle.forward(spec, x, wr, b, src.get)
    ld = np.bincount(ref["ids"].ravel(), minlength=w.n_experts)
    assert ld.max() > 2 * ld.mean()
    C.check_ids_w(ids.cpu().numpy(), wts.cpu().numpy(), ref["ids"], ref["w"])
    C.check_out(C.bits_of(out), ref["out"])


ODD_SHAPES = [
    # name, T, H, I, E, G, Gk, K, alpha, weight: smallest legal dims; no group limit with 32-row streaming
    # tiles (K = 6); every group kept (LDS-tiled GEMMs); fp8 on the LDS-tiled path; the
    # one-workgroup-per-CU gate/up (375 rows per expert on average: 272-row tiles, tall and short);
    # both one-workgroup-per-CU GEMMs at about 60 rows per expert (96-row tiles), bf16, fp8 and MXFP4
    # (MXFP4 also over two rounds of the four-window ring, whose scale bytes arrive one load per round)
    # and T*K/E at the schedule boundaries: exactly 32 and 64 rows per expert on average (the 96-row
    # one-workgroup-per-CU GEMMs) and one token to either side (streaming, LDS-tiled); exactly 192
    # (the 272-row gate/up) and one token below (LDS-tiled)
    ("h128", 37, 128, 128, 16, 4, 2, 4, 1.0, "bf16"),
    ("g1_k6", 300, 384, 256, 64, 1, 1, 6, 2.5, "bf16"),
    ("all_groups", 700, 256, 256, 32, 8, 8, 8, 2.5, "bf16"),
    ("fp8_tiled", 600, 256, 128, 32, 8, 4, 8, 2.5, "fp8"),
    ("wide_gateup", 1500, 256, 256, 32, 8, 4, 8, 2.5, "bf16"),
    ("moderate_bf16", 250, 512, 256, 32, 8, 4, 8, 2.5, "bf16"),
    ("moderate_fp8", 240, 512, 256, 32, 8, 4, 8, 2.5, "fp8"),
    ("moderate_mx", 230, 512, 512, 32, 8, 4, 8, 2.5, "mxfp4"),
    ("moderate_mx_2rounds", 220, 1024, 1024, 32, 8, 4, 8, 2.5, "mxfp4"),
    ("edge_32_rows", 128, 512, 256, 32, 8, 4, 8, 2.5, "bf16"),
    ("edge_below_32", 127, 512, 256, 32, 8, 4, 8, 2.5, "bf16"),
    ("edge_64_rows", 256, 512, 256, 32, 8, 4, 8, 2.5, "bf16"),
    ("edge_above_64", 257, 512, 256, 32, 8, 4, 8, 2.5, "bf16"),
    ("edge_192_rows", 768, 512, 256, 32, 8, 4, 8, 2.5, "bf16"),
    ("edge_below_192", 767, 512, 256, 32, 8, 4, 8, 2.5, "bf16"),
    # the LDS-tiled down GEMM over 320-column tiles (H a multiple of 320 and 256): 288-row tiles from
    # the tiled gate/up (about 150 rows per expert), and 272-row tiles from the one-workgroup-per-CU
    # gate/up (about 375 rows per expert: two tiles each, the second ragged)
    ("down320_tiled", 600, 1280, 256, 32, 8, 4, 8, 2.5, "bf16"),
    ("down320_wide", 1500, 1280, 256, 32, 8, 4, 8, 2.5, "bf16"),
]


@pytest.mark.parametrize("name,T,H,I,E,G,Gk,K,alpha,weight", ODD_SHAPES, ids=[o[0] for o in ODD_SHAPES])
def test_odd_shapes(name, T, H, I, E, G, Gk, K, alpha, weight):
    w = gen.Workload("odd_" + name, 1, T, H, I, E, G, Gk, K, alpha, 0.05, 0.02, "zero", weight, 1)
    C.say(f"[odd {name}] T={T} H={H} I={I} E={E} G={G} Gk={Gk} K={K}")
    spec, x, wr, b = C.guarded(w, 8)
    W, src = C.host_expert_weights(w, 8)
    out, ids, wts = C.run_forward(w, *C.router_tensors(x, wr, b), W)
    ref = oracle.forward(spec, x, wr, b, src.get)
    C.check_ids_w(ids.cpu().numpy(), wts.cpu().numpy(), ref["ids"], ref["w"])
    C.check_out(C.bits_of(out), ref["out"])


def test_tiny_fp8_weights():
    w = gen.Workload("tiny_fp8", 1, 96, 256, 128, 32, 8, 4, 8, 2.5, 0.05, 0.02, "zero", "fp8", 1)
    spec, x, wr, b = C.guarded(w, 4)
    W, src = C.host_expert_weights(w, 4)
    out, ids, wts = C.run_forward(w, *C.router_tensors(x, wr, b), W)
    ref = oracle.forward(spec, x, wr, b, src.get)
    C.check_ids_w(ids.cpu().numpy(), wts.cpu().numpy(), ref["ids"], ref["w"])
    C.check_out(C.bits_of(out), ref["out"])


def test_tiny_deterministic():
    w = gen.workload("tiny", 777)
    spec, x, wr, b = C.guarded(w, 6)
    W, _ = C.host_expert_weights(w, 6)
    t = C.router_tensors(x, wr, b)
    a = C.bits_of(C.run_forward(w, *t, W)[0])
    c = C.bits_of(C.run_forward(w, *t, W)[0])
    assert np.array_equal(a, c)


def test_zero_tokens():
    import sparse_moe_layer_top_amd as bm
    w = gen.workload("tiny")
    W, _ = C.host_expert_weights(w, 0)
    x = torch.empty(0, w.hidden, dtype=torch.bfloat16, device=C.dev())
    wr = torch.zeros(w.hidden, w.n_experts, device=C.dev())
    out = bm.beam_moe_forward(C.cfg_of(w), x, wr, None, W["gate"], W["up"], W["down"])
    assert out.shape == (0, w.hidden)


def test_permute_max_tokens():
    """The largest T the ABI accepts: 262144 tokens x 8 slots, random distinct ids per token."""
    import sparse_moe_layer_top_amd as bm
    T, E, K = bm.MAX_TOKENS, 256, 8
    rng = np.random.default_rng(11)
    ids = np.sort(np.argsort(rng.random((T, E), dtype=np.float32), axis=1)[:, :K], axis=1).astype(np.int32)
    cfg = bm.Config()
    off, sp, p2r = bm.beam_moe_permute(cfg, torch.from_numpy(ids).to(C.dev()))
    torch.cuda.synchronize()
    C.check_permutation(ids, off.cpu().numpy(), sp.cpu().numpy(), p2r.cpu().numpy(), E)


# ------------------------------------------------------------ real shape ---

_SOURCES = {}
_WEIGHTS = {}
_KIND_WORKLOAD = {"bf16": "decode", "fp8": "fp8_decode", "mxfp4": "mxfp4_decode"}


def real_source(kind):
    """All 256 experts of the real-shape layer's weights (bf16, fp8 or MXFP4) on the host, generated
    once: the oracle reads them here and the device copy is uploaded from them."""
    if kind not in _SOURCES:
        w = gen.workload(_KIND_WORKLOAD[kind])
        C.say(f"generating {kind} expert weights on the host (256 experts, real shape)")
        src = gen.ExpertSource(w, 0)
        src.prefetch(range(w.n_experts))
        _SOURCES[kind] = src
    return _SOURCES[kind]


def real_weights(kind):
    if kind not in _WEIGHTS:
        w = gen.workload(_KIND_WORKLOAD[kind])
        src = real_source(kind)
        d = C.dev()
        div = 2 if kind == "mxfp4" else 1
        E = w.n_experts
        if kind == "bf16":
            t = {k: torch.empty(E, *(w.inter, w.hidden) if k != "down" else (w.hidden, w.inter),
                                dtype=torch.bfloat16, device=d) for k in ("gate", "up", "down")}
            for k in t:
                for e in range(E):
                    t[k][e].copy_(torch.from_numpy(src.get(k, e).view(np.int16)).view(torch.bfloat16))
        else:
            t = {}
            for k in ("gate", "up", "down"):
                t[k] = torch.from_numpy(np.stack([src.get(k, e)[0] for e in range(E)])).to(d)
                t["s_" + k] = torch.from_numpy(np.stack([src.get(k, e)[1] for e in range(E)])).to(d)
            assert t["gate"].shape[-1] == w.hidden // div
        C.say(f"{kind} expert weights on the device")
        _WEIGHTS[kind] = t
    return _WEIGHTS[kind]


# real-shape workloads; output parity on a few sampled tokens (decode shapes) or on at least 128
# tokens covering every row of the most loaded expert's row tiles (the prefill shapes)
REAL = [("decode", 8), ("prefill", 128), ("skew", 128), ("fp8_decode", 8), ("fp8_prefill", 128),
        ("mxfp4_decode", 8), ("mxfp4_prefill", 128)]


@pytest.mark.parametrize("name,n_sample", REAL)
def test_real_shape_forward(name, n_sample):
    w = gen.workload(name)
    C.say(f"[{name}] T={w.T} inputs")
    spec, x, wr, b = C.guarded(w, 0)
    W = real_weights(w.weight)
    C.say(f"[{name}] forward on the GPU")
    out, ids, wts = C.run_forward(w, *C.router_tensors(x, wr, b), W)
    C.say(f"[{name}] oracle routing over all {w.T} tokens")
    rid, rw = oracle.route(spec, x, wr, b)
    C.check_ids_w(ids.cpu().numpy(), wts.cpu().numpy(), rid, rw)
    if n_sample >= 128:
        sample, e, ne = C.coverage_sample(rid, w.n_experts, n_min=n_sample, seed=1234)
        C.say(f"[{name}] {len(sample)} tokens: every permuted row of expert {e} ({ne} rows, up to 576, "
              f"and its last 288) and seeded others")
    else:
        rng = np.random.default_rng(1234)
        sample = np.unique(np.concatenate([[0, w.T - 1], rng.choice(w.T, n_sample, replace=False)]))
    src = real_source(w.weight)
    C.say(f"[{name}] oracle forward on {len(sample)} sampled tokens")
    ref = C.oracle_forward_threads(spec, x[sample], wr, b, src.get)
    assert np.array_equal(ref["ids"], rid[sample])
    C.check_out(C.bits_of(out)[sample], ref["out"], what=f"{name} output")


def test_real_shape_skew_tile_edges():
    """Skewed routing at T = 8192: 256 rows per expert on average, so the GEMMs run one workgroup
    per CU over row tiles; the most loaded expert spans many tiles, others fall just above 256 rows
    or hold a handful.  Ids and weights for every token; outputs for tokens at row-tile edges (the
    first row, and rows k*t - 1 and k*t for tile heights t of 144, 272 and 288 and k = 1..3, and the
    last row of the most loaded expert; the rows past 256 of an expert with 257..272; the least
    loaded expert's first row)."""
    w = gen.workload("skew", 8192)
    spec, x, wr, b = C.guarded(w, 0)
    W = real_weights("bf16")
    out, ids, wts = C.run_forward(w, *C.router_tensors(x, wr, b), W)
    rid, rw = oracle.route(spec, x, wr, b)
    C.check_ids_w(ids.cpu().numpy(), wts.cpu().numpy(), rid, rw)
    load = np.bincount(rid.ravel(), minlength=w.n_experts)
    assert load.max() > 2 * 272, "the skewed draw no longer gives an expert several tiles"

    def tokens_of(e):   # permuted row r of expert e is its r-th token in ascending order
        return np.nonzero((rid == e).any(axis=1))[0]

    picks = []
    big = tokens_of(int(load.argmax()))
    edges = {0} | {k * t + d for t in (144, 272, 288) for k in (1, 2, 3) for d in (-1, 0)}
    picks += [big[r] for r in sorted(edges) if r < len(big)] + [big[-1]]
    near = np.nonzero((load > 256) & (load <= 272))[0]
    if len(near):
        t = tokens_of(int(near[0]))
        picks += [t[256], t[-1]]
    small = np.nonzero(load > 0)[0][np.argmin(load[load > 0])]
    picks.append(tokens_of(int(small))[0])
    sample = np.unique(np.array(picks))
    C.say(f"[skew 8192] max load {load.max()}, oracle forward on {len(sample)} tokens")
    ref = C.oracle_forward_threads(spec, x[sample], wr, b, real_source("bf16").get)
    assert np.array_equal(ref["ids"], rid[sample])
    C.check_out(C.bits_of(out)[sample], ref["out"], what="skew 8192 output")


def test_real_shape_max_tokens():
    """The largest T the ABI accepts, 262,144 tokens (2M (token, slot) pairs, about 8K rows per
    expert: the tiled kernels with some 29 row tiles per expert), balanced routing.  Ids and
    weights bit-exact / to 1e-5 for every token whose oracle score gaps clear the guard; the
    others (near-ties, not re-drawn at this size) must still be valid selections; outputs on
    sampled tokens."""
    import sparse_moe_layer_top_amd as bm
    w = gen.workload("prefill", bm.MAX_TOKENS)
    spec = oracle.LayerSpec.of(w)
    C.say(f"[max tokens] T={w.T} inputs")
    x, wr, b = gen.router_inputs(w, 0)
    W = real_weights("bf16")
    C.say("[max tokens] forward on the GPU")
    out, ids, wts = C.run_forward(w, *C.router_tensors(x, wr, b), W)
    ids, wts = ids.cpu().numpy(), wts.cpu().numpy()
    C.say("[max tokens] oracle routing in chunks")
    near = []
    chunk = 16384
    for s0 in range(0, w.T, chunk):
        sl = slice(s0, min(s0 + chunk, w.T))
        rid, rw = oracle.route(spec, x[sl], wr, b)
        bad = oracle.gap_violations(spec, x[sl], wr, b)
        ok = np.ones(len(rid), bool)
        ok[bad] = False
        C.check_ids_w(ids[sl][ok], wts[sl][ok], rid[ok], rw[ok])
        near.extend((s0 + bad).tolist())
    near = np.asarray(near, np.int64)
    C.say(f"[max tokens] {len(near)} near-tie tokens: kept groups and top-{w.top_k} valid within 1e-6, weights")
    if len(near):
        C.check_valid_selection(spec, oracle.router_scores(x[near], wr, b), ids[near], wts[near], tol=1e-6)
    rng = np.random.default_rng(77)
    cand = np.setdiff1d(np.concatenate([[0, w.T - 1], rng.choice(w.T, 8, replace=False)]), near)
    C.say(f"[max tokens] oracle forward on {len(cand)} sampled tokens")
    ref = C.oracle_forward_threads(spec, x[cand], wr, b, real_source("bf16").get)
    assert np.array_equal(ref["ids"], ids[cand])
    C.check_out(C.bits_of(out)[cand], ref["out"], what="max tokens output")


@pytest.mark.parametrize("name", ["decode", "prefill", "skew"])
def test_real_shape_permute(name):
    import sparse_moe_layer_top_amd as bm
    w = gen.workload(name)
    spec, x, wr, b = C.guarded(w, 0)
    rid, _ = oracle.route(spec, x, wr, b)
    off, sp, p2r = bm.beam_moe_permute(C.cfg_of(w), torch.from_numpy(rid).to(C.dev()))
    torch.cuda.synchronize()
    C.check_permutation(rid, off.cpu().numpy(), sp.cpu().numpy(), p2r.cpu().numpy(), w.n_experts)


def test_real_shape_deterministic():
    w = gen.workload("decode")
    spec, x, wr, b = C.guarded(w, 0)
    W = real_weights("bf16")
    t = C.router_tensors(x, wr, b)
    a = C.bits_of(C.run_forward(w, *t, W)[0])
    c = C.bits_of(C.run_forward(w, *t, W)[0])
    assert np.array_equal(a, c)
