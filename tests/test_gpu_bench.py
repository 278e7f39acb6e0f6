"""bench.py's measurement on small workloads (the MoE forward, the whole sublayer, the dense MLP):
each path runs, times its stages and reports its figures, so a change to the bench or the library's
argument checks cannot leave one of the bench's workloads broken."""
import numpy as np
import pytest
import torch

from synth import gen

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,block,layout", [("tiny", False, 1), ("tiny", True, 1), ("dense_tiny", False, 1),
                                               ("tiny", False, 0), ("dense_tiny", False, 0)])
def test_measure_runs(name, block, layout):
    import bench
    import sparse_moe_layer_top_amd as bm
    w = gen.workload(name)
    dev = torch.device("cuda:0")
    x, wr, b = gen.router_inputs(w, 0)
    W = gen.device_expert_weights(w, 0, dev)
    if layout:
        W = {k: (bm.beam_moe_pack_weights(v) if k in ("gate", "up", "down") else
                 bm.beam_moe_pack_scales(v) if v.dtype == torch.uint8 else v) for k, v in W.items()}
    m = bench.measure(w, W, x, wr, b, steps=3, warmup=1, block=block, layout=layout)
    assert m["ms_per_step"] > 0 and m["tokens_per_s"] > 0
    stages = bench.BLOCK_STAGES if block else (bench.DENSE_STAGES if w.n_experts == 1 else bench.STAGES)
    assert set(m["stage_ms"]) == set(stages)
    assert all(np.isfinite(v) and v >= 0 for v in m["stage_ms"].values())
    st = m["step_ms"]
    assert 0 < st["min"] <= st["median"] <= st["max"]
    assert m["roofline"]["kernel"] and m["roofline"]["frac"] > 0
    if w.n_experts > 1:
        assert m["routing"]["touched_experts"] > 0


def test_gemm_ceiling_reports_each_shape():
    import bench
    dev = torch.device("cuda:0")
    r = bench.gemm_ceiling(torch, dev, shapes=[(256, 512, 384)], reps=2, warmup=1)
    (g,) = r["gemm_ceiling"]
    assert (g["M"], g["K"], g["N"]) == (256, 512, 384)
    assert g["ms"] > 0 and g["TFLOPs"] > 0
    assert abs(g["frac"] - g["TFLOPs"] / bench.PEAK_BF16_TFLOPS) < 1e-3
