"""The build's check of the compiler's per-kernel resource report: a kernel that spills registers or
uses scratch memory fails the build (each spill is a round trip to memory in the hot loop)."""
import importlib.util
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _build_module():
    spec = importlib.util.spec_from_file_location("_beam_build_t", os.path.join(ROOT, "sparse_moe_layer_top_amd",
                                                                                 "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _remarks(name, vgprs, scratch, vspill, sspill=0):
    tag = " [-Rpass-analysis=kernel-resource-usage]"
    return "\n".join([
        f"k.hip:1:1: remark: Function Name: {name}{tag}",
        "   1 | void k() {",
        "      | ^",
        f"k.hip:1:1: remark:     TotalSGPRs: 40{tag}",
        f"k.hip:1:1: remark:     VGPRs: {vgprs}{tag}",
        f"k.hip:1:1: remark:     AGPRs: 0{tag}",
        f"k.hip:1:1: remark:     ScratchSize [bytes/lane]: {scratch}{tag}",
        f"k.hip:1:1: remark:     Dynamic Stack: False{tag}",
        f"k.hip:1:1: remark:     Occupancy [waves/SIMD]: 2{tag}",
        f"k.hip:1:1: remark:     SGPRs Spill: {sspill}{tag}",
        f"k.hip:1:1: remark:     VGPRs Spill: {vspill}{tag}",
        f"k.hip:1:1: remark:     LDS Size [bytes/block]: 0{tag}",
    ])


def test_resource_report_parsed_per_kernel():
    b = _build_module()
    text = "\n".join([_remarks("clean", 248, 0, 0), _remarks("spills", 256, 12, 2), _remarks("sgpr", 64, 0, 0, 3)])
    ks = b.kernel_resources(text)
    assert [k["kernel"] for k in ks] == ["clean", "spills", "sgpr"]
    assert ks[0]["VGPRs"] == 248 and ks[0]["ScratchSize"] == 0 and ks[0]["Occupancy"] == 2
    assert ks[1]["VGPRs Spill"] == 2 and ks[1]["ScratchSize"] == 12
    assert [k["kernel"] for k in b.spilling(ks)] == ["spills", "sgpr"]


def test_resource_flag_in_compile_command():
    b = _build_module()
    assert b.RESOURCE_REMARKS == "-Rpass-analysis=kernel-resource-usage"
    assert b.spilling(b.kernel_resources("no remarks here")) == []
