"""The library build refuses decode kernels that use scratch memory: their
LDS copies are waited for with static vmcnt counts that a spill's scratch
loads and stores would throw off (silently wrong results)."""
import importlib.util
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _build_mod():
    spec = importlib.util.spec_from_file_location("_kvq_build_t", os.path.join(ROOT, "decode_attention_asym_amd", "build.py"))
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


def _remarks(name, scratch=0, vspill=0, sspill=0):
    f = "x.hip:1:1: remark: {}: {} [-Rpass-analysis=kernel-resource-usage]"
    return "\n".join([
        "x.hip:1:1: remark: Function Name: " + name + " [-Rpass-analysis=kernel-resource-usage]",
        f.format("    VGPRs", 137), f.format("    ScratchSize [bytes/lane]", scratch),
        f.format("    SGPRs Spill", sspill), f.format("    VGPRs Spill", vspill),
        f.format("    LDS Size [bytes/block]", 11264),
    ])


def test_clean_decode_kernels_pass():
    b = _build_mod()
    txt = _remarks("_ZN3kvq12_GLOBAL__N_113decode_kernelILi128E") + "\n" + _remarks("_ZN3kvq5mergeE", scratch=64)
    u = b.resource_usage(txt)
    assert u["_ZN3kvq12_GLOBAL__N_113decode_kernelILi128E"]["ScratchSize [bytes/lane]"] == "0"
    b.check_no_scratch(u)  # only decode kernels are held to it


@pytest.mark.parametrize("kw", [{"scratch": 16}, {"vspill": 3}, {"sspill": 2}])
def test_spilling_decode_kernel_fails(kw):
    b = _build_mod()
    u = b.resource_usage(_remarks("_ZN3kvq12_GLOBAL__N_119decode_mixed_kernelILi128E", **kw))
    with pytest.raises(RuntimeError, match="must not use scratch"):
        b.check_no_scratch(u)


def test_missing_remarks_fail():
    b = _build_mod()
    with pytest.raises(RuntimeError, match="no decode kernel"):
        b.check_no_scratch({})
