"""The build fails on register spills: the resource-report parser, the
allowance mechanism, and a real gfx950 build (hipcc cross-compiles without a
GPU) in which no kernel spills or uses scratch memory."""

import os

import pytest

from mla_decode_amd import build as B

REPORT = """\
x.hip:5:1: remark: Function Name: _ZN3mla6kernelEv [-Rpass-analysis=kernel-resource-usage]
x.hip:5:1: remark:     VGPRs: 243 [-Rpass-analysis=kernel-resource-usage]
x.hip:5:1: remark:     AGPRs: 0 [-Rpass-analysis=kernel-resource-usage]
x.hip:5:1: remark:     ScratchSize [bytes/lane]: 8 [-Rpass-analysis=kernel-resource-usage]
x.hip:5:1: remark:     Dynamic Stack: False [-Rpass-analysis=kernel-resource-usage]
x.hip:5:1: remark:     SGPRs Spill: 0 [-Rpass-analysis=kernel-resource-usage]
x.hip:5:1: remark:     VGPRs Spill: 2 [-Rpass-analysis=kernel-resource-usage]
x.hip:9:1: remark: Function Name: _ZN3mla5otherEv [-Rpass-analysis=kernel-resource-usage]
x.hip:9:1: remark:     VGPRs: 20 [-Rpass-analysis=kernel-resource-usage]
x.hip:9:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]
x.hip:9:1: remark:     SGPRs Spill: 0 [-Rpass-analysis=kernel-resource-usage]
x.hip:9:1: remark:     VGPRs Spill: 0 [-Rpass-analysis=kernel-resource-usage]
"""


def test_parse_report():
    u = B.parse_resource_usage(REPORT)
    assert set(u) == {"_ZN3mla6kernelEv", "_ZN3mla5otherEv"}
    k = u["_ZN3mla6kernelEv"]
    assert k["VGPRs"] == 243 and k["ScratchSize [bytes/lane]"] == 8 and k["VGPRs Spill"] == 2
    assert k["Dynamic Stack"] == "False"


def test_spills_fail_unless_allowed():
    u = B.parse_resource_usage(REPORT)
    probs = B.spill_problems(u, allowance={})
    assert len(probs) == 1 and "_ZN3mla6kernelEv" in probs[0]
    assert B.spill_problems(u, allowance={"_ZN3mla6kernelEv": (8, 2, 0)}) == []
    assert len(B.spill_problems(u, allowance={"_ZN3mla6kernelEv": (8, 1, 0)})) == 1   # the ratchet


def test_real_build_has_no_unallowed_spills(tmp_path):
    out = B.build(out=str(tmp_path / "libmla_check.so"))
    assert os.path.exists(out)
    u = B.LAST_USAGE
    assert B.spill_problems(u) == []
    # every kernel of the library: no spills and no scratch
    assert B.SPILL_ALLOWANCE == {}
    for name, r in u.items():
        assert r["ScratchSize [bytes/lane]"] == 0 and r["VGPRs Spill"] == 0 and r["SGPRs Spill"] == 0, name
    for k in ("decode64_kernel", "decode_kernel", "metadata_kernel", "combine_kernel"):
        assert any(k in n for n in u), k
