"""The compiler's resource figures of every kernel in the last build (CPU).

A kernel that spills vector registers keeps them in scratch memory: each
reload is a vector-memory load, and in the expert GEMMs the wait for it also
waits for every transfer and store issued before it (the vector-memory
counter completes in order), which stalls the k-stage pipeline. So no kernel
may spill VGPRs or use scratch at all. SGPR spills go to VGPR lanes, not to
memory, and are allowed.
"""
import json
import os

import pytest

from sparse_moe_diffusion_amd import build as B


def _usage():
    if not os.path.exists(B.RESOURCES):
        pytest.skip("no resource figures: the library was not built here")
    with open(B.RESOURCES) as f:
        return json.load(f)


def test_every_source_reports():
    u = _usage()
    srcs = {v["source"] for v in u.values()}
    assert srcs == {s for s in B.SOURCES if s.endswith(".hip")}, srcs
    # the expert GEMM's forms are all there
    assert sum("gemm_bf16_kernel" in k for k in u) >= 10


def test_no_vgpr_spills_or_scratch():
    bad = {k: (v.get("VGPRs"), v.get("VGPRs Spill"), v.get("ScratchSize [bytes/lane]"))
           for k, v in _usage().items()
           if v.get("VGPRs Spill", 0) or v.get("ScratchSize [bytes/lane]", 0)
           or v.get("Dynamic Stack") == "True"}
    assert not bad, bad


def test_vgpr_budget_fits_occupancy():
    # one workgroup per CU of 8 waves (2 per SIMD) leaves 256 VGPRs per wave,
    # and the compiler's occupancy figure must allow the launch's waves
    for k, v in _usage().items():
        assert v["VGPRs"] + v.get("AGPRs", 0) <= 512, k
        if "gemm_bf16_kernel" in k:
            assert v["Occupancy [waves/SIMD]"] >= 2, (k, v)


def test_parse_resource_usage():
    text = (
        "a.hip:1:1: remark: Function Name: _Zk1 [-Rpass-analysis=kernel-resource-usage]\n"
        "   59 |     foo\n"
        "a.hip:1:1: remark:     VGPRs: 59 [-Rpass-analysis=kernel-resource-usage]\n"
        "a.hip:1:1: remark:     LDS Size [bytes/block]: 1024 [-Rpass-analysis=kernel-resource-usage]\n"
        "a.hip:1:1: remark:     Dynamic Stack: False [-Rpass-analysis=kernel-resource-usage]\n"
        "a.hip:9:1: remark: Function Name: _Zk2 [-Rpass-analysis=kernel-resource-usage]\n"
        "a.hip:9:1: remark:     VGPRs Spill: 3 [-Rpass-analysis=kernel-resource-usage]\n")
    u = B.parse_resource_usage(text)
    assert u == {"_Zk1": {"VGPRs": 59, "LDS Size [bytes/block]": 1024,
                          "Dynamic Stack": "False"},
                 "_Zk2": {"VGPRs Spill": 3}}
