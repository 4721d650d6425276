"""CPU checks of what the compiler made of the kernels (no GPU needed).

The build records each kernel's registers, spills and scratch from hipcc's
resource-usage remarks.  A kernel here streams the cache and must keep its
tiles in registers: scratch traffic per lane would add to every tile's
latency.  A lambda or helper that stops being inlined shows up as a stack
frame in scratch and a jump in VGPRs (the fp32 mirror kernel once went from
114 to 225 VGPRs this way), so every kernel must use no scratch, except the
decode partial kernel at eight query heads per KV head, whose register tiles
exceed the 256 VGPRs of one wave (it runs correctly and is not a measured
configuration).
"""
import json
import os

import pytest

from decode_attention_int8_kv_amd import build

# kernels allowed a scratch frame (mangled-name fragments)
SPILL_ALLOWED = ("q8_attn_partial_kernelILi8E",)


@pytest.fixture(scope="module")
def resources():
    if not os.path.exists(build.RESOURCES) or (
            os.path.exists(build.OUT) and os.path.getmtime(build.RESOURCES) < os.path.getmtime(build.OUT) - 60):
        build.build()
    return json.load(open(build.RESOURCES))


def test_remark_parser_reads_the_fields():
    text = "\n".join([
        "a.hip:1:1: remark: Function Name: _Z3fooPi [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:1:1: remark:     VGPRs: 37 [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:1:1: remark:     ScratchSize [bytes/lane]: 16 [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:1:1: remark:     Occupancy [waves/SIMD]: 8 [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:9:1: remark: Function Name: _Z3barv [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:9:1: remark:     VGPRs Spill: 3 [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:2:2: warning: unrelated",
    ])
    got = build.parse_resource_remarks(text)
    assert got == {"_Z3fooPi": {"vgprs": 37, "scratch": 16, "occupancy": 8}, "_Z3barv": {"vgpr_spill": 3}}


def test_every_kernel_is_recorded(resources):
    names = " ".join(resources)
    for frag in ("q8_append_kernel", "q8_attn_partial_kernelILi2ELb1E", "q8_attn_partial_kernelILi4ELb1E",
                 "q8_attn_merge_kernel", "q8_attn_f32_partial_kernel", "q8_step_plan_kernel",
                 "q8_prefill_kernel", "q8_sparse_probe_kernel", "q8_sparse_select_kernel",
                 "q8_sparse_attend_kernel", "q8_quantize_q_kernel", "q8_stream_read_kernel"):
        assert frag in names, frag


def test_no_kernel_uses_scratch(resources):
    bad = {k: v for k, v in resources.items()
           if (v.get("scratch", 0) or v.get("vgpr_spill", 0)) and not any(a in k for a in SPILL_ALLOWED)}
    assert not bad, json.dumps(bad, indent=1)


def test_streaming_kernels_keep_their_occupancy(resources):
    # waves per SIMD the tile pipelines were tuned for: the G = 2 decode (the
    # 2B shape), of either cut (third template argument: false for the
    # balanced cut, true for the batch-invariant one, which also holds the
    # next chunk's tile while a chunk's state is written), keeps three; the
    # fp32 mirror decode at G = 2 keeps four
    def occ(frag):
        return min(v["occupancy"] for k, v in resources.items() if frag in k)
    assert occ("q8_attn_partial_kernelILi2ELb1ELb0E") >= 3
    assert occ("q8_attn_partial_kernelILi2ELb1ELb1E") >= 3
    assert occ("q8_attn_f32_partial_kernelILi2E") >= 4
    assert occ("q8_attn_partial_kernelILi4ELb1E") >= 2
    # the prefill's 8-wave workgroup needs two waves per SIMD (one workgroup per CU)
    assert occ("q8_prefill_kernel") >= 2
