"""The build refuses kernels that spill to scratch memory: the parser of the
compiler's resource remarks that it relies on."""

from quantized_speculative_expert_amd.build import scratch_users


def test_scratch_users_names_spilling_kernels_only():
    remarks = "\n".join([
        "a.hip:9:1: remark: Function Name: _Zspill [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:9:1: remark:     VGPRs: 128 [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:9:1: remark:     ScratchSize [bytes/lane]: 20 [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:9:1: remark: Function Name: _Zclean [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:9:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]",
        "warning: unknown target feature 'packed-fp32-ops'",
    ])
    assert scratch_users(remarks) == [("_Zspill", 20)]
    assert scratch_users("") == []
