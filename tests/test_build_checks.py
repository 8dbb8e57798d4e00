"""The build refuses hot kernels that would keep state in scratch memory.

The compiler's kernel-resource remarks are parsed per kernel; a hot kernel
(MFMA prefill / decode, split-K decode) with scratch bytes or VGPR spills makes
the build fail instead of shipping a many-times-slower library.
"""
import pytest

from sparse_attention_layerrouter_amd import build

REMARKS = """\
prefill.hip:150:1: remark: Function Name: _ZN2fa12_GLOBAL__N_119prefill_bf16_kernelILi128ELi1EEEvPKt [-Rpass-analysis=kernel-resource-usage]
prefill.hip:150:1: remark:     VGPRs: 202 [-Rpass-analysis=kernel-resource-usage]
prefill.hip:150:1: remark:     AGPRs: 0 [-Rpass-analysis=kernel-resource-usage]
prefill.hip:150:1: remark:     ScratchSize [bytes/lane]: {scratch} [-Rpass-analysis=kernel-resource-usage]
prefill.hip:150:1: remark:     Occupancy [waves/SIMD]: 2 [-Rpass-analysis=kernel-resource-usage]
prefill.hip:150:1: remark:     VGPRs Spill: {spill} [-Rpass-analysis=kernel-resource-usage]
prefill.hip:150:1: remark:     LDS Size [bytes/block]: 65536 [-Rpass-analysis=kernel-resource-usage]
prefill.hip:400:1: remark: Function Name: _ZN2fa12_GLOBAL__N_122prefill_generic_kernelIfLi128ELi1EEEv [-Rpass-analysis=kernel-resource-usage]
prefill.hip:400:1: remark:     ScratchSize [bytes/lane]: 64 [-Rpass-analysis=kernel-resource-usage]
prefill.hip:400:1: remark:     VGPRs Spill: 0 [-Rpass-analysis=kernel-resource-usage]
"""


def test_remarks_parse_per_kernel():
    res = build._resources(REMARKS.format(scratch=0, spill=0))
    hot = [k for k in res if "prefill_bf16_kernel" in k]
    assert len(res) == 2 and len(hot) == 1
    assert res[hot[0]]["VGPRs"] == 202 and res[hot[0]]["LDS Size [bytes/block]"] == 65536


def test_clean_hot_kernels_pass_and_cold_scratch_is_allowed():
    build.check_resources(build._resources(REMARKS.format(scratch=0, spill=0)))


@pytest.mark.parametrize("scratch,spill", [(768, 0), (8, 1)])
def test_hot_kernel_with_scratch_or_spills_is_refused(scratch, spill):
    with pytest.raises(RuntimeError, match="prefill_bf16_kernel"):
        build.check_resources(build._resources(REMARKS.format(scratch=scratch, spill=spill)))
