"""The build refuses kernels that spill to scratch (parser of the compiler's
resource remarks, on a block of the form hipcc prints)."""
import pytest

from recurrent_state_updates_amd import build as B

BLOCK = """x.hip:9:1: remark: Function Name: _ZN3dlk6kernelEv [-Rpass-analysis=kernel-resource-usage]
    9 |   int a) {
      | ^
x.hip:9:1: remark:     TotalSGPRs: 18 [-Rpass-analysis=kernel-resource-usage]
x.hip:9:1: remark:     VGPRs: 158 [-Rpass-analysis=kernel-resource-usage]
x.hip:9:1: remark:     ScratchSize [bytes/lane]: {scratch} [-Rpass-analysis=kernel-resource-usage]
x.hip:9:1: remark:     Occupancy [waves/SIMD]: 3 [-Rpass-analysis=kernel-resource-usage]
x.hip:9:1: remark:     SGPRs Spill: 0 [-Rpass-analysis=kernel-resource-usage]
x.hip:9:1: remark:     VGPRs Spill: {spill} [-Rpass-analysis=kernel-resource-usage]"""


def _lines(spill, scratch):
    return BLOCK.replace("{spill}", str(spill)).replace("{scratch}", str(scratch)).splitlines()


def test_clean_kernel_passes():
    B.check_resources("x.hip", _lines(0, 0))


@pytest.mark.parametrize("spill,scratch", [(12, 48), (0, 16)])
def test_spilling_kernel_is_refused(spill, scratch):
    with pytest.raises(RuntimeError, match="_ZN3dlk6kernelEv"):
        B.check_resources("x.hip", _lines(spill, scratch))
