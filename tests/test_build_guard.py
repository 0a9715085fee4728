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


def test_no_remarks_at_all_is_refused():
    """A source whose compile printed no resource remarks (renamed fields, or
    remarks no longer forwarded from the device pass) cannot pass unchecked."""
    with pytest.raises(RuntimeError, match="no kernel resource remarks"):
        B.check_resources("x.hip", ["x.hip:1:1: warning: something else"])


@pytest.mark.parametrize("drop", ["VGPRs Spill", "ScratchSize"])
def test_block_missing_a_field_is_refused(drop):
    lines = [ln for ln in _lines(0, 0) if drop not in ln]
    with pytest.raises(RuntimeError, match="without a spill count or a scratch size"):
        B.check_resources("x.hip", lines)


def test_fields_are_reported_per_kernel():
    blocks = B.check_resources("x.hip", _lines(0, 0))
    assert blocks["_ZN3dlk6kernelEv"]["VGPRs"] == 158
    assert blocks["_ZN3dlk6kernelEv"]["Occupancy [waves/SIMD]"] == 3


def test_a_failed_build_leaves_no_library(tmp_path, monkeypatch):
    """The library is removed before compiling, so a refused build cannot
    leave an older library next to the package for load_library() to find."""
    lib = tmp_path / "libdeltalog.so"
    lib.write_bytes(b"stale")
    monkeypatch.setattr(B, "LIB", str(lib))
    monkeypatch.setattr(B, "BUILD_DIR", str(tmp_path / "_build"))
    monkeypatch.setattr(B, "SOURCES", [("does_not_exist.hip", "does_not_exist", [])])
    with pytest.raises(RuntimeError):
        B.build()
    assert not lib.exists()
