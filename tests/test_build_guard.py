"""The build's resource guard (host-only): a kernel report with a VGPR spill
or scratch use must be flagged, an SGPR spill (which goes to VGPR lanes) and
a clean report must not."""

from lm_head_vocab_amd.build import resource_problems

CLEAN = """x.hip:1:1: remark: Function Name: _Z3fooPf [-Rpass-analysis=kernel-resource-usage]
x.hip:1:1: remark:     SGPRs: 40 [-Rpass-analysis=kernel-resource-usage]
x.hip:1:1: remark:     VGPRs: 61 [-Rpass-analysis=kernel-resource-usage]
x.hip:1:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]
x.hip:1:1: remark:     SGPRs Spill: 4 [-Rpass-analysis=kernel-resource-usage]
x.hip:1:1: remark:     VGPRs Spill: 0 [-Rpass-analysis=kernel-resource-usage]
"""


def test_clean_report_passes():
    assert resource_problems(CLEAN) == []


def test_vgpr_spill_and_scratch_are_flagged():
    bad = CLEAN.replace("VGPRs Spill: 0", "VGPRs Spill: 47").replace("ScratchSize [bytes/lane]: 0",
                                                                      "ScratchSize [bytes/lane]: 192")
    out = resource_problems(bad)
    assert len(out) == 2 and all(o.startswith("_Z3fooPf") for o in out)
    assert any("VGPRs Spill = 47" in o for o in out) and any("ScratchSize" in o for o in out)
