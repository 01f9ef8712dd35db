"""Host-side checks of the build's register / scratch guard (no GPU, no compiler run)."""

from causal_sliding_window_amd import build

REMARKS = """\
x.hip:5:1: remark: Function Name: kern_a [-Rpass-analysis=kernel-resource-usage]
x.hip:5:1: remark:     VGPRs: 256 [-Rpass-analysis=kernel-resource-usage]
x.hip:5:1: remark:     AGPRs: 184 [-Rpass-analysis=kernel-resource-usage]
x.hip:5:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]
x.hip:5:1: remark:     SGPRs Spill: 3 [-Rpass-analysis=kernel-resource-usage]
x.hip:5:1: remark:     VGPRs Spill: 0 [-Rpass-analysis=kernel-resource-usage]
    5 | __global__ void kern_a() {
      | ^
x.hip:9:1: remark: Function Name: kern_b [-Rpass-analysis=kernel-resource-usage]
x.hip:9:1: remark:     VGPRs: 512 [-Rpass-analysis=kernel-resource-usage]
x.hip:9:1: remark:     ScratchSize [bytes/lane]: 260 [-Rpass-analysis=kernel-resource-usage]
x.hip:9:1: remark:     SGPRs Spill: 0 [-Rpass-analysis=kernel-resource-usage]
x.hip:9:1: remark:     VGPRs Spill: 96 [-Rpass-analysis=kernel-resource-usage]
"""


def test_resource_report_parses_each_kernel():
    k = build.resource_report(REMARKS)
    assert set(k) == {"kern_a", "kern_b"}
    assert k["kern_a"]["AGPRs"] == "184"
    assert k["kern_b"]["ScratchSize [bytes/lane]"] == "260"


def test_guard_flags_vector_spills_and_scratch_only():
    bad = build.check_resources("x.hip", build.resource_report(REMARKS))
    assert len(bad) == 1 and "kern_b" in bad[0] and "260" in bad[0] and "96" in bad[0]
