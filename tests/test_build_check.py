"""The build's kernel-resource check (no GPU): `build()` compiles every HIP
source with the compiler's per-kernel resource report and fails when a kernel
keeps anything in scratch memory.  Here the report parser is fed report lines
of the compiler's format, good and bad."""
import pytest

import __graft_entry__ as ge

GOOD = """\
x.hip:9:1: remark: Function Name: _Z4goodv [-Rpass-analysis=kernel-resource-usage]
x.hip:9:1: remark:     VGPRs: 32 [-Rpass-analysis=kernel-resource-usage]
x.hip:9:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]
x.hip:9:1: remark:     Dynamic Stack: False [-Rpass-analysis=kernel-resource-usage]
x.hip:9:1: remark:     SGPRs Spill: 12 [-Rpass-analysis=kernel-resource-usage]
x.hip:9:1: remark:     VGPRs Spill: 0 [-Rpass-analysis=kernel-resource-usage]
"""


def test_clean_report_passes(tmp_path):
    src = tmp_path / "x.hip"
    src.write_text("__global__ void good() {}\n")
    ge._check_resources(str(src), GOOD)  # scalar spills go to vector lanes: allowed


@pytest.mark.parametrize("bad", ["ScratchSize [bytes/lane]: 176", "VGPRs Spill: 4", "Dynamic Stack: True"])
def test_scratch_fails_the_build(tmp_path, bad):
    src = tmp_path / "x.hip"
    src.write_text("__global__ void bad() {}\n")
    key = bad.split(":")[0]
    lines = [l if key not in l else l.split("remark:")[0] + "remark:     " + bad + " [-Rpass-analysis=kernel-resource-usage]"
             for l in GOOD.splitlines()]
    with pytest.raises(RuntimeError, match="_Z4goodv"):
        ge._check_resources(str(src), "\n".join(lines))


def test_a_kernel_source_without_a_report_fails(tmp_path):
    src = tmp_path / "x.hip"
    src.write_text("__global__ void k() {}\n")
    with pytest.raises(RuntimeError, match="no kernel resource usage"):
        ge._check_resources(str(src), "")
    src.write_text("__device__ int table[4];\n")  # no kernels: nothing to report
    ge._check_resources(str(src), "")
