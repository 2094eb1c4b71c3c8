"""The build's check on the compiler's resource remarks: a slot-scheduled kernel (name
holding "wide") that spills to scratch memory fails the build (no GPU)."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
from io_aware_exact_fa2_amd import build  # noqa: E402

REMARKS = """\
a.hpp:9:1: remark: Function Name: _ZN2fa18fa_fwd_wide_kernelILb1ELi128E [-Rpass-analysis=kernel-resource-usage]
  9 | fa_fwd_wide_kernel(const Params p) {
a.hpp:9:1: remark:     VGPRs: 256 [-Rpass-analysis=kernel-resource-usage]
a.hpp:9:1: remark:     ScratchSize [bytes/lane]: {wide} [-Rpass-analysis=kernel-resource-usage]
b.hpp:3:1: remark: Function Name: _ZN2fa16fa_bwd_dq_kernelILb1E [-Rpass-analysis=kernel-resource-usage]
b.hpp:3:1: remark:     ScratchSize [bytes/lane]: 16 [-Rpass-analysis=kernel-resource-usage]
"""


def test_resource_remarks_parse():
    u = build.resource_usage(REMARKS.replace("{wide}", "0"))
    assert u["_ZN2fa18fa_fwd_wide_kernelILb1ELi128E"] == {
        "VGPRs": "256", "ScratchSize [bytes/lane]": "0"}
    assert u["_ZN2fa16fa_bwd_dq_kernelILb1E"]["ScratchSize [bytes/lane]"] == "16"


def test_spill_of_a_slot_scheduled_kernel_fails():
    build.check_no_spills(build.resource_usage(REMARKS.replace("{wide}", "0")))  # others may
    with pytest.raises(RuntimeError, match="fa_fwd_wide_kernel"):
        build.check_no_spills(build.resource_usage(REMARKS.replace("{wide}", "48")))


def test_build_messages_drop_remarks():
    res = type("R", (), {"stdout": "", "stderr": REMARKS + "x.hip:1:2: warning: real one\n"})()
    msgs = build._messages(res)
    assert msgs == ["x.hip:1:2: warning: real one"]
