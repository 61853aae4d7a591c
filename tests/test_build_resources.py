"""The build's kernel resource guard (host logic, no GPU): the compiler's per-kernel
resource remarks are parsed, and scratch memory anywhere, LDS beyond the LDS-shared
prefill kernel's five stages or LDS in a decode kernel fails the build.  (A run-time
index into a register array once made the compiler move the MXFP4 staging registers to
LDS: 94 208 bytes against the 49 152 of the three stages the kernel had then, and a 20 %
slower prefill call.)"""
from paged_kv_cache_413_amd import build as B

REMARKS = """\
x.hip:216:1: remark: Function Name: _ZN3pkv12_GLOBAL__N_118prefill_lds_kernelILi3ELi128ELi4EEEvNS_8AttnArgsE [-Rpass-analysis=kernel-resource-usage]
x.hip:216:1: remark:     TotalSGPRs: 74 [-Rpass-analysis=kernel-resource-usage]
x.hip:216:1: remark:     VGPRs: 248 [-Rpass-analysis=kernel-resource-usage]
x.hip:216:1: remark:     AGPRs: 0 [-Rpass-analysis=kernel-resource-usage]
x.hip:216:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]
x.hip:216:1: remark:     Dynamic Stack: False [-Rpass-analysis=kernel-resource-usage]
x.hip:216:1: remark:     Occupancy [waves/SIMD]: 2 [-Rpass-analysis=kernel-resource-usage]
x.hip:216:1: remark:     SGPRs Spill: 0 [-Rpass-analysis=kernel-resource-usage]
x.hip:216:1: remark:     VGPRs Spill: 0 [-Rpass-analysis=kernel-resource-usage]
x.hip:216:1: remark:     LDS Size [bytes/block]: 81920 [-Rpass-analysis=kernel-resource-usage]
  216 | __global__ void prefill_lds_kernel(AttnArgs a) {
      | ^
x.hip:106:1: remark: Function Name: _ZN3pkv12_GLOBAL__N_118decode_auto_kernelILi2ELi128ELi4ELb0ELb0EEEvNS_8AttnArgsE [-Rpass-analysis=kernel-resource-usage]
x.hip:106:1: remark:     VGPRs: 254 [-Rpass-analysis=kernel-resource-usage]
x.hip:106:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]
x.hip:106:1: remark:     SGPRs Spill: 35 [-Rpass-analysis=kernel-resource-usage]
x.hip:106:1: remark:     LDS Size [bytes/block]: 0 [-Rpass-analysis=kernel-resource-usage]
"""

PF = "_ZN3pkv12_GLOBAL__N_118prefill_lds_kernelILi3ELi128ELi4EEEvNS_8AttnArgsE"
DEC = "_ZN3pkv12_GLOBAL__N_118decode_auto_kernelILi2ELi128ELi4ELb0ELb0EEEvNS_8AttnArgsE"


def test_remarks_parse_into_fields():
    u = B.parse_resource_remarks(REMARKS)
    assert set(u) == {PF, DEC}
    assert u[PF]["VGPRs"] == "248" and u[PF]["LDS Size"] == "81920" and u[PF]["ScratchSize"] == "0"
    assert u[PF]["Occupancy"] == "2" and u[DEC]["SGPRs Spill"] == "35"


def test_clean_report_passes_and_register_spills_are_not_failures():
    assert B.check_resources(B.parse_resource_remarks(REMARKS)) == []


def test_scratch_and_excess_prefill_lds_fail():
    u = B.parse_resource_remarks(REMARKS)
    u[PF]["LDS Size"] = "94208"
    u[DEC]["ScratchSize"] = "16"
    bad = B.check_resources(u)
    assert len(bad) == 2
    assert any("LDS 94208" in b and "81920" in b for b in bad)
    assert any("scratch 16" in b for b in bad)


def test_stage_bytes_follow_head_dim():
    assert B._prefill_stage_lds("_ZN3pkv12_GLOBAL__N_118prefill_lds_kernelILi1ELi64ELi8EEEvNS_8AttnArgsE") == 40960
    assert B._prefill_stage_lds(PF) == 81920
    assert B._prefill_stage_lds(DEC) is None


def test_lds_in_a_decode_kernel_fails():
    """The decode kernels use no LDS: 4 608 bytes (72 per lane) appeared once when a
    run-time chunk index into the per-wave sequence cache made the compiler move it there."""
    u = B.parse_resource_remarks(REMARKS)
    u[DEC]["LDS Size"] = "4608"
    bad = B.check_resources(u)
    assert len(bad) == 1 and "LDS 4608" in bad[0] and "uses none" in bad[0]
