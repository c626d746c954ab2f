"""The build's refusal of kernels that use scratch or call out-of-line device
functions, checked on synthetic compiler resource reports (no GPU, no hipcc)."""
from gqa_kv_cache_02_amd import build

_R = "[-Rpass-analysis=kernel-resource-usage]"


def _report(*funcs):
    lines = []
    for name, scratch in funcs:
        lines.append(f"x.hip:10:1: remark: Function Name: {name} {_R}")
        lines.append(f"x.hip:10:1: remark:     VGPRs: 217 {_R}")
        lines.append(f"x.hip:10:1: remark:     ScratchSize [bytes/lane]: {scratch} {_R}")
    return "\n".join(lines)


def test_kernels_without_scratch_pass():
    rep = _report(("_ZN3gqa19prefill_mfma_kernelILi128ELb0EEEvNS_11PrefillArgsE", 0),
                  ("_ZN3gqa13decode_kernelILi64ELb1ELb0EEEvNS_10DecodeArgsE", 0),
                  ("_ZN3gqa19decode_merge_kernelILi128ELb0EEEvNS_9MergeArgsE", 0))
    assert build.resource_violations(rep) == []


def test_scratch_and_outlined_functions_are_refused():
    lam = "_ZZN3gqa19prefill_mfma_kernelILi64ELb0EEEvNS_11PrefillArgsEENKUliPKhE_clEiS3_"
    rep = _report((lam, 0), ("_ZN3gqa19prefill_mfma_kernelILi64ELb0EEEvNS_11PrefillArgsE", 640))
    bad = build.resource_violations(rep)
    assert len(bad) == 2
    assert bad[0].startswith(lam) and "out of line" in bad[0]
    assert "640 bytes of scratch" in bad[1]
