"""Register and scratch gate (CPU: the compiler's own resource report, no GPU).

LDS or register overflow spills silently to scratch memory (CK/MI50 notes section 4.3,
first pitfall).  Every kernel of the library is compiled here with the resource report
and must keep zero scratch and zero spilled registers, except the fp32 accuracy-path
kernels listed below, whose spills are known and may not grow.  The fast paths' waves
per SIMD are pinned too: losing one is a silent slowdown."""
import re
import tempfile

import pytest

from exact_attention_90_amd import build

# fp32 inputs run on the fp32 matrix cores with fp32 P; at d >= 128 their registers
# overflow (the accuracy path, not a speed path): bytes of scratch per lane, at most
KNOWN_SCRATCH = {
    r"fa_fwd32_kernelILi128ELb0E": 56,
    r"fa_fwd32_kernelILi128ELb1E": 68,   # the statistics-recording form
    r"fa_fwd32_kernelILi256ELb0E": 404,
    r"fa_fwd32_kernelILi256ELb1E": 400,
    r"fa_bwd32_dkdv_kernelILi128E": 84,
}
# (kernel name pattern, waves per SIMD) of the production 16-bit forward kernels
OCCUPANCY = [
    (r"fa_fwd16_kernelILi128ELb[01]ELi8ELi1ELb0E", 2),
    (r"fa_fwd16_kernelILi64ELb[01]ELi4ELi2ELb0E", 2),
    (r"fa_fwd16_kernelILi256ELb[01]ELi4ELi1ELb0E", 1),
]


@pytest.fixture(scope="module")
def usage():
    with tempfile.TemporaryDirectory() as d:
        return build.resource_usage(d)


def test_every_kernel_reported(usage):
    names = " ".join(usage)
    for part in ("fa_fwd16_kernel", "fa_fwd32_kernel", "fa_merge_kernel", "naive_scores_kernel",
                 "naive_softmax_kernel", "naive_pv_kernel", "fa_bwd_dkdv_kernel",
                 "fa_bwd_dq_kernel", "fa_bwd_prep_kernel", "fa_sum_slots"):
        assert part in names, f"no resource record for {part}"
    for name, rec in usage.items():
        assert {"vgpr", "scratch", "vgpr_spill"} <= set(rec), (name, rec)


def test_no_scratch_or_spills_outside_the_known_fp32_kernels(usage):
    for name, rec in usage.items():
        limit = next((v for pat, v in KNOWN_SCRATCH.items() if re.search(pat, name)), None)
        if limit is None:
            assert rec["scratch"] == 0 and rec["vgpr_spill"] == 0 and rec.get("sgpr_spill", 0) == 0, (
                f"{name} spills: {rec}")
        else:
            assert rec["scratch"] <= limit, f"{name} scratch grew: {rec['scratch']} > {limit} B/lane"


def test_fast_paths_keep_their_waves_per_simd(usage):
    for pat, waves in OCCUPANCY:
        hits = [n for n in usage if re.search(pat, n)]
        assert len(hits) == 2, (pat, hits)  # binary16 and bfloat16
        for n in hits:
            assert usage[n]["occupancy"] == waves, f"{n}: {usage[n]['occupancy']} waves/SIMD"
