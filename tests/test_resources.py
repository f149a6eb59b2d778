"""Register and scratch gate (CPU: the compiler's own resource report, no GPU).

LDS or register overflow spills silently to scratch memory (CK/MI50 notes section 4.3,
first pitfall).  Every kernel of the library is compiled here with the resource report
and must keep zero scratch and zero spilled registers, except the fp32 accuracy-path
kernels listed below, whose spills are known and may not grow, and the persistent forward
kernels, which may keep scalar registers in vector-register lanes (no memory) as long as
no such spill or restore sits in their steady-state loop.  The fast paths' waves per SIMD
are pinned too: losing one is a silent slowdown."""
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
# the persistent forward kernels (d = 128 and 256): scalar spills into vector-register
# lanes, at most
PERSISTENT_128 = r"fa_fwd16_kernelILi128ELb[01]ELi8ELi1ELb0ELb1E"
PERSISTENT_256 = r"fa_fwd16_kernelILi256ELb[01]ELi4ELi1ELb0ELb1E"
PERSISTENT = f"({PERSISTENT_128}|{PERSISTENT_256})"
PERSISTENT_SGPR_SPILLS = 96
# (kernel name pattern, waves per SIMD) of the production 16-bit forward kernels
OCCUPANCY = [
    (r"fa_fwd16_kernelILi128ELb[01]ELi8ELi1ELb0ELb0E", 2),
    (PERSISTENT_128, 2),
    (PERSISTENT_256, 1),
    (r"fa_fwd16_kernelILi64ELb[01]ELi4ELi2ELb0ELb0E", 2),
    (r"fa_fwd16_kernelILi256ELb[01]ELi4ELi1ELb0ELb0E", 1),
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
        if re.search(PERSISTENT, name):
            assert rec["scratch"] == 0 and rec["vgpr_spill"] == 0, f"{name} spills: {rec}"
            assert rec.get("sgpr_spill", 0) <= PERSISTENT_SGPR_SPILLS, f"{name}: {rec}"
        elif limit is None:
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


@pytest.mark.parametrize("unit,pattern,mfma", [("fa_fwd16_d128.hip", PERSISTENT_128, 32),
                                               ("fa_fwd16.hip", PERSISTENT_256, 64)])
def test_persistent_kernels_spill_nothing_in_their_steady_loop(unit, pattern, mfma):
    # the innermost loop of each persistent kernel (the steady-state key-tile loop, mfma
    # products per tile) holds no spill or restore of a scalar register (v_writelane /
    # v_readlane)
    with tempfile.TemporaryDirectory() as d:
        asm = build.device_assembly(unit, f"{d}/out.s")
    lines = asm.split("\n")
    starts = [i for i, l in enumerate(lines) if re.match(r"^(_Z\w+):", l) and re.search(pattern, l)]
    assert len(starts) == 2, starts
    for st in starts:
        end = next(j for j in range(st, len(lines)) if "s_endpgm" in lines[j])
        body = lines[st:end]
        hdr = next(i for i, l in enumerate(body) if "Inner Loop Header" in l)
        lab = hdr
        while not body[lab].startswith(".LBB"):
            lab -= 1
        label = body[lab].split(":")[0]
        back = max(i for i, l in enumerate(body)
                   if ("s_cbranch" in l or "s_branch" in l) and l.split(";")[0].strip().endswith(label))
        loop = [l.split(";")[0].strip() for l in body[lab:back + 1]]
        assert sum("v_mfma" in l for l in loop) == mfma, "not the key-tile loop"
        assert not [l for l in loop if l.startswith(("v_readlane", "v_writelane"))], body[0]
