"""Hazard gate for the instructions written as inline assembly (CPU: the compiler's gfx950
assembly, no GPU).

The compiler inserts the wait states its own instructions need, but it does not look inside
inline assembly: neither the latency of the matrix-core products written there nor the
scalar registers the loads into LDS written there read.  In every kernel of every unit,
along every control-flow path (fall-through and branches, backwards from each instruction):
  * a vector instruction that reads an AGPR written by a matrix-core product must come at
    least 19 wait states later (the longest, 16-pass, product's latency plus margin);
  * a matrix-core product that reads, as its A or B operand, a VGPR last written by a
    (non-matrix-core) vector instruction must come at least 2 wait states after it;
  * a vector-memory instruction that reads a scalar register (buffer resource, offset, m0)
    must come at least 5 wait states after a vector instruction that writes it (a scalar
    restored from a spill with v_readlane, a v_readfirstlane, a compare into a mask).
`s_nop k` counts k + 1 wait states and every other instruction one.  The rules apply to
the instructions written as assembly; the compiler keeps its own instructions' wait states
with their exact latencies.  The test also plants each mistake in a copy of a unit and
checks that the scan sees it."""
import os
import re
import shutil
import tempfile

import pytest

from exact_attention_90_amd import build

UNITS = ["fa_fwd16.hip", "fa_fwd16_d128.hip", "fa_bwd_d128.hip", "fa_bwd_d256.hip",
         "fa_fused.hip", "fa_bwd.hip", "fa_bwd32.hip", "fa_naive.hip"]
AGPR_READ_WAIT = 19
VALU_TO_MFMA_WAIT = 2
VALU_SGPR_TO_VMEM_WAIT = 5
VMEM_PREFIX = ("buffer_", "global_", "flat_")
# vector instructions with a scalar second destination (carry out or the like)
SDST2 = ("v_add_co_", "v_sub_co_", "v_subrev_co_", "v_addc_co_", "v_subb_co_", "v_subbrev_co_",
         "v_div_scale_", "v_mad_u64_u32", "v_mad_i64_i32")


def _sregs(tok):
    """Scalar registers a token names (sN, s[a:b], m0, vcc, vcc_lo, vcc_hi)."""
    if tok in ("m0", "vcc_lo", "vcc_hi"):
        return {tok}
    if tok == "vcc":
        return {"vcc_lo", "vcc_hi"}
    return _regs(tok, "s")


def _valu_sdst(op, args):
    """Scalar registers a vector instruction writes."""
    if not op.startswith("v_") or op.startswith("v_mfma") or not args or not args[0]:
        return set()
    out = _sregs(args[0])
    if op.startswith(SDST2) and len(args) > 1:
        out |= _sregs(args[1])
    if op.startswith("v_cmp") and op.endswith("_e32"):
        out |= {"vcc_lo", "vcc_hi"}
    return out


def _regs(tok, kind):
    m = re.match(kind + r"\[(\d+):(\d+)\]$", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(kind + r"(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def _kernels(asm):
    """(name, instructions, label -> index of its first instruction, indices of the
    instructions written as inline assembly) per kernel."""
    lines = asm.split("\n")
    for i, line in enumerate(lines):
        m = re.match(r"^(_Z\w+):", line)
        if not m:
            continue
        end = next(j for j in range(i, len(lines)) if "s_endpgm" in lines[j])
        insts, labels, in_asm, asm_idx = [], {}, False, set()
        for raw in lines[i + 1:end + 1]:
            if ";;#ASMSTART" in raw:
                in_asm = True
            elif ";;#ASMEND" in raw:
                in_asm = False
            t = raw.split(";")[0].strip()
            lm = re.match(r"^(\.L\w+):", t)
            if lm:
                labels[lm.group(1)] = len(insts)
                continue
            if not t or t.startswith("."):
                continue
            op = t.split()[0]
            if in_asm:
                asm_idx.add(len(insts))
            insts.append((op, [a.strip() for a in t[len(op):].split(",")], t))
        yield m.group(1), insts, labels, asm_idx


def _preds(insts, labels):
    """Predecessor instruction indices of each instruction index."""
    preds = [[] for _ in insts]
    for n, (op, args, _) in enumerate(insts):
        if n + 1 < len(insts) and op not in ("s_branch", "s_endpgm", "s_setpc_b64"):
            preds[n + 1].append(n)
        if op.startswith("s_cbranch") or op == "s_branch":
            tgt = labels.get(args[0])
            if tgt is not None and tgt < len(insts):
                preds[tgt].append(n)
    return preds


def _cost(op, args):
    return int(args[0]) + 1 if op == "s_nop" else 1


def _search(insts, preds, start, hit, stop, limit):
    """Walk backwards from the instruction before `start` along every path; return the
    (wait states, index) of the first instruction n where hit(n) holds with fewer than
    `limit` wait states, else None.  stop(n) ends a path without a hit."""
    seen = {}
    work = [(p, 0) for p in preds[start]]
    while work:
        n, ws = work.pop()
        if ws >= limit or seen.get(n, limit + 1) <= ws:
            continue
        seen[n] = ws
        op, args, _ = insts[n]
        if hit(n):
            return ws, n
        if stop(n):
            continue
        work.extend((p, ws + _cost(op, args)) for p in preds[n])
    return None


def _check(name, insts, labels, asm_idx):
    """The three rules for the instructions written as assembly (the compiler keeps its own
    instructions' wait states, with exact per-instruction latencies)."""
    preds = _preds(insts, labels)
    bad = []
    for n, (op, args, text) in enumerate(insts):
        if op.startswith("v_") and not op.startswith("v_mfma"):
            reads = set()
            for a in args[1:]:
                reads |= _regs(a, "a")
            if reads:
                r = _search(insts, preds, n,
                            lambda k, rd=reads: k in asm_idx and insts[k][0].startswith("v_mfma")
                            and bool(_regs(insts[k][1][0], "a") & rd),
                            lambda k: False, AGPR_READ_WAIT)
                if r:
                    bad.append(f"{name}: '{text}' {r[0]} wait states after '{insts[r[1]][2]}'")
        if op.startswith("v_mfma") and n in asm_idx:
            for reg in _regs(args[1], "v") | _regs(args[2], "v"):
                def writes(k, reg=reg):
                    o, a, _ = insts[k]
                    return bool(a) and reg in _regs(a[0], "v") and not o.startswith(
                        ("s_", "ds_write", "buffer_store", "global_store"))
                r = _search(insts, preds, n,
                            lambda k, w=writes: w(k) and insts[k][0].startswith("v_")
                            and not insts[k][0].startswith("v_mfma"),
                            writes, VALU_TO_MFMA_WAIT)
                if r:
                    bad.append(f"{name}: '{text}' reads v{reg} {r[0]} wait states after "
                               f"'{insts[r[1]][2]}'")
        if op.startswith(VMEM_PREFIX) and n in asm_idx:
            sreads = set()
            for a in args:
                if a:
                    sreads |= _sregs(a.split()[0])
            if " lds" in text:  # the LDS address comes from m0
                sreads.add("m0")
            r = _search(insts, preds, n,
                        lambda k, rd=sreads: bool(_valu_sdst(insts[k][0], insts[k][1]) & rd),
                        lambda k: False, VALU_SGPR_TO_VMEM_WAIT)
            if r:
                bad.append(f"{name}: '{text}' reads a scalar {r[0]} wait states after "
                           f"'{insts[r[1]][2]}'")
    return bad


def _scan(asm):
    kernels = list(_kernels(asm))
    assert kernels
    return kernels, [b for name, ins, lab, ai in kernels for b in _check(name[:60], ins, lab, ai)]


@pytest.mark.parametrize("unit", UNITS)
def test_assembly_products_keep_their_wait_states(unit):
    with tempfile.TemporaryDirectory() as d:
        asm = build.device_assembly(unit, f"{d}/out.s")
    kernels, bad = _scan(asm)
    assert kernels
    assert not bad, "\n".join(bad[:10])


def test_the_scan_sees_planted_mistakes():
    # the d = 256 backward unit without the waits for its dQ products (in the loop and
    # before the epilogue), and without the two wait states before the first dQ product of
    # a key step
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "csrc")
        shutil.copytree(build.CSRC, src)
        path = os.path.join(src, "fa_bwd.hpp")
        text = open(path).read()
        drain = "    // the assembly products' results: wait for the last, then fresh definitions\n    mfma_drain();"
        loop_drain = "    if constexpr (D == 256) mfma_drain();\n"
        nop = 'asm volatile("s_nop 1\\n\\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"'
        assert text.count(drain) == 1 and text.count(loop_drain) == 1 and text.count(nop) == 1
        for mutant, expect in [(text.replace(drain, "").replace(loop_drain, ""), "wait states after 'v_mfma"),
                               (text.replace(nop, 'asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"'),
                                "reads v")]:
            open(path, "w").write(mutant)
            old = build.CSRC
            build.CSRC = src
            try:
                asm = build.device_assembly("fa_bwd_d256.hip", os.path.join(d, "m.s"))
            finally:
                build.CSRC = old
            _, bad = _scan(asm)
            assert any(expect in b for b in bad), f"planted mistake not seen ({expect})"


def test_the_scan_sees_a_scalar_written_just_before_a_load_into_lds():
    # the offset of every load into LDS of the plain form (the backward kernels' form)
    # taken from a v_readfirstlane just before the load, with that form's one wait state
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "csrc")
        shutil.copytree(build.CSRC, src)
        path = os.path.join(src, "fa_device.hpp")
        text = open(path).read()
        plain = ('    asm volatile("s_nop 0\\n\\tbuffer_load_dwordx4 %0, %1, %2 offen lds"\n'
                 '                 :\n'
                 '                 : "v"(voff), "s"(r), "s"(soff), "{m0}"(m0v)')
        assert text.count(plain) == 1
        open(path, "w").write(plain.join(text.split(plain)).replace(
            plain, plain.replace('"s"(soff)', '"s"(__builtin_amdgcn_readfirstlane(voff + soff))')))
        old = build.CSRC
        build.CSRC = src
        try:
            asm = build.device_assembly("fa_bwd_d128.hip", os.path.join(d, "m.s"))
        finally:
            build.CSRC = old
        _, bad = _scan(asm)
        assert any("reads a scalar" in b and "v_readfirstlane" in b for b in bad)
