"""Hazard gate for the matrix-core products written as inline assembly (CPU: the compiler's
gfx950 assembly, no GPU).

The compiler inserts the wait states its own matrix-core products need, but it does not see
the latency of products written as assembly.  In every kernel of the units that contain
such products, along every control-flow path (fall-through and branches, backwards from
each instruction):
  * a vector instruction that reads an AGPR written by a matrix-core product must come at
    least 19 wait states later (the longest, 16-pass, product's latency plus margin);
  * a matrix-core product that reads, as its A or B operand, a VGPR last written by a
    (non-matrix-core) vector instruction must come at least 2 wait states after it.
`s_nop k` counts k + 1 wait states and every other instruction one.  The kernels that use
only the compiler's products satisfy both by construction; the scan covers them too.  The
test also plants both mistakes in a copy of one unit and checks that the scan sees them."""
import os
import re
import shutil
import tempfile

import pytest

from exact_attention_90_amd import build

UNITS = ["fa_fwd16.hip", "fa_fwd16_d128.hip", "fa_bwd_d128.hip", "fa_bwd_d256.hip"]
AGPR_READ_WAIT = 19
VALU_TO_MFMA_WAIT = 2


def _regs(tok, kind):
    m = re.match(kind + r"\[(\d+):(\d+)\]$", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(kind + r"(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def _kernels(asm):
    """(name, instructions, label -> index of its first instruction) per kernel."""
    lines = asm.split("\n")
    for i, line in enumerate(lines):
        m = re.match(r"^(_Z\w+):", line)
        if not m:
            continue
        end = next(j for j in range(i, len(lines)) if "s_endpgm" in lines[j])
        insts, labels = [], {}
        for raw in lines[i + 1:end + 1]:
            t = raw.split(";")[0].strip()
            lm = re.match(r"^(\.L\w+):", t)
            if lm:
                labels[lm.group(1)] = len(insts)
                continue
            if not t or t.startswith("."):
                continue
            op = t.split()[0]
            insts.append((op, [a.strip() for a in t[len(op):].split(",")], t))
        yield m.group(1), insts, labels


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
    (wait states, index) of the first instruction where hit() holds with fewer than
    `limit` wait states, else None.  stop() ends a path without a hit."""
    seen = {}
    work = [(p, 0) for p in preds[start]]
    while work:
        n, ws = work.pop()
        if ws >= limit or seen.get(n, limit + 1) <= ws:
            continue
        seen[n] = ws
        op, args, _ = insts[n]
        if hit(op, args):
            return ws, n
        if stop(op, args):
            continue
        work.extend((p, ws + _cost(op, args)) for p in preds[n])
    return None


def _check(name, insts, labels):
    preds = _preds(insts, labels)
    bad = []
    for n, (op, args, text) in enumerate(insts):
        if op.startswith("v_") and not op.startswith("v_mfma"):
            reads = set()
            for a in args[1:]:
                reads |= _regs(a, "a")
            if reads:
                r = _search(insts, preds, n,
                            lambda o, a: o.startswith("v_mfma") and bool(_regs(a[0], "a") & reads),
                            lambda o, a: False, AGPR_READ_WAIT)
                if r:
                    bad.append(f"{name}: '{text}' {r[0]} wait states after '{insts[r[1]][2]}'")
        if op.startswith("v_mfma"):
            for reg in _regs(args[1], "v") | _regs(args[2], "v"):
                def writes(o, a, reg=reg):
                    return bool(a) and reg in _regs(a[0], "v") and not o.startswith(
                        ("s_", "ds_write", "buffer_store", "global_store"))
                r = _search(insts, preds, n,
                            lambda o, a, w=writes: w(o, a) and not o.startswith("v_mfma")
                            and o.startswith("v_"),
                            lambda o, a, w=writes: w(o, a), VALU_TO_MFMA_WAIT)
                if r:
                    bad.append(f"{name}: '{text}' reads v{reg} {r[0]} wait states after "
                               f"'{insts[r[1]][2]}'")
    return bad


def _scan(asm):
    kernels = list(_kernels(asm))
    assert kernels
    return kernels, [b for name, ins, lab in kernels for b in _check(name[:60], ins, lab)]


@pytest.mark.parametrize("unit", UNITS)
def test_assembly_products_keep_their_wait_states(unit):
    with tempfile.TemporaryDirectory() as d:
        asm = build.device_assembly(unit, f"{d}/out.s")
    kernels, bad = _scan(asm)
    assert any(";;#ASMSTART" in asm and "v_mfma" in t for _, ins, _ in kernels for _, _, t in ins)
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
