"""The compiled gfx950 code of every GEMM kernel leaves at least 4
instructions (an s_nop N counts N + 1) between an MFMA and any VALU
instruction that writes one of the MFMA's A or B source registers, and at
least 2 between a VALU write of such a register and the MFMA that reads it.

A VALU write right behind an MFMA into its source registers corrupted the
MFMA's operand (the 16x16x32 f16 form, in an earlier decode kernel), and the
compiler inserts no wait states for that pattern, so the kernels keep
operands live on purpose (keep_live, mfma_drain in nvfp4_gemm.hip).  This
test checks the GEMM source's gfx950 assembly (the gemm_kernels_asm fixture), so that a
change of code or compiler that brings such a write closer fails here, on
the CPU.  Needs hipcc (skipped without it).

The second check covers the other order.  For MFMAs written through the
compiler builtin the compiler inserts the wait states itself (2 on gfx950,
the count the builtin kernels here show); the streaming kernels issue their
MFMAs as inline asm, which the compiler's hazard model does not see into,
so a dequantization step scheduled right in front of the MFMA that reads
its result gave wrong sums in one accumulator block (seen when a loop exit
test let the compiler sink a stage's last multiplies into the next stage)."""
import re

MIN_DISTANCE = 4
MIN_WRITE_TO_READ = 2

_REG = re.compile(r"\b([va])(\d+)\b|\b([va])\[(\d+):(\d+)\]")


def _regs(text):
    out = set()
    for m in _REG.finditer(text):
        if m.group(1):
            out.add((m.group(1), int(m.group(2))))
        else:
            out.update((m.group(3), r) for r in range(int(m.group(4)), int(m.group(5)) + 1))
    return out


def _closest_source_writes(insts):
    """For every MFMA: the distance to the first later VALU writing its A/B
    registers, if within MIN_DISTANCE - 1 wait states."""
    bad = []
    for i, s in enumerate(insts):
        if not s.startswith("v_mfma"):
            continue
        ops = [o.strip() for o in s.split(None, 1)[1].split(",")]
        src = _regs(ops[1]) | _regs(ops[2])
        dist = 0
        for t in insts[i + 1:]:
            op = t.split()[0]
            if op == "s_nop":
                dist += int(t.split()[1], 0) + 1
            else:
                dist += 1
            if dist >= MIN_DISTANCE:
                break
            if op.startswith("v_") and not op.startswith("v_mfma") and " " in t:
                if _regs(t.split(None, 1)[1].split(",")[0]) & src:
                    bad.append((dist, s, t))
                    break
    return bad


def _closest_source_writes_before(insts):
    """For every MFMA: the distance back to the last VALU writing its A/B
    registers, if within MIN_WRITE_TO_READ - 1 wait states."""
    bad = []
    for i, s in enumerate(insts):
        if not s.startswith("v_mfma"):
            continue
        ops = [o.strip() for o in s.split(None, 1)[1].split(",")]
        src = _regs(ops[1]) | _regs(ops[2])
        dist = 0
        for t in reversed(insts[max(0, i - 16):i]):
            op = t.split()[0]
            if op.startswith("v_") and not op.startswith("v_mfma") and " " in t:
                if _regs(t.split(None, 1)[1].split(",")[0]) & src:
                    bad.append((dist, s, t))
                    break
            dist += int(t.split()[1], 0) + 1 if op == "s_nop" else 1
            if dist >= MIN_WRITE_TO_READ:
                break
    return bad


def test_no_valu_write_into_mfma_sources_right_before_the_mfma(gemm_kernels_asm):
    report = []
    for name, ins in gemm_kernels_asm.items():
        for d, mfma, valu in _closest_source_writes_before(ins):
            report.append(f"{name[:80]}: `{valu}` {d} before `{mfma}`")
    assert not report, (f"{len(report)} VALU writes into MFMA sources within {MIN_WRITE_TO_READ} before the "
                        "MFMA:\n" + "\n".join(report[:10]))


def test_no_valu_write_into_mfma_sources_right_behind_the_mfma(gemm_kernels_asm):
    kernels = gemm_kernels_asm
    n_mfma = sum(1 for ins in kernels.values() for s in ins if s.startswith("v_mfma"))
    assert n_mfma > 1000, "no MFMA code found: the listing format changed"
    report = []
    for name, ins in kernels.items():
        for d, mfma, valu in _closest_source_writes(ins):
            report.append(f"{name[:80]}: {d} after `{mfma}`: `{valu}`")
    assert not report, f"{len(report)} VALU writes into MFMA sources within {MIN_DISTANCE}:\n" + "\n".join(report[:10])
