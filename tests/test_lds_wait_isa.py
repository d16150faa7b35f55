"""CPU: in the split-KV kernel, no LDS read's destination is touched before it lands.

The tile loop issues its LDS reads (K fragments, transposed V fragments) from
inline assembly and waits for them with explicit lgkmcnt waits computed from
its static slot schedule. The compiler treats an asm output as written when
the asm statement ends, so nothing in the language stops it from copying or
reusing such a register before the data has arrived. This test compiles the
kernel for gfx950 to assembly and runs a small dataflow analysis over each
instance's control-flow graph: at every instruction, the set of LDS reads
that may still be in flight (with how many LDS operations were issued after
each); an instruction that reads or writes a register of an in-flight LDS read
is an error.

An lgkmcnt(N) wait covers an LDS read once at least N LDS operations were
issued after it (LDS operations return in order). Scalar memory loads also
count in lgkmcnt but return out of order, so while one may be in flight only
lgkmcnt(0) counts as covering anything.
"""

import os
import re
import shutil
import subprocess

import pytest

from speculative_decoding_verification_hybrid_amd import _build

KERNEL = re.compile(r"^(_ZN3hta4mfma12_GLOBAL__N_118prefix_mfma_kernelILi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)E\S*):", re.M)
DS = re.compile(r"^\s*ds_(\w+)")
SMEM = re.compile(r"^\s*(s_load|s_buffer_load|s_dcache|s_scratch|s_atc|s_memtime|s_memrealtime)")
FLAT = re.compile(r"^\s*flat_")
WAIT = re.compile(r"^\s*s_waitcnt\b(.*)$")
LABEL = re.compile(r"^(\.LBB\w+|\w+):")
BRANCH = re.compile(r"^\s*(s_branch|s_cbranch_\w+)\s+(\S+)")


def _regs(text):
    used = set()
    for kind, a, b in re.findall(r"\b([va])\[(\d+):(\d+)\]", text):
        used.update((kind, r) for r in range(int(a), int(b) + 1))
    for kind, r in re.findall(r"\b([va])(\d+)\b", text):
        used.add((kind, int(r)))
    return used


def _lgkm_of(wait_args):
    m = re.search(r"lgkmcnt\((\d+)\)", wait_args)
    return int(m.group(1)) if m else None


def blocks_of(lines):
    """Splits instruction lines into basic blocks: (label, lines, successors)."""
    blocks, cur, label = [], [], "<entry>"
    for l in lines:
        m = LABEL.match(l)
        if m:
            blocks.append([label, cur])
            cur, label = [], m.group(1)
            continue
        cur.append(l)
        if BRANCH.match(l) or re.match(r"^\s*s_endpgm", l):
            blocks.append([label, cur])
            cur, label = [], None
    blocks.append([label, cur])
    blocks = [b for b in blocks if b[1] or b[0] is not None]
    index = {b[0]: i for i, b in enumerate(blocks) if b[0] is not None}
    succ = []
    for i, (_, body) in enumerate(blocks):
        last = body[-1] if body else ""
        s = []
        m = BRANCH.match(last)
        if m:
            if m.group(2) in index:
                s.append(index[m.group(2)])
            if m.group(1) != "s_branch" and i + 1 < len(blocks):
                s.append(i + 1)
        elif not re.match(r"^\s*s_endpgm", last) and i + 1 < len(blocks):
            s.append(i + 1)
        succ.append(s)
    return blocks, succ


def check_kernel(lines):
    """Returns (number of LDS reads, offending lines) for one kernel's instruction lines."""
    blocks, succ = blocks_of(lines)
    # state: frozenset of (read id, regs, ops issued after) plus an "smem in flight" flag
    entry = [None] * len(blocks)
    entry[0] = (frozenset(), False)
    reads = set()
    bad = set()
    work = [0]
    while work:
        b = work.pop()
        pend = {rid: (regs, n) for rid, regs, n in entry[b][0]}
        smem = entry[b][1]
        for li, l in enumerate(blocks[b][1]):
            w = WAIT.match(l)
            if w:
                n = _lgkm_of(w.group(1))
                if n is not None:
                    if n == 0:
                        pend, smem = {}, False
                    elif not smem:
                        pend = {rid: v for rid, v in pend.items() if v[1] < n}
                continue
            regs = _regs(l)
            touched = [rid for rid, (rr, _) in pend.items() if rr & regs]
            if touched:
                bad.add(l.strip())
            d = DS.match(l)
            is_lgkm = bool(d) or bool(SMEM.match(l)) or bool(FLAT.match(l))
            if is_lgkm:
                pend = {rid: (rr, k + 1) for rid, (rr, k) in pend.items()}
            if SMEM.match(l) or FLAT.match(l):
                smem = True
            if d and (d.group(1).startswith("read") or d.group(1) in ("bpermute_b32", "permute_b32", "swizzle_b32")):
                dst = l.split(None, 1)[1].split(",")[0]
                rid = (b, li)
                reads.add(rid)
                pend[rid] = (frozenset(_regs(dst)), 0)
        out = (frozenset((rid, rr, n) for rid, (rr, n) in pend.items()), smem)
        for s in succ[b]:
            if entry[s] is None:
                new = out
            else:
                # join: every read in flight on either path, with the fewer issued-after count
                merged = {}
                for rid, rr, n in list(entry[s][0]) + list(out[0]):
                    merged[rid] = (rr, min(n, merged[rid][1]) if rid in merged else n)
                new = (frozenset((rid, rr, n) for rid, (rr, n) in merged.items()), entry[s][1] or out[1])
            if new != entry[s]:
                entry[s] = new
                work.append(s)
    return len(reads), sorted(bad)


def _kernels(src):
    out_dir = os.environ.get("TMPDIR", "/tmp")
    out = os.path.join(out_dir, f"lds_wait_{os.getpid()}_{src}.s")
    cmd = [_build.hipcc()] + _build.flags_for(src) + ["--cuda-device-only", "-S", os.path.join(_build.CSRC, src),
                                                      "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    s = open(out).read()
    os.remove(out)
    for m in KERNEL.finditer(s):
        end = s.index("s_endpgm", m.end()) + len("s_endpgm")
        lines = [l for l in s[m.end():end].split("\n")
                 if l.strip() and not l.strip().startswith(";") and not l.strip().startswith(".")
                 or LABEL.match(l)]
        yield m, lines


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not available")
def test_lds_reads_untouched_until_waited():
    n_inst = 0
    for m, lines in _kernels("prefix_mfma.hip"):
        n, bad = check_kernel(lines)
        n_inst += 1
        assert n > 0 and not bad, f"D={m.group(2)} QB={m.group(3)} waves={m.group(4)}: {bad[:4]}"
    assert n_inst == 13


def test_checker_catches_early_use():
    """The checker itself: a use before the covering wait fails, across a loop back-edge too."""
    body = [
        "ds_read_b128 v[4:7], v1",
        "ds_read_b128 v[8:11], v2",
        "s_waitcnt lgkmcnt(2)",  # covers nothing (only one LDS op issued after the first read)
        "v_mov_b32 v20, v5",
        "s_waitcnt lgkmcnt(0)",
        "s_endpgm",
    ]
    n, bad = check_kernel(body)
    assert n == 2 and bad == ["v_mov_b32 v20, v5"]
    ok = body[:2] + ["s_waitcnt lgkmcnt(1)", "v_mov_b32 v20, v5", "s_endpgm"]
    assert check_kernel(ok) == (2, [])
    # a scalar load in flight makes lgkmcnt(1) cover nothing
    smem = ["ds_read_b128 v[4:7], v1", "s_load_dword s4, s[0:1], 0x0", "ds_read_b128 v[8:11], v2",
            "s_waitcnt lgkmcnt(1)", "v_mov_b32 v20, v5", "s_endpgm"]
    assert check_kernel(smem)[1] == ["v_mov_b32 v20, v5"]
    # read at the end of a loop body, used at the top of the next iteration without a wait
    loop = [".LBB0_1:", "v_mov_b32 v20, v5", "ds_read_b128 v[4:7], v1", "s_cbranch_scc1 .LBB0_1",
            "s_waitcnt lgkmcnt(0)", "s_endpgm"]
    # (the read itself, issued again while the previous iteration's is in flight, is flagged too)
    assert check_kernel(loop)[1] == ["ds_read_b128 v[4:7], v1", "v_mov_b32 v20, v5"]
    loop_ok = [".LBB0_1:", "s_waitcnt lgkmcnt(0)", "v_mov_b32 v20, v5", "ds_read_b128 v[4:7], v1",
               "s_cbranch_scc1 .LBB0_1", "s_waitcnt lgkmcnt(0)", "s_endpgm"]
    assert check_kernel(loop_ok)[1] == []


# ----------------------------------------------------------------------------
# MFMA result hazards of the inline-assembly MFMAs
# ----------------------------------------------------------------------------
#
# The P.V MFMAs are issued from inline assembly (their accumulators pinned to
# AGPRs), so the compiler does not insert the wait states their results need.
# This check walks the same control-flow graph and, for every MFMA that came
# from inline assembly, counts wait states (one per instruction, N+1 per
# s_nop N) until anything other than an MFMA accumulating into exactly the
# same registers reads or writes its destination: at least MFMA_RESULT_WAIT
# must have passed (more than an 8- or 16-pass XDL result needs on gfx950).
# Before such an MFMA, no VALU instruction may have written one of its source
# registers within VALU_TO_MFMA_WAIT wait states.

MFMA_RESULT_WAIT = 19
VALU_TO_MFMA_WAIT = 4
MFMA = re.compile(r"^\s*v_mfma\w*\s+(\S+),\s*(\S+),\s*(\S+),\s*(\S+)")


def _wait_states(line):
    m = re.match(r"^\s*s_nop\s+(\d+)", line)
    return int(m.group(1)) + 1 if m else 1


def _tagged_lines(lines):
    """(line, from_inline_asm) for every instruction or label line."""
    out, in_asm = [], False
    for l in lines:
        if ";;#ASMSTART" in l:
            in_asm = True
            continue
        if ";;#ASMEND" in l:
            in_asm = False
            continue
        if l.strip().startswith(";") or (l.strip().startswith(".") and not LABEL.match(l)):
            continue
        out.append((l, in_asm))
    return out


def check_mfma_hazards(tagged):
    blocks, succ = blocks_of([l for l, _ in tagged])
    # asm flags per block line, in the same order blocks_of split them
    flags = iter([f for l, f in tagged if not LABEL.match(l)])
    bflags = [[next(flags) for _ in body] for _, body in blocks]
    entry = [None] * len(blocks)
    entry[0] = (frozenset(), frozenset())  # (pending asm MFMA results, recent VALU writes)
    bad, n_asm = set(), set()
    work = [0]
    while work:
        b = work.pop()
        pend = dict((k, (regs, w)) for k, regs, w in entry[b][0])
        recent = dict((k, (regs, w)) for k, regs, w in entry[b][1])
        for li, (l, asm) in enumerate(zip(blocks[b][1], bflags[b])):
            ws = _wait_states(l)
            m = MFMA.match(l)
            regs = _regs(l)
            if m:
                dst, srcs = _regs(m.group(1)), _regs(",".join(m.group(i) for i in (2, 3, 4)))
                for k, (rr, w) in list(pend.items()):
                    if rr & regs and not (rr == dst and rr & _regs(m.group(4)) == rr):
                        bad.add(l.strip())
                if asm:
                    n_asm.add((b, li))
                    for k, (rr, w) in recent.items():
                        if rr & srcs:
                            bad.add(l.strip())
            else:
                for k, (rr, w) in pend.items():
                    if rr & regs:
                        bad.add(l.strip())
            # advance time, then record this instruction's effects
            pend = {k: (rr, w - ws) for k, (rr, w) in pend.items() if w - ws > 0}
            recent = {k: (rr, w - ws) for k, (rr, w) in recent.items() if w - ws > 0}
            if m and asm:
                pend[(b, li)] = (frozenset(dst), MFMA_RESULT_WAIT)
            elif re.match(r"^\s*v_", l) and not m:
                first = l.split(None, 1)[1].split(",")[0] if len(l.split(None, 1)) > 1 else ""
                recent[(b, li)] = (frozenset(_regs(first)), VALU_TO_MFMA_WAIT)
        out = (frozenset((k, rr, w) for k, (rr, w) in pend.items()),
               frozenset((k, rr, w) for k, (rr, w) in recent.items()))
        for s in succ[b]:
            if entry[s] is None:
                new = out
            else:
                merged = []
                for part in (0, 1):
                    d = {}
                    for k, rr, w in list(entry[s][part]) + list(out[part]):
                        d[k] = (rr, max(w, d[k][1]) if k in d else w)
                    merged.append(frozenset((k, rr, w) for k, (rr, w) in d.items()))
                new = tuple(merged)
            if new != entry[s]:
                entry[s] = new
                work.append(s)
    return len(n_asm), sorted(bad)


def _kernels_tagged(src):
    out = os.path.join(os.environ.get("TMPDIR", "/tmp"), f"mfma_hz_{os.getpid()}_{src}.s")
    cmd = [_build.hipcc()] + _build.flags_for(src) + ["--cuda-device-only", "-S", os.path.join(_build.CSRC, src),
                                                      "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    s = open(out).read()
    os.remove(out)
    for m in KERNEL.finditer(s):
        end = s.index("s_endpgm", m.end()) + len("s_endpgm")
        yield m, _tagged_lines(s[m.end():end].split("\n"))


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not available")
def test_asm_mfma_results_not_touched_early():
    n_inst = 0
    for m, tagged in _kernels_tagged("prefix_mfma.hip"):
        n, bad = check_mfma_hazards(tagged)
        n_inst += 1
        # eight waves keep the P.V accumulators in VGPRs with compiler-visible MFMAs
        vgpr_form = int(m.group(4)) == 8
        assert (n == 0 if vgpr_form else n > 0) and not bad, f"D={m.group(2)} QB={m.group(3)} waves={m.group(4)}: {bad[:4]}"
    assert n_inst == 13


def test_mfma_hazard_checker_catches_early_reads():
    asm = [(";;#ASMSTART", False)]
    body = [("v_mfma_f32_32x32x16_bf16 a[0:15], v[4:7], v[8:11], a[0:15]", True),
            ("v_accvgpr_read_b32 v20, a3", False), ("s_endpgm", False)]
    assert check_mfma_hazards(body)[1] == ["v_accvgpr_read_b32 v20, a3"]
    ok = body[:1] + [("s_nop 7", False), ("s_nop 7", False), ("s_nop 3", False)] + body[1:]
    assert check_mfma_hazards(ok) == (1, [])
    # an accumulation into exactly the same registers is allowed right after
    chain = body[:1] + [("v_mfma_f32_32x32x16_bf16 a[0:15], v[12:15], v[8:11], a[0:15]", True), ("s_endpgm", False)]
    assert check_mfma_hazards(chain)[1] == []
    # a VALU write of a source right before the MFMA is not
    raw = [("v_mov_b32 v9, 0", False)] + body[:1] + [("s_endpgm", False)]
    assert check_mfma_hazards(raw)[1] == ["v_mfma_f32_32x32x16_bf16 a[0:15], v[4:7], v[8:11], a[0:15]"]
    assert asm  # (tagging itself is exercised on the real kernels)
