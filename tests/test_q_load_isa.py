"""CPU: the split-KV kernel's asynchronous Q loads are not read before they land.

The kernel issues its Q fragment loads as inline-asm global loads ahead of the
first KV tile copies and only waits for them with the explicit vmcnt wait that
also covers the first tile. The compiler sees the asm outputs as written when
the asm statement ends, so nothing in the language stops it from copying or
reusing those registers before the data has arrived. This test compiles the
kernel for gfx950 to assembly and checks, for every template instance, that no
instruction between a Q load and the first wait that provably covers it reads
or writes that load's destination registers.

A vector-memory wait ``vmcnt(N)`` covers a load once at least N vector-memory
operations were issued after it (gfx9 returns them in order).
"""

import os
import re
import shutil
import subprocess

import pytest

from speculative_decoding_verification_hybrid_amd import _build

VMEM = re.compile(r"^\s*(global_|buffer_|flat_|scratch_)(load|store|atomic)")
# the prologue's inline-asm loads: Q fragments (dwordx4) and the parent word (dword), addressed by a VGPR pair
LOAD = re.compile(r"^\s*global_load_dword(?:x4)? (v\[\d+:\d+\]|v\d+), v\[\d+:\d+\], off")
KERNEL = re.compile(r"^(_ZN3hta4mfma12_GLOBAL__N_118prefix_mfma_kernelILi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)E\S*):", re.M)


def _regs(line):
    used = set()
    for a, b in re.findall(r"\bv\[(\d+):(\d+)\]", line):
        used.update(range(int(a), int(b) + 1))
    used.update(int(r) for r in re.findall(r"\bv(\d+)\b", line))
    return used


def check_kernel(body):
    """Returns (number of Q loads, offending lines) for one kernel's instruction lines."""
    loads = [i for i, l in enumerate(body) if LOAD.match(l)]
    if not loads:
        return 0, ["no Q loads found"]
    pending = {}  # register -> index of the load that writes it
    issued_after = {}  # load index -> vector-memory ops issued after it
    bad = []
    for i in range(loads[0], len(body)):
        l = body[i]
        m = re.match(r"^\s*s_waitcnt\b.*vmcnt\((\d+)\)", l)
        if m:
            n = int(m.group(1))
            done = {j for j, k in issued_after.items() if k >= n}
            pending = {r: j for r, j in pending.items() if j not in done}
            for j in done:
                del issued_after[j]
            if not issued_after:
                break
            continue
        if i in loads:
            d = LOAD.match(l)
            if _regs(l) & set(pending):
                bad.append(l.strip())
            for j in issued_after:
                issued_after[j] += 1
            issued_after[i] = 0
            for r in _regs(d.group(1)):
                pending[r] = i
            continue
        if _regs(l) & set(pending):
            bad.append(l.strip())
        if VMEM.match(l):
            for j in issued_after:
                issued_after[j] += 1
    else:
        bad.append("no covering vmcnt wait before the end of the kernel")
    return len(loads), bad


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not available")
@pytest.mark.parametrize("src,instances", [("prefix_mfma.hip", 13)])
def test_q_fragment_loads_untouched_until_waited(tmp_path, src, instances):
    out = tmp_path / (src + ".s")
    cmd = [_build.hipcc()] + _build.flags_for(src) + ["--cuda-device-only", "-S", os.path.join(_build.CSRC, src),
                                                      "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    s = out.read_text()
    kernels = list(KERNEL.finditer(s))
    assert len(kernels) == instances  # every (D, QB, waves, stages) instance
    for m in kernels:
        end = s.index("s_endpgm", m.end())
        body = [l for l in s[m.end():end].split("\n") if l.strip() and not l.strip().startswith(";")
                and not l.strip().startswith(".")]
        n, bad = check_kernel(body)
        assert n > 0 and not bad, f"D={m.group(2)} QB={m.group(3)} waves={m.group(4)}: {bad[:3]}"


def test_checker_catches_early_use():
    """The checker itself: a read of a pending register before the covering wait fails."""
    body = [
        "global_load_dwordx4 v[4:7], v[0:1], off",
        "global_load_lds_dwordx4 v2, s[0:1]",
        "global_load_lds_dwordx4 v3, s[0:1]",
        "s_waitcnt vmcnt(3)",  # does not cover the Q load (only 2 issued after it)
        "v_mov_b32 v8, v5",
        "s_waitcnt vmcnt(1)",
    ]
    n, bad = check_kernel(body)
    assert n == 1 and bad == ["v_mov_b32 v8, v5"]
    body_ok = body[:3] + ["s_waitcnt vmcnt(2)", "v_mov_b32 v8, v5"]
    assert check_kernel(body_ok) == (1, [])
