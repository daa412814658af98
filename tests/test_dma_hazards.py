"""The global -> LDS loads are inline asm, which the compiler's hazard checks do
not see.  Compile the kernels that use them to gfx950 assembly and check that
every such load has the wait states gfx950 requires after a VALU write of an
SGPR it reads (five; v_readlane restoring a spilled resource word is the case
that occurs) and after the M0 write that carries its LDS address (one).

CPU only: hipcc cross-compiles for gfx950 without a GPU.
"""
import os
import re
import shutil
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

from nvfp4_bit_block_amd import build as nvbuild

SOURCES = ["gemm_stream.hip", "gemm_a16.hip"]
VALU_SGPR_WAIT = 5
M0_WAIT = 1


def _sgprs(text):
    regs = set()
    for m in re.finditer(r"\bs\[(\d+):(\d+)\]", text):
        regs |= {f"s{i}" for i in range(int(m.group(1)), int(m.group(2)) + 1)}
    regs |= {f"s{m.group(1)}" for m in re.finditer(r"\bs(\d+)\b", text)}
    if re.search(r"\bm0\b", text):
        regs.add("m0")
    return regs


def _instructions(asm):
    out = []
    for line in asm.splitlines():
        line = line.split(";")[0].strip()
        if not line or line.startswith(".") or line.endswith(":"):
            continue
        out.append(line)
    return out


def hazards(asm):
    """(load, writer, wait states) for each LDS-DMA load whose SGPR operands
    were written too few wait states before it on the fall-through path."""
    found = []
    ins = _instructions(asm)
    for i, load in enumerate(ins):
        if not re.match(r"buffer_load_\w+\s.*\blds$", load):
            continue
        reads = _sgprs(load.split(None, 1)[1]) | {"m0"}
        waits = 0
        for prev in reversed(ins[max(0, i - 16):i]):
            if waits >= VALU_SGPR_WAIT:
                break
            m = re.match(r"s_nop\s+(\d+)", prev)
            if m:
                waits += int(m.group(1)) + 1
                continue
            op, _, args = prev.partition(" ")
            dst = _sgprs(args.split(",")[0]) if args else set()
            if op.startswith("v_") and dst & reads:
                found.append((load, prev, waits))
            elif op.startswith("s_") and "m0" in dst and waits < M0_WAIT:
                found.append((load, prev, waits))
            waits += 1
    return found


def test_scanner_flags_a_readlane_before_the_load():
    bad = "v_readlane_b32 s23, v116, 7\n\ts_nop 0\n\tbuffer_load_dword v72, s[20:23], s9 offen lds\n"
    good = "v_readlane_b32 s23, v116, 7\n\ts_nop 4\n\tbuffer_load_dword v72, s[20:23], s9 offen lds\n"
    m0 = "s_mov_b32 m0, s4\n\tbuffer_load_dword v72, s[20:23], s9 offen lds\n"
    assert len(hazards(bad)) == 1 and hazards(good) == [] and len(hazards(m0)) == 1


@pytest.mark.skipif(not os.path.exists(nvbuild.HIPCC) and shutil.which("hipcc") is None, reason="hipcc not found")
def test_lds_dma_loads_have_their_wait_states():
    with tempfile.TemporaryDirectory() as tmp:
        def compile_asm(src):
            out = os.path.join(tmp, src + ".s")
            cmd = [nvbuild.HIPCC, *nvbuild.FLAGS, "--cuda-device-only", "-S", "-x", "hip",
                   os.path.join(nvbuild.CSRC, src), "-o", out]
            r = subprocess.run(cmd, capture_output=True, text=True)
            assert r.returncode == 0, r.stderr[-2000:]
            with open(out) as f:
                return src, f.read()

        with ThreadPoolExecutor(max_workers=len(SOURCES)) as pool:
            asms = list(pool.map(compile_asm, SOURCES))
    for src, asm in asms:
        assert re.search(r"buffer_load_\w+\s.*\blds$", asm, re.M), f"{src}: no LDS-DMA loads found"
        bad = hazards(asm)
        assert not bad, f"{src}: {len(bad)} loads too close to an SGPR write, e.g. {bad[:3]}"
