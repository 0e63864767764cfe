"""Static check of the library's gfx950 code for the wide-store data hazard.

A vector-memory store of more than 8 bytes reads its data registers after it
issues; a VALU instruction that writes one of those registers within two wait
states of the store can change what the store writes. The compiler counts
these wait states for global stores and for buffer stores with a constant
soffset, but not for buffer stores whose soffset is a register (the state
update's snapshot stores, which take their plane offset there, wrote wrong
lanes under load before they were guarded). This test compiles every HIP
source of the library to gfx950 assembly with the library's own flags and
checks each 12- or 16-byte store: the two wait states after it (one per
instruction, s_nop N counting N + 1) must not hold a VALU write to its data
registers. v_permlane*_swap writes both of its operands.
"""
import os
import re
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

from chunk_wise_weight_amd import build as B

STORE = re.compile(r"^\s*(buffer|global|flat)_store_dwordx[34]\s+(.*)$")


def _store_data(m):
    """The data registers of a wide store: the first operand of a buffer store, the second of a global or flat one."""
    ops = [o.strip() for o in m.group(2).split(",")]
    return _vregs(ops[0] if m.group(1) == "buffer" else ops[1])


def _vregs(text):
    regs = set()
    for lo, hi in re.findall(r"\bv\[(\d+):(\d+)\]", text):
        regs.update(range(int(lo), int(hi) + 1))
    regs.update(int(r) for r in re.findall(r"\bv(\d+)\b", text))
    return regs


def _written(ins):
    """VGPRs a VALU instruction writes (its first operand; both for the swaps)."""
    op, _, rest = ins.partition(" ")
    if not op.startswith("v_") or op.startswith(("v_cmp", "v_readlane", "v_readfirstlane")):
        return set()
    ops = [o.strip() for o in rest.split(",")]
    out = _vregs(ops[0]) if ops else set()
    if op.startswith(("v_permlane16_swap", "v_permlane32_swap", "v_swap")) and len(ops) > 1:
        out |= _vregs(ops[1])
    return out


def exposed_stores(asm_text):
    """(store, instruction) pairs where a VALU write hits a wide store's data within two wait states."""
    lines = [l.split(";")[0].strip() for l in asm_text.splitlines()]
    lines = [l for l in lines if l and not l.startswith(".") and not l.endswith(":")]
    bad = []
    for i, l in enumerate(lines):
        m = STORE.match(l)
        if not m:
            continue
        data = _store_data(m)
        waits = 0
        for n in lines[i + 1:]:
            if waits >= 2:
                break
            if n.startswith("s_nop"):
                waits += int(n.split()[1], 0) + 1
                continue
            if _written(n) & data:
                bad.append((l, n))
                break
            waits += 1
    return bad


def test_checker_flags_an_exposed_store_and_passes_a_guarded_one():
    exposed = "buffer_store_dwordx4 v[4:7], v0, s[0:3], s8 offen\nv_mov_b32_e32 v6, v9\n"
    swapped = "buffer_store_dwordx4 v[4:7], v0, s[0:3], s8 offen\nv_permlane16_swap_b32_e32 v1, v5\n"
    guarded = "buffer_store_dwordx4 v[4:7], v0, s[0:3], s8 offen\ns_nop 1\nv_mov_b32_e32 v6, v9\n"
    later = "global_store_dwordx4 v0, v[4:7], s[2:3]\nv_add_u32_e32 v1, 1, v2\ns_nop 0\nv_mov_b32_e32 v4, v9\n"
    narrow = "buffer_store_dwordx2 v[4:5], v0, s[0:3], s8 offen\nv_mov_b32_e32 v4, v9\n"
    assert len(exposed_stores(exposed)) == 1
    assert len(exposed_stores(swapped)) == 1
    assert exposed_stores(guarded) == []
    assert exposed_stores(later) == []
    assert exposed_stores(narrow) == []


def test_library_wide_stores_are_not_overwritten_within_two_wait_states():
    try:
        hipcc = B._hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    inc = ["-I", os.path.join(B.ROOT, "include"), "-I", B.CSRC]
    flags = [f for f in B.HIPCC_FLAGS if f != "-fPIC"]
    with tempfile.TemporaryDirectory() as tmp:
        def asm(src):
            out = os.path.join(tmp, src + ".s")
            r = subprocess.run([hipcc, *flags, *inc, "-S", "--cuda-device-only", os.path.join(B.CSRC, src),
                                "-o", out], capture_output=True, text=True)
            assert r.returncode == 0, r.stderr[-2000:]
            with open(out) as fh:
                return src, fh.read()

        with ThreadPoolExecutor(max_workers=4) as ex:
            texts = list(ex.map(asm, B.SOURCES))
    wide = sum(len([l for l in t.splitlines() if STORE.match(l)]) for _, t in texts)
    assert wide > 0, "expected the 16-byte stores of the up/gate and update kernels"
    bad = [(src, s, n) for src, t in texts for s, n in exposed_stores(t)]
    assert bad == [], bad[:5]
