"""Store-data hazard check over the built library's gfx950 code.

A vector memory store of more than 64 bits (dwordx3 / dwordx4) reads its data
registers after it issues: the next instruction must not write them (one wait
state).  The compiler inserts that wait for global stores, and for buffer
stores only when the store's SGPR offset field holds no register, so a buffer
store with its offset in an SGPR can be followed at once by a write of its data
and store the new value in some lanes.  This test disassembles every gfx950 code
object in liblores.so and fails on any store of more than 64 bits whose data
registers the next instruction (past an exec restore) writes, and on any such
buffer store with a register in the SGPR offset field.
"""
import os
import re
import shutil
import struct
import subprocess
import tempfile

import pytest

LIB = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "quantized_linear_recurrence_amd", "liblores.so")
LLVM = "/opt/rocm/llvm/bin"
MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"

STORE = re.compile(r"\b(buffer|global|flat)_store_dwordx[34]\s+(.*)")
VREG = re.compile(r"^v(?:\[(\d+):(\d+)\]|(\d+))$")
VDEF = re.compile(r"^\s*v_\w+\s+v(?:\[(\d+):(\d+)\]|(\d+))\b")


def _vrange(op):
    m = VREG.match(op.strip())
    if not m:
        return None
    return (int(m.group(1)), int(m.group(2))) if m.group(1) is not None else (int(m.group(3)),) * 2


def _tool(name):
    path = os.path.join(LLVM, name)
    return path if os.path.exists(path) else shutil.which(name)


def _code_objects(fatbin):
    """The gfx950 device images of every offload bundle in the section."""
    out = []
    pos = fatbin.find(MAGIC)
    while pos >= 0:
        n = struct.unpack_from("<Q", fatbin, pos + len(MAGIC))[0]
        p = pos + len(MAGIC) + 8
        for _ in range(n):
            off, size, tlen = struct.unpack_from("<QQQ", fatbin, p)
            triple = fatbin[p + 24:p + 24 + tlen].decode()
            p += 24 + tlen
            if "gfx950" in triple:
                out.append(fatbin[pos + off:pos + off + size])
        pos = fatbin.find(MAGIC, pos + len(MAGIC))
    return out


def _violations(asm_lines):
    stores = bad = 0
    msgs = []
    lines = [ln.split("//")[0].rstrip() for ln in asm_lines]
    for i, ln in enumerate(lines):
        m = STORE.search(ln)
        if not m:
            continue
        stores += 1
        ops = [o.strip() for o in m.group(2).split(",")]
        # buffer: vdata, voffset, srsrc, soffset [modifiers]; global / flat: vaddr, vdata, ...
        lo, hi = _vrange(ops[0] if m.group(1) == "buffer" else ops[1])
        if m.group(1) == "buffer":
            soff = ops[3].split()[0] if len(ops) > 3 else "0"
            if soff.startswith("s") or soff.startswith("ttmp"):
                bad += 1
                msgs.append(f"register soffset: {ln.strip()}")
        # the next instruction, past an exec restore of a skipped-store branch
        j = i + 1
        while j < len(lines):
            t = lines[j].strip()
            if not t or t.endswith(">:") or t.startswith("s_or_b64 exec") or t.startswith("s_or_saveexec"):
                j += 1
                continue
            # objdump lines: "<insn operands>" possibly after an address column
            d = VDEF.match(t)
            if d:
                a = int(d.group(1) if d.group(1) is not None else d.group(3))
                b = int(d.group(2) if d.group(2) is not None else d.group(3))
                if a <= hi and b >= lo:
                    bad += 1
                    msgs.append(f"data rewritten at once: {ln.strip()} -> {t}")
            break
    return stores, bad, msgs


@pytest.mark.skipif(not os.path.exists(LIB), reason="liblores.so is not built")
def test_no_store_data_rewrite():
    objcopy, objdump = _tool("llvm-objcopy"), _tool("llvm-objdump")
    if not objcopy or not objdump:
        pytest.skip("llvm-objcopy / llvm-objdump not found")
    with tempfile.TemporaryDirectory() as td:
        fb = os.path.join(td, "fatbin")
        subprocess.run([objcopy, f"--dump-section=.hip_fatbin={fb}", LIB, os.path.join(td, "x")],
                       check=True, capture_output=True)
        with open(fb, "rb") as f:
            images = _code_objects(f.read())
        assert images, "no gfx950 code object in liblores.so"
        total = bad = 0
        msgs = []
        for k, img in enumerate(images):
            path = os.path.join(td, f"co{k}.o")
            with open(path, "wb") as f:
                f.write(img)
            asm = subprocess.run([objdump, "-d", "--no-show-raw-insn", "--no-leading-addr",
                                  "--mcpu=gfx950", path],
                                 check=True, capture_output=True, text=True).stdout
            s, b, m = _violations(asm.splitlines())
            total += s
            bad += b
            msgs += m
    assert total > 0, "no store of more than 64 bits found: the disassembly was not parsed"
    assert bad == 0, f"{bad} hazards, e.g.:\n" + "\n".join(msgs[:10])


def test_checker_flags_a_rewrite():
    """The scan itself: an immediate rewrite and a register soffset are caught,
    a store followed by a wait state is not."""
    hazard = ["buffer_store_dwordx4 v[128:131], v97, s[36:39], 0 offen nt",
              "v_perm_b32 v128, v127, v65, s66"]
    assert _violations(hazard)[1] == 1
    sgpr = ["buffer_store_dwordx4 v[8:11], v1, s[0:3], s48 offen nt", "s_nop 0",
            "v_mov_b32 v8, 0"]
    assert _violations(sgpr)[1] == 1
    ok = ["buffer_store_dwordx4 v[128:131], v97, s[36:39], 0 offen nt", "s_nop 0",
          "v_perm_b32 v128, v127, v65, s66"]
    assert _violations(ok) == (1, 0, [])
    exec_restore = ["global_store_dwordx4 v[0:1], v[4:7], off", "s_or_b64 exec, exec, s[30:31]",
                    "v_mov_b32 v5, 0"]
    assert _violations(exec_restore)[1] == 1
