"""Checks on the gfx950 code the pipelined kernels compile to (CPU only: hipcc
cross-compiles, nothing runs).

The pipelined SpMM issues its global loads from inline assembly and waits for
them with explicit `s_waitcnt vmcnt` statements that take the destination
registers as operands.  The data of such a load arrives asynchronously, so no
instruction may read or overwrite its destination registers between the load
and the wait -- otherwise a register copy would read stale data, or a
register reused for an address would be overwritten by the late load.  This
test compiles the kernels to assembly and walks every instantiation.
"""

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_matmul_ffns_amd", "csrc")


def _hipcc():
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return None


def _regs(text):
    out = set()
    for m in re.finditer(r"\bv\[(\d+):(\d+)\]", text):
        out |= set(range(int(m.group(1)), int(m.group(2)) + 1))
    for m in re.finditer(r"\bv(\d+)\b", text):
        out.add(int(m.group(1)))
    return out


def async_register_violations(asm_lines):
    """Instructions that touch a pending inline-asm load destination before its wait."""
    pending, bad, in_asm = set(), [], False
    for i, line in enumerate(asm_lines):
        s = line.strip()
        if s.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if s.startswith(";;#ASMEND"):
            in_asm = False
            continue
        if in_asm and s.startswith("global_load_dwordx4"):
            pending |= _regs(s.split()[1].rstrip(","))
            continue
        if in_asm and s.startswith("s_waitcnt") and "vmcnt" in s:
            pending.clear()
            continue
        if not s or s.startswith((";", ".")) or s.endswith(":"):
            continue
        operands = s.split(None, 1)[1] if " " in s else ""
        if _regs(operands) & pending:
            bad.append((i + 1, s))
    return bad


def _kernels(asm_text, prefix):
    """Device kernel bodies (label .. s_endpgm) whose symbol starts with prefix."""
    out, cur, body = {}, None, []
    for line in asm_text.splitlines():
        label = line.split(";")[0].strip()
        if label.startswith(prefix) and label.endswith(":"):
            cur, body = label[:-1], []
            continue
        if cur is not None:
            body.append(line)
            if "s_endpgm" in line:
                out[cur] = body
                cur = None
    return out


@pytest.mark.skipif(_hipcc() is None, reason="hipcc not available")
def test_pipelined_spmm_never_touches_in_flight_registers(tmp_path):
    from sparse_matmul_ffns_amd import build
    asm = tmp_path / "spmm_dma.s"
    cmd = [_hipcc(), *build.FLAGS, "-S", "-o", str(asm), os.path.join(CSRC, "spmm_dma.hip")]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    kernels = _kernels(asm.read_text(), "_ZN3nms15spmm_dma_kernel")
    assert len(kernels) >= 3
    for name, lines in kernels.items():
        assert any("global_load_dwordx4" in l for l in lines), name
        bad = async_register_violations(lines)
        assert not bad, f"{name}: {bad[:5]}"


def test_checker_catches_a_reused_register():
    # a load whose destination is overwritten before the wait must be flagged
    asm = """
    ;;#ASMSTART
    global_load_dwordx4 v[4:7], v[0:1], off
    ;;#ASMEND
    v_add_u32_e32 v5, 1, v9
    ;;#ASMSTART
    s_waitcnt vmcnt(0)
    ;;#ASMEND
    v_mov_b32_e32 v4, v10
    """.splitlines()
    bad = async_register_violations(asm)
    assert len(bad) == 1 and "v5" in bad[0][1]
